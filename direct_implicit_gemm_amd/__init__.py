"""Python binding of libconv, the gfx950 forward-convolution library.

Argument marshalling only: every convolution runs in the HIP kernels of
``libconv.so`` (built from ``csrc/`` by ``python -m direct_implicit_gemm_amd.build``).
There is no fallback: if the library is missing, importing the raw entry
points raises.  PyTorch supplies device memory and the current stream.

Raw entry points (same names and argument order as ``include/libconv.h``)
take integer device addresses and return the status code.  The tensor-level
helpers ``conv2d`` / ``conv3d`` allocate the output and raise ``LibconvError``
on a non-zero status.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence, Tuple, Union

_HERE = os.path.dirname(os.path.abspath(__file__))
# LIBCONV_LIBRARY selects another build of the same library (the sanitizer
# build, libconv_san.so); the default is the in-tree libconv.so.
LIB_PATH = os.environ.get("LIBCONV_LIBRARY") or os.path.join(_HERE, "libconv.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "libconv.h")

F32, F16, BF16 = 0, 1, 2
ACT_NONE, ACT_RELU = 0, 1
ALGO_AUTO, ALGO_DIRECT, ALGO_IGEMM = 0, 1, 2

STATUS = {
    0: "OK", 1: "ERR_NULL_POINTER", 2: "ERR_BAD_SHAPE", 3: "ERR_BAD_DTYPE",
    4: "ERR_BAD_ACTIVATION", 5: "ERR_ALIAS", 6: "ERR_UNSUPPORTED", 7: "ERR_NO_DEVICE",
    8: "ERR_LAUNCH", 9: "ERR_BAD_ALGO", 10: "ERR_TOO_LARGE", 11: "ERR_OUT_OF_MEMORY",
    12: "ERR_MISALIGNED", 13: "ERR_SCRATCH_TOO_SMALL",
}
_ALGOS = {"auto": ALGO_AUTO, "direct": ALGO_DIRECT, "igemm": ALGO_IGEMM}
_ACTS = {"none": ACT_NONE, "relu": ACT_RELU}


class LibconvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libconv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m direct_implicit_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    I, P, LL = ctypes.c_int, ctypes.c_void_p, ctypes.c_longlong
    lib.conv2d_forward.argtypes = [P, P, P, P] + [I] * 13 + [P]
    lib.conv2d_forward.restype = I
    lib.conv3d_forward.argtypes = [P, P, P, P] + [I] * 17 + [P]
    lib.conv3d_forward.restype = I
    lib.libconv_forward_algo.argtypes = [P, P, P, P] + [I] * 18 + [P]
    lib.libconv_forward_algo.restype = I
    lib.libconv_query_algo.argtypes = [I] * 18 + [ctypes.POINTER(I), ctypes.POINTER(I),
                                                  ctypes.POINTER(LL)]
    lib.libconv_query_algo.restype = I
    lib.libconv_query_plan.argtypes = [I] * 19 + [LL, ctypes.POINTER(I), ctypes.POINTER(I),
                                                  ctypes.POINTER(LL), ctypes.POINTER(I)]
    lib.libconv_query_plan.restype = I
    lib.conv2d_forward_ws.argtypes = [P, P, P, P] + [I] * 13 + [P, LL, P]
    lib.conv2d_forward_ws.restype = I
    lib.conv3d_forward_ws.argtypes = [P, P, P, P] + [I] * 17 + [P, LL, P]
    lib.conv3d_forward_ws.restype = I
    lib.libconv_forward_ex.argtypes = [P, P, P, P, P] + [I] * 20 + [P, LL, P]
    lib.libconv_forward_ex.restype = I
    lib.libconv_workspace_size.argtypes = [I] * 20
    lib.libconv_workspace_size.restype = LL
    lib.conv3d_forward_noalloc.argtypes = [P, P, P, P] + [I] * 17 + [P]
    lib.conv3d_forward_noalloc.restype = I
    lib.libconv_tile_name.argtypes = [I]
    lib.libconv_tile_name.restype = ctypes.c_char_p
    lib.libconv_tile_occupancy.argtypes = [I, I, I]
    lib.libconv_tile_occupancy.restype = I
    lib.libconv_out_size.argtypes = [I, I, I, I]
    lib.libconv_out_size.restype = I
    lib.libconv_status_string.argtypes = [I]
    lib.libconv_status_string.restype = ctypes.c_char_p
    lib.libconv_device_supported.argtypes = [I]
    lib.libconv_device_supported.restype = I
    lib.libconv_version.argtypes = []
    lib.libconv_version.restype = I
    lib.libconv_packed_weight_bytes.argtypes = [I] * 6
    lib.libconv_packed_weight_bytes.restype = LL
    lib.libconv_pack_weights.argtypes = [P, P, LL] + [I] * 6 + [P]
    lib.libconv_pack_weights.restype = I
    lib.libconv_forward_packed.argtypes = [P, P, P, P] + [I] * 17 + [P]
    lib.libconv_forward_packed.restype = I
    lib.conv2d_forward_pool.argtypes = [P, P, P, P] + [I] * 13 + [P]
    lib.conv2d_forward_pool.restype = I
    lib.conv3d_forward_tpad.argtypes = [P, P, P, P, P] + [I] * 18 + [P]
    lib.conv3d_forward_tpad.restype = I
    lib.libconv_out_size2.argtypes = [I] * 5
    lib.libconv_out_size2.restype = I
    IP = ctypes.POINTER(ctypes.c_int)
    lib.libconv_frame_window.argtypes = [I] * 7 + [IP, IP]
    lib.libconv_frame_window.restype = I
    lib.conv3d_forward_frames.argtypes = [P, P, P, P, P] + [I] * 20 + [P]
    lib.conv3d_forward_frames.restype = I
    lib.libconv_chunked_workspace_bytes.argtypes = [I] * 18
    lib.libconv_chunked_workspace_bytes.restype = LL
    lib.conv3d_forward_chunked.argtypes = [P, P, P, P, P] + [I] * 17 + [P, LL, I, I, P, P, P]
    lib.conv3d_forward_chunked.restype = I
    lib.libconv_cpack_bytes.argtypes = [I] * 6
    lib.libconv_cpack_bytes.restype = LL
    lib.libconv_pack_activations.argtypes = [P, P] + [I] * 6 + [P]
    lib.libconv_pack_activations.restype = I
    lib.libconv_unpack_activations.argtypes = [P, P] + [I] * 6 + [P]
    lib.libconv_unpack_activations.restype = I
    lib.conv3d_forward_cpack.argtypes = [P, P, P, P, P] + [I] * 18 + [P]
    lib.conv3d_forward_cpack.restype = I
    FP = ctypes.POINTER(ctypes.c_float)
    lib.libconv_fold_batchnorm.argtypes = [FP] * 6 + [ctypes.c_float, I, I, FP, FP]
    lib.libconv_fold_batchnorm.restype = I
    _lib = lib
    return lib


def header_functions() -> list:
    """Names of the functions declared in include/libconv.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:libconv_status|int|long long|const char\*)\s+(\w+)\s*\(", text,
                      flags=re.M)


# ------------------------------------------------------------ raw entry points
def conv2d_forward(x, w, bias, y, N, C_in, H, W, C_out, KH, KW, pad_h, pad_w,
                   stride_h, stride_w, dtype, act, stream) -> int:
    return load().conv2d_forward(x, w, bias, y, N, C_in, H, W, C_out, KH, KW, pad_h, pad_w,
                                 stride_h, stride_w, dtype, act, stream)


def conv3d_forward(x, w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_h, pad_w,
                   stride_t, stride_h, stride_w, dtype, act, stream) -> int:
    return load().conv3d_forward(x, w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW,
                                 pad_t, pad_h, pad_w, stride_t, stride_h, stride_w,
                                 dtype, act, stream)


def libconv_forward_algo(x, w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_h,
                         pad_w, stride_t, stride_h, stride_w, dtype, act, algo, stream) -> int:
    return load().libconv_forward_algo(x, w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW,
                                       pad_t, pad_h, pad_w, stride_t, stride_h, stride_w,
                                       dtype, act, algo, stream)


PLAN_CAPTURING, PLAN_POOL2, PLAN_CPACK, PLAN_PACKED_W = 1, 2, 4, 8


def conv2d_forward_ws(x, w, bias, y, N, C_in, H, W, C_out, KH, KW, pad_h, pad_w, stride_h,
                      stride_w, dtype, act, workspace, workspace_bytes, stream) -> int:
    return load().conv2d_forward_ws(x, w, bias, y, N, C_in, H, W, C_out, KH, KW, pad_h, pad_w,
                                    stride_h, stride_w, dtype, act, workspace, workspace_bytes,
                                    stream)


def conv3d_forward_ws(x, w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_h, pad_w,
                      stride_t, stride_h, stride_w, dtype, act, workspace, workspace_bytes,
                      stream) -> int:
    return load().conv3d_forward_ws(x, w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t,
                                    pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act,
                                    workspace, workspace_bytes, stream)


def libconv_forward_ex(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW,
                       pad_t_front, pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w,
                       dtype, act, algo, flags, workspace, workspace_bytes, stream) -> int:
    return load().libconv_forward_ex(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH,
                                     KW, pad_t_front, pad_t_back, pad_h, pad_w, stride_t,
                                     stride_h, stride_w, dtype, act, algo, flags, workspace,
                                     workspace_bytes, stream)


SCRATCH_BYTES = 64 << 20


def conv3d_forward_noalloc(x, w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_h,
                           pad_w, stride_t, stride_h, stride_w, dtype, act, stream) -> int:
    return load().conv3d_forward_noalloc(x, w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW,
                                         pad_t, pad_h, pad_w, stride_t, stride_h, stride_w,
                                         dtype, act, stream)


def libconv_workspace_size(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t_front, pad_t_back,
                           pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, algo,
                           flags) -> int:
    return load().libconv_workspace_size(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t_front,
                                         pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w,
                                         dtype, act, algo, flags)


def conv2d_forward_pool(x, w, bias, y, N, C_in, H, W, C_out, KH, KW, pad_h, pad_w, stride_h,
                        stride_w, dtype, act, stream) -> int:
    return load().conv2d_forward_pool(x, w, bias, y, N, C_in, H, W, C_out, KH, KW, pad_h, pad_w,
                                      stride_h, stride_w, dtype, act, stream)


def conv3d_forward_tpad(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW,
                        pad_t_front, pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w,
                        dtype, act, stream) -> int:
    return load().conv3d_forward_tpad(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH,
                                      KW, pad_t_front, pad_t_back, pad_h, pad_w, stride_t,
                                      stride_h, stride_w, dtype, act, stream)


def libconv_out_size2(n_in, k, pad_lo, pad_hi, stride) -> int:
    return load().libconv_out_size2(n_in, k, pad_lo, pad_hi, stride)


def libconv_cpack_bytes(N, C, T, H, W, dtype) -> int:
    return load().libconv_cpack_bytes(N, C, T, H, W, dtype)


def libconv_pack_activations(x, x_packed, N, C, T, H, W, dtype, stream) -> int:
    return load().libconv_pack_activations(x, x_packed, N, C, T, H, W, dtype, stream)


def libconv_unpack_activations(x_packed, x, N, C, T, H, W, dtype, stream) -> int:
    return load().libconv_unpack_activations(x_packed, x, N, C, T, H, W, dtype, stream)


def conv3d_forward_cpack(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW,
                         pad_t_front, pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w,
                         dtype, act, stream) -> int:
    return load().conv3d_forward_cpack(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH,
                                       KW, pad_t_front, pad_t_back, pad_h, pad_w, stride_t,
                                       stride_h, stride_w, dtype, act, stream)


def libconv_frame_window(T, KT, pad_t_front, pad_t_back, stride_t, out_frame0,
                         out_frames) -> Tuple[int, int, int]:
    """Returns (status, in_frame0, in_frames)."""
    f0, tw = ctypes.c_int(-1), ctypes.c_int(-1)
    st = load().libconv_frame_window(T, KT, pad_t_front, pad_t_back, stride_t, out_frame0,
                                     out_frames, ctypes.byref(f0), ctypes.byref(tw))
    return st, f0.value, tw.value


def conv3d_forward_frames(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW,
                          pad_t_front, pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w,
                          out_frame0, out_frames, dtype, act, stream) -> int:
    return load().conv3d_forward_frames(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT,
                                        KH, KW, pad_t_front, pad_t_back, pad_h, pad_w, stride_t,
                                        stride_h, stride_w, out_frame0, out_frames, dtype, act,
                                        stream)


def libconv_chunked_workspace_bytes(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t_front,
                                    pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w,
                                    chunk_frames, dtype) -> int:
    return load().libconv_chunked_workspace_bytes(N, C_in, T, H, W, C_out, KT, KH, KW,
                                                  pad_t_front, pad_t_back, pad_h, pad_w,
                                                  stride_t, stride_h, stride_w, chunk_frames,
                                                  dtype)


def conv3d_forward_chunked(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW,
                           pad_t_front, pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w,
                           chunk_frames, workspace, workspace_bytes, dtype, act, stream,
                           copy_in_stream, copy_out_stream) -> int:
    return load().conv3d_forward_chunked(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT,
                                         KH, KW, pad_t_front, pad_t_back, pad_h, pad_w,
                                         stride_t, stride_h, stride_w, chunk_frames, workspace,
                                         workspace_bytes, dtype, act, stream, copy_in_stream,
                                         copy_out_stream)


def fold_batchnorm(w, b, gamma, beta, mean, var, eps: float):
    """libconv_fold_batchnorm on host numpy arrays: returns (w_folded, b_folded)
    as float32 arrays shaped like w and [C_out].  b may be None."""
    import numpy as np
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    w32 = f32(w)
    C_out = w32.shape[0]
    k = int(w32.size // C_out)
    gamma, beta, mean, var = (f32(a).reshape(C_out) for a in (gamma, beta, mean, var))
    b32 = None if b is None else f32(b).reshape(C_out)
    wo = np.empty_like(w32)
    bo = np.empty(C_out, np.float32)
    fp = lambda a: None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    st = load().libconv_fold_batchnorm(fp(w32), fp(b32), fp(gamma), fp(beta), fp(mean), fp(var),
                                       float(eps), C_out, k, fp(wo), fp(bo))
    if st != 0:
        raise LibconvError(st, "libconv_fold_batchnorm")
    return wo, bo


def libconv_packed_weight_bytes(C_in, C_out, KT, KH, KW, dtype) -> int:
    return load().libconv_packed_weight_bytes(C_in, C_out, KT, KH, KW, dtype)


def libconv_pack_weights(w, packed, packed_bytes, C_in, C_out, KT, KH, KW, dtype, stream) -> int:
    return load().libconv_pack_weights(w, packed, packed_bytes, C_in, C_out, KT, KH, KW, dtype,
                                       stream)


def libconv_forward_packed(x, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t,
                           pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, stream) -> int:
    return load().libconv_forward_packed(x, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH,
                                         KW, pad_t, pad_h, pad_w, stride_t, stride_h, stride_w,
                                         dtype, act, stream)


def libconv_query_algo(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_h, pad_w,
                       stride_t, stride_h, stride_w, dtype, act, algo) -> Tuple[int, int, int, int]:
    """Returns (status, algo, tile_id, grid)."""
    a, t, g = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_longlong(-1)
    st = load().libconv_query_algo(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_h, pad_w,
                                   stride_t, stride_h, stride_w, dtype, act, algo,
                                   ctypes.byref(a), ctypes.byref(t), ctypes.byref(g))
    return st, a.value, t.value, g.value


def libconv_query_plan(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_h, pad_w,
                       stride_t, stride_h, stride_w, dtype, act, algo,
                       flags, workspace_bytes=0) -> Tuple[int, int, int, int, int]:
    """Returns (status, algo, tile_id, grid, ksplit)."""
    a, t, g, k = ctypes.c_int(-1), ctypes.c_int(-1), ctypes.c_longlong(-1), ctypes.c_int(-1)
    st = load().libconv_query_plan(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_h, pad_w,
                                   stride_t, stride_h, stride_w, dtype, act, algo, flags,
                                   int(workspace_bytes), ctypes.byref(a), ctypes.byref(t),
                                   ctypes.byref(g), ctypes.byref(k))
    return st, a.value, t.value, g.value, k.value


def libconv_tile_name(tile_id: int) -> str:
    return load().libconv_tile_name(tile_id).decode()


def libconv_tile_occupancy(tile_id: int, dtype: int, measured: bool = False) -> int:
    return load().libconv_tile_occupancy(tile_id, dtype, int(measured))


def libconv_out_size(n_in: int, k: int, pad: int, stride: int) -> int:
    return load().libconv_out_size(n_in, k, pad, stride)


def libconv_status_string(status: int) -> str:
    return load().libconv_status_string(status).decode()


status_string = libconv_status_string


def libconv_device_supported(device: int) -> int:
    return load().libconv_device_supported(device)


def libconv_version() -> int:
    return load().libconv_version()


# ------------------------------------------------------- tensor-level helpers
def _triple(v, nd: int) -> Tuple[int, ...]:
    if isinstance(v, int):
        return (v,) * nd
    v = tuple(int(t) for t in v)
    if len(v) != nd:
        raise ValueError(f"expected {nd} values, got {v}")
    return v


def _dtype_code(t) -> int:
    import torch
    m = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _run_ex(what, x_ptr, w, b, y_ptr, dims, pads, strides, dt, act, algo, flags, device,
            stream, workspace):
    """libconv_forward_ex with a workspace sized by libconv_workspace_size.

    w is a device tensor (OI(D)HW) or PackedWeights; dims (N, C, T, H, W, K,
    KT, KH, KW), pads (front, back, h, w), strides (t, h, w).  workspace: True
    (allocate what the best plan takes, through torch), False/None (none: the
    plan packs nothing and splits nothing), or a uint8 device tensor to use.
    """
    import torch
    lib = load()
    packed = isinstance(w, PackedWeights)
    ws_ptr, ws_n = None, 0
    if workspace is not None and workspace is not False:
        need = lib.libconv_workspace_size(*dims, *pads, *strides, dt, _ACTS[act], _ALGOS[algo],
                                          flags | (PLAN_PACKED_W if packed else 0))
        if workspace is True:
            if need > 0:
                buf = torch.empty(need, dtype=torch.uint8, device=device)
                ws_ptr, ws_n = buf.data_ptr(), need
        else:
            ws_ptr, ws_n = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(device).cuda_stream
    st_ = lib.libconv_forward_ex(x_ptr, None if packed else _ptr(w),
                                 w.data.data_ptr() if packed else None, _ptr(b), y_ptr, *dims,
                                 *pads, *strides, dt, _ACTS[act], _ALGOS[algo], flags, ws_ptr,
                                 ws_n, stream)
    if st_ != 0:
        raise LibconvError(st_, what)


def conv_nd(x, w, b=None, stride: Union[int, Sequence[int]] = 1,
            padding: Union[int, Sequence[int]] = 0, act: str = "none", algo: str = "auto",
            out=None, stream=None, workspace=True):
    """Convolution of CUDA (HIP) tensors through libconv; 2-D or 3-D by x.ndim.
    workspace: True (allocate what the best plan takes), False (none, as
    conv2d_forward / conv3d_forward), or a uint8 device tensor."""
    import torch
    nd = x.dim() - 2
    if nd not in (2, 3) or w.dim() != x.dim():
        raise ValueError("x must be NCHW or NCDHW and w OIHW or OIDHW")
    for t in (x, w) + ((b,) if b is not None else ()):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype:
            raise ValueError("x, w, b must be contiguous device tensors of one dtype")
    s = _triple(stride, nd)
    p = _triple(padding, nd)
    dt = _dtype_code(x)
    if nd == 2:
        N, C, H, W = x.shape
        T, KT, st, pt = 1, 1, 1, 0
        K, _, KH, KW = w.shape
        sh, sw = s
        ph, pw = p
    else:
        N, C, T, H, W = x.shape
        K, _, KT, KH, KW = w.shape
        st, sh, sw = s
        pt, ph, pw = p
    if w.shape[1] != C:
        raise ValueError("channel mismatch")
    lib = load()
    ot = lib.libconv_out_size(T, KT, pt, st)
    oh = lib.libconv_out_size(H, KH, ph, sh)
    ow = lib.libconv_out_size(W, KW, pw, sw)
    if min(ot, oh, ow) < 1:
        raise LibconvError(2, "conv")
    shape = (N, K, oh, ow) if nd == 2 else (N, K, ot, oh, ow)
    y = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    if tuple(y.shape) != shape or not y.is_contiguous() or y.dtype != x.dtype:
        raise ValueError("bad output tensor")
    _run_ex("libconv_forward_ex", _ptr(x), w, b, _ptr(y), (N, C, T, H, W, K, KT, KH, KW),
            (pt, pt, ph, pw), (st, sh, sw), dt, act, algo, 0, x.device, stream, workspace)
    return y


class PackedWeights:
    """Weights in the packed layout, with the shape they were packed from."""

    def __init__(self, data, w_shape, dtype):
        self.data = data          # uint8 device tensor
        self.w_shape = tuple(w_shape)
        self.dtype = dtype


def pack_weights(w, stream=None) -> PackedWeights:
    """Pack OIHW / OIDHW weights (device tensor) for libconv_forward_packed."""
    import torch
    if not w.is_cuda or not w.is_contiguous():
        raise ValueError("w must be a contiguous device tensor")
    K, C = w.shape[:2]
    ks = tuple(w.shape[2:])
    KT, KH, KW = (1,) + ks if len(ks) == 2 else ks
    dt = _dtype_code(w)
    nbytes = load().libconv_packed_weight_bytes(C, K, KT, KH, KW, dt)
    if nbytes < 0:
        raise LibconvError(6, "libconv_packed_weight_bytes")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    if stream is None:
        stream = torch.cuda.current_stream(w.device).cuda_stream
    st = load().libconv_pack_weights(w.data_ptr(), buf.data_ptr(), nbytes, C, K, KT, KH, KW, dt,
                                     stream)
    if st != 0:
        raise LibconvError(st, "libconv_pack_weights")
    return PackedWeights(buf, w.shape, w.dtype)


def conv_nd_packed(x, pw: PackedWeights, b=None, stride=1, padding=0, act="none", out=None,
                   stream=None, workspace=None):
    """Convolution with weights packed by pack_weights (libconv_forward_packed;
    with a workspace (True or a tensor), libconv_forward_ex, which may split
    the reduction)."""
    import torch
    nd = x.dim() - 2
    if pw.dtype != x.dtype or len(pw.w_shape) != x.dim():
        raise ValueError("packed weights do not match x")
    s = _triple(stride, nd)
    p = _triple(padding, nd)
    if nd == 2:
        N, C, H, W = x.shape
        T, KT, st, pt = 1, 1, 1, 0
        K, _, KH, KW = pw.w_shape
        sh, sw = s
        ph, pw_ = p
    else:
        N, C, T, H, W = x.shape
        K, _, KT, KH, KW = pw.w_shape
        st, sh, sw = s
        pt, ph, pw_ = p
    lib = load()
    ot = lib.libconv_out_size(T, KT, pt, st)
    oh = lib.libconv_out_size(H, KH, ph, sh)
    ow = lib.libconv_out_size(W, KW, pw_, sw)
    if min(ot, oh, ow) < 1:
        raise LibconvError(2, "conv")
    shape = (N, K, oh, ow) if nd == 2 else (N, K, ot, oh, ow)
    y = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    if workspace is None or workspace is False:
        st_ = lib.libconv_forward_packed(x.data_ptr(), pw.data.data_ptr(), _ptr(b), y.data_ptr(),
                                         N, C, T, H, W, K, KT, KH, KW, pt, ph, pw_, st, sh, sw,
                                         _dtype_code(x), _ACTS[act], stream)
        if st_ != 0:
            raise LibconvError(st_, "libconv_forward_packed")
    else:
        _run_ex("libconv_forward_ex", x.data_ptr(), pw, b, y.data_ptr(),
                (N, C, T, H, W, K, KT, KH, KW), (pt, pt, ph, pw_), (st, sh, sw), _dtype_code(x),
                act, "igemm", 0, x.device, stream, workspace)
    return y


def conv2d_pool(x, w, b=None, stride=1, padding=0, act="none", out=None, stream=None,
                workspace=True):
    """2-D convolution, activation and 2x2 stride-2 max pooling in one call
    (conv2d_forward_pool); returns y [N][C_out][OH/2][OW/2]."""
    import torch
    if x.dim() != 4 or w.dim() != 4 or w.shape[1] != x.shape[1]:
        raise ValueError("x must be NCHW and w OIHW with x's channel count")
    for t in (x, w) + ((b,) if b is not None else ()):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype:
            raise ValueError("x, w, b must be contiguous device tensors of one dtype")
    sh, sw = _triple(stride, 2)
    ph, pw_ = _triple(padding, 2)
    N, C, H, W = x.shape
    K, _, KH, KW = w.shape
    lib = load()
    oh = lib.libconv_out_size(H, KH, ph, sh)
    ow = lib.libconv_out_size(W, KW, pw_, sw)
    if min(oh, ow) < 2:
        raise LibconvError(2, "conv2d_pool")
    shape = (N, K, oh // 2, ow // 2)
    y = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    if tuple(y.shape) != shape or not y.is_contiguous() or y.dtype != x.dtype:
        raise ValueError("bad output tensor")
    _run_ex("conv2d_forward_pool", _ptr(x), w, b, _ptr(y), (N, C, 1, H, W, K, 1, KH, KW),
            (0, 0, ph, pw_), (1, sh, sw), _dtype_code(x), act, "auto", PLAN_POOL2, x.device,
            stream, workspace)
    return y


def conv3d_tpad(x, w, b=None, pad_t=(0, 0), stride=1, padding_hw=0, act="none", out=None,
                stream=None, workspace=True):
    """3-D convolution with pad_t = (frames before, frames after); (KT-1, 0) is
    the causal convolution.  w: OIDHW device tensor or PackedWeights."""
    import torch
    if x.dim() != 5:
        raise ValueError("x must be NCDHW")
    packed = isinstance(w, PackedWeights)
    w_shape = w.w_shape if packed else tuple(w.shape)
    if len(w_shape) != 5 or w_shape[1] != x.shape[1]:
        raise ValueError("w must be OIDHW with x's channel count")
    for t in (x,) + (() if packed else (w,)) + ((b,) if b is not None else ()):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype:
            raise ValueError("x, w, b must be contiguous device tensors of one dtype")
    if packed and w.dtype != x.dtype:
        raise ValueError("packed weights do not match x")
    st, sh, sw = _triple(stride, 3)
    ph, pw_ = _triple(padding_hw, 2)
    pf, pb = (int(pad_t[0]), int(pad_t[1]))
    N, C, T, H, W = x.shape
    K, _, KT, KH, KW = w_shape
    lib = load()
    ot = lib.libconv_out_size2(T, KT, pf, pb, st)
    oh = lib.libconv_out_size(H, KH, ph, sh)
    ow = lib.libconv_out_size(W, KW, pw_, sw)
    if min(ot, oh, ow) < 1:
        raise LibconvError(2, "conv3d_tpad")
    shape = (N, K, ot, oh, ow)
    y = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    if tuple(y.shape) != shape or not y.is_contiguous() or y.dtype != x.dtype:
        raise ValueError("bad output tensor")
    _run_ex("conv3d_forward_tpad", _ptr(x), w, b, _ptr(y), (N, C, T, H, W, K, KT, KH, KW),
            (pf, pb, ph, pw_), (st, sh, sw), _dtype_code(x), act, "auto", 0, x.device, stream,
            workspace)
    return y


def _video_args(x, w, b, stride, padding_hw, pad_t, what, x_on_host_ok):
    if x.dim() != 5:
        raise ValueError("x must be NCDHW")
    packed = isinstance(w, PackedWeights)
    w_shape = w.w_shape if packed else tuple(w.shape)
    if len(w_shape) != 5 or w_shape[1] != x.shape[1]:
        raise ValueError("w must be OIDHW with x's channel count")
    if not x.is_contiguous() or (not x.is_cuda and not x_on_host_ok):
        raise ValueError(f"{what}: x must be a contiguous device tensor")
    for t in (() if packed else (w,)) + ((b,) if b is not None else ()):
        if not t.is_cuda or not t.is_contiguous() or t.dtype != x.dtype:
            raise ValueError(f"{what}: w, b must be contiguous device tensors of x's dtype")
    if packed and w.dtype != x.dtype:
        raise ValueError("packed weights do not match x")
    st, sh, sw = _triple(stride, 3)
    ph, pw_ = _triple(padding_hw, 2)
    return packed, w_shape, (st, sh, sw), (ph, pw_), (int(pad_t[0]), int(pad_t[1]))


def conv3d_frames(x, w, b=None, T=None, out_frames=(0, 1), pad_t=(0, 0), stride=1,
                  padding_hw=0, act="none", out=None, stream=None):
    """Output frames [o0, o0 + n) (out_frames = (o0, n)) of the convolution
    over a T-frame video, from x holding only the input frames
    libconv_frame_window names for them (x [N, C, in_frames, H, W])."""
    import torch
    packed, w_shape, (st, sh, sw), (ph, pw_), (pf, pb) = _video_args(
        x, w, b, stride, padding_hw, pad_t, "conv3d_frames", False)
    N, C, TX, H, W = x.shape
    K, _, KT, KH, KW = w_shape
    o0, on = int(out_frames[0]), int(out_frames[1])
    if T is None:
        raise ValueError("conv3d_frames: T (the whole video's frame count) is required")
    # x must hold exactly the window the library will read for these frames:
    # the C side takes its frame count from that window, not from x
    wst, f0, nfr = libconv_frame_window(int(T), KT, pf, pb, st, o0, on)
    if wst != 0:
        raise LibconvError(wst, "libconv_frame_window")
    if TX != nfr:
        raise ValueError(f"conv3d_frames: x holds {TX} frames, but output frames "
                         f"[{o0}, {o0 + on}) read the {nfr} input frames from {f0}")
    lib = load()
    oh = lib.libconv_out_size(H, KH, ph, sh)
    ow = lib.libconv_out_size(W, KW, pw_, sw)
    if min(oh, ow) < 1 or on < 1:
        raise LibconvError(2, "conv3d_frames")
    shape = (N, K, on, oh, ow)
    y = torch.empty(shape, dtype=x.dtype, device=x.device) if out is None else out
    if tuple(y.shape) != shape or not y.is_contiguous() or y.dtype != x.dtype or not y.is_cuda:
        raise ValueError("bad output tensor")
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st_ = lib.conv3d_forward_frames(_ptr(x), None if packed else _ptr(w),
                                    w.data.data_ptr() if packed else None, _ptr(b), _ptr(y),
                                    N, C, int(T), H, W, K, KT, KH, KW, pf, pb, ph, pw_, st, sh, sw,
                                    o0, on, _dtype_code(x), _ACTS[act], stream)
    if st_ != 0:
        raise LibconvError(st_, "conv3d_forward_frames")
    return y


class PackedActivations:
    """A channel-packed activation tensor on the device: ``data`` holds
    [N][ceil(C/g)][T][H][W][g] (g = 16 bytes of channels) as raw bytes;
    ``shape`` is the plain (N, C, [T,] H, W) shape it stands for."""

    def __init__(self, data, shape, dtype):
        self.data = data
        self.shape = tuple(shape)
        self.dtype = dtype

    @property
    def group(self) -> int:
        import torch
        return 4 if self.dtype == torch.float32 else 8

    def _dims(self):
        if len(self.shape) == 4:
            n, c, h, w = self.shape
            return n, c, 1, h, w
        return self.shape


def pack_activations(x, stream=None) -> PackedActivations:
    """Plain NC(T)HW device tensor -> channel-packed copy."""
    import torch
    if x.dim() not in (4, 5) or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous NCHW or NCDHW device tensor")
    dims = (x.shape[0], x.shape[1], 1, x.shape[2], x.shape[3]) if x.dim() == 4 else tuple(x.shape)
    dt = _dtype_code(x)
    lib = load()
    nb = lib.libconv_cpack_bytes(*dims, dt)
    if nb < 0:
        raise LibconvError(2, "pack_activations")
    data = torch.empty(max(nb, 1), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    st = lib.libconv_pack_activations(_ptr(x), data.data_ptr(), *dims, dt, stream)
    if st != 0:
        raise LibconvError(st, "libconv_pack_activations")
    return PackedActivations(data, x.shape, x.dtype)


def unpack_activations(xp: PackedActivations, out=None, stream=None):
    """Channel-packed -> plain NC(T)HW device tensor."""
    import torch
    y = torch.empty(xp.shape, dtype=xp.dtype, device=xp.data.device) if out is None else out
    if tuple(y.shape) != xp.shape or y.dtype != xp.dtype or not y.is_contiguous():
        raise ValueError("bad output tensor")
    if stream is None:
        stream = torch.cuda.current_stream(y.device).cuda_stream
    st = load().libconv_unpack_activations(xp.data.data_ptr(), _ptr(y), *xp._dims(),
                                           _dtype_code(y), stream)
    if st != 0:
        raise LibconvError(st, "libconv_unpack_activations")
    return y


def conv_cpack(xp: PackedActivations, w, b=None, stride=1, padding=0, pad_t=None, act="none",
               out=None, stream=None, workspace=True) -> PackedActivations:
    """Convolution on channel-packed activations; returns the packed output.
    w: OI(D)HW device tensor or PackedWeights.  2-D when xp stands for NCHW.
    padding: (h, w) or (t, h, w); pad_t = (front, back) overrides the time
    padding."""
    import torch
    packed = isinstance(w, PackedWeights)
    w_shape = w.w_shape if packed else tuple(w.shape)
    N, C, T, H, W = xp._dims()
    nd = len(xp.shape) - 2
    if len(w_shape) != nd + 2 or w_shape[1] != C:
        raise ValueError("w does not match the activations")
    if not packed and (not w.is_cuda or not w.is_contiguous() or w.dtype != xp.dtype):
        raise ValueError("w must be a contiguous device tensor of the activations' dtype")
    if b is not None and (not b.is_cuda or not b.is_contiguous() or b.dtype != xp.dtype):
        raise ValueError("b must be a contiguous device tensor of the activations' dtype")
    K = w_shape[0]
    if nd == 2:
        KT, (KH, KW) = 1, w_shape[2:]
        st, (sh, sw) = 1, _triple(stride, 2)
        pf = pb = 0
        ph, pw_ = _triple(padding, 2)
    else:
        KT, KH, KW = w_shape[2:]
        st, sh, sw = _triple(stride, 3)
        pt_, ph, pw_ = _triple(padding, 3)
        pf, pb = (pt_, pt_) if pad_t is None else (int(pad_t[0]), int(pad_t[1]))
    lib = load()
    ot = lib.libconv_out_size2(T, KT, pf, pb, st)
    oh = lib.libconv_out_size(H, KH, ph, sh)
    ow = lib.libconv_out_size(W, KW, pw_, sw)
    if min(ot, oh, ow) < 1:
        raise LibconvError(2, "conv_cpack")
    dt = _dtype_code(torch.empty(0, dtype=xp.dtype))
    nb = lib.libconv_cpack_bytes(N, K, ot, oh, ow, dt)
    if nb < 0:
        raise LibconvError(10, "conv_cpack")
    shape = (N, K, oh, ow) if nd == 2 else (N, K, ot, oh, ow)
    if out is None:
        out = PackedActivations(torch.empty(max(nb, 1), dtype=torch.uint8, device=xp.data.device),
                                shape, xp.dtype)
    elif out.shape != shape or out.dtype != xp.dtype or out.data.numel() < nb:
        raise ValueError("bad output tensor")
    _run_ex("conv3d_forward_cpack", xp.data.data_ptr(), w, b, out.data.data_ptr(),
            (N, C, T, H, W, K, KT, KH, KW), (pf, pb, ph, pw_), (st, sh, sw), dt, act, "auto",
            PLAN_CPACK, xp.data.device, stream, workspace)
    return out


_copy_streams = {}


def conv3d_chunked(x, w, b=None, chunk_frames=17, pad_t=(0, 0), stride=1, padding_hw=0,
                   act="none", out=None, stream=None, copy_streams=None):
    """The whole-video convolution streamed through the device in chunks of
    chunk_frames output frames.  x (and the output) may live in host memory
    (pinned for asynchronous copies) or on the device; weights and bias are
    device tensors.  copy_streams: (in, out) stream handles for the copies
    (default: two streams of this module's own; (s, s) with s the compute
    stream runs everything in order).  A host output is complete when this
    returns; a device output is ordered on `stream` as usual."""
    import torch
    packed, w_shape, (st, sh, sw), (ph, pw_), (pf, pb) = _video_args(
        x, w, b, stride, padding_hw, pad_t, "conv3d_chunked", True)
    dev = (w.data if packed else w).device
    N, C, T, H, W = x.shape
    K, _, KT, KH, KW = w_shape
    lib = load()
    ot = lib.libconv_out_size2(T, KT, pf, pb, st)
    oh = lib.libconv_out_size(H, KH, ph, sh)
    ow = lib.libconv_out_size(W, KW, pw_, sw)
    if min(ot, oh, ow) < 1:
        raise LibconvError(2, "conv3d_chunked")
    shape = (N, K, ot, oh, ow)
    if out is None:
        out = (torch.empty(shape, dtype=x.dtype, device=dev) if x.is_cuda else
               torch.empty(shape, dtype=x.dtype, pin_memory=True))
    if tuple(out.shape) != shape or not out.is_contiguous() or out.dtype != x.dtype:
        raise ValueError("bad output tensor")
    dt = _dtype_code(x)
    ws_bytes = lib.libconv_chunked_workspace_bytes(N, C, T, H, W, K, KT, KH, KW, pf, pb, ph, pw_,
                                                   st, sh, sw, int(chunk_frames), dt)
    if ws_bytes < 0:
        raise LibconvError(2, "conv3d_chunked")
    cur = torch.cuda.current_stream(dev)
    if stream is None:
        stream = cur.cuda_stream
    if copy_streams is None:
        pair = _copy_streams.get(dev.index)
        if pair is None:
            pair = _copy_streams[dev.index] = (torch.cuda.Stream(dev), torch.cuda.Stream(dev))
        copy_streams = (pair[0].cuda_stream, pair[1].cuda_stream)
    # allocated on torch's current stream: later work there is ordered after
    # `stream` has waited for the last copy, when `stream` is that stream
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    st_ = lib.conv3d_forward_chunked(_ptr(x), None if packed else _ptr(w),
                                     w.data.data_ptr() if packed else None, _ptr(b), _ptr(out),
                                     N, C, T, H, W, K, KT, KH, KW, pf, pb, ph, pw_, st, sh, sw,
                                     int(chunk_frames), ws.data_ptr(), ws_bytes, dt, _ACTS[act],
                                     stream, copy_streams[0], copy_streams[1])
    if st_ != 0:
        raise LibconvError(st_, "conv3d_forward_chunked")
    if not out.is_cuda or stream != cur.cuda_stream:
        # host memory is read by the caller next; a foreign stream does not
        # order the workspace's release
        torch.cuda.synchronize(dev)
    return out


def conv2d(x, w, b=None, stride=1, padding=0, act="none", algo="auto", out=None, stream=None,
           workspace=True):
    if x.dim() != 4:
        raise ValueError("conv2d takes NCHW")
    return conv_nd(x, w, b, stride, padding, act, algo, out, stream, workspace)


def conv3d(x, w, b=None, stride=1, padding=0, act="none", algo="auto", out=None, stream=None,
           workspace=True):
    if x.dim() != 5:
        raise ValueError("conv3d takes NCDHW")
    return conv_nd(x, w, b, stride, padding, act, algo, out, stream, workspace)
