"""TEST INFRASTRUCTURE ONLY: Python binding of the fp64 CPU convolution oracle.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``libconv`` and
``direct_implicit_gemm_amd``) never does.

The arithmetic lives in ``conv_oracle.c`` (plain C, fp64, OpenMP over output
elements); this module only marshals numpy arrays.  Definition followed: the
gather-form direct convolution of the page "PP-OCR on Vulkan compute shaders"
(section 2.2), with ReLU fused after the bias (section 4.4), extended by one
frame axis as in the Convolution3D layer of the page "SeedVR2 NCNN Vulkan"
(section 3.2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "conv_oracle.c")
# ORACLE_LIBRARY selects another build (the sanitizer build, liboracle_san.so)
LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
SAN_LIB_PATH = os.path.join(_HERE, "liboracle_san.so")


def build(sanitize: bool = False) -> str:
    """Compile liboracle.so with gcc (fp64, OpenMP, no fast-math).  With
    sanitize: liboracle_san.so with AddressSanitizer and
    UndefinedBehaviorSanitizer, by the clang that ships with the HIP compiler
    (so that it shares one ASan runtime with the library's sanitizer build)."""
    if sanitize:
        cmd = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-fast-math", "-ffp-contract=off",
               "-fopenmp", "-shared", "-fPIC", "-Wall", "-Werror", "-o", SAN_LIB_PATH, SRC_PATH,
               "-lm"]
        subprocess.run(cmd, check=True)
        return SAN_LIB_PATH
    out = os.path.join(_HERE, "liboracle.so")
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-shared", "-fPIC", "-Wall", "-Werror", "-o", out, SRC_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        lib.oracle_out_extent.argtypes = [ctypes.c_long] * 4
        lib.oracle_out_extent.restype = ctypes.c_long
        lib.oracle_out_extent2.argtypes = [ctypes.c_long] * 5
        lib.oracle_out_extent2.restype = ctypes.c_long
        lib.oracle_threads.argtypes = [ctypes.c_int]
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_conv.argtypes = [dp, dp, dp, dp, dp, lp, ctypes.c_int, ctypes.c_int]
        lib.oracle_conv.restype = ctypes.c_int
        lib.oracle_conv_points.argtypes = [dp, dp, dp, ctypes.POINTER(ctypes.c_int64),
                                           ctypes.c_long, dp, dp, lp, ctypes.c_int,
                                           ctypes.c_int]
        lib.oracle_conv_points.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dp(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def out_extent(n_in: int, k: int, pad: int, stride: int) -> int:
    return int(_load().oracle_out_extent(n_in, k, pad, stride))


def out_extent2(n_in: int, k: int, pad_lo: int, pad_hi: int, stride: int) -> int:
    """Output positions with pad_lo before and pad_hi after the input."""
    return int(_load().oracle_out_extent2(n_in, k, pad_lo, pad_hi, stride))


def threads(requested: int = 0) -> int:
    """OpenMP threads the oracle will use (after applying ``requested`` if > 0)."""
    return int(_load().oracle_threads(requested))


def _as5d(x: np.ndarray, w: np.ndarray):
    """View 2-D (NCHW / OIHW) operands as 3-D with one frame and one time tap."""
    if x.ndim == 4:
        return x[:, :, None], w[:, :, None], 2
    if x.ndim == 5:
        return x, w, 3
    raise ValueError("x must be NCHW or NCDHW")


def _dims(x5, w5, stride, pad, pad_t_back):
    N, C, T, H, W = x5.shape
    CO, C2, KT, KH, KW = w5.shape
    if C2 != C:
        raise ValueError("channel mismatch")
    return np.array([N, C, T, H, W, CO, KT, KH, KW, pad[0], pad[1], pad[2],
                     stride[0], stride[1], stride[2], pad_t_back], dtype=np.int64)


def _norm3(v, nd) -> Tuple[int, int, int]:
    if isinstance(v, int):
        return (v, v, v)
    v = tuple(int(t) for t in v)
    if len(v) == 2:
        return (0, v[0], v[1])
    if len(v) == 3:
        return v
    raise ValueError(v)


def _spatial(x5, w5, stride3, pad3, pad_t_back):
    _, _, T, H, W = x5.shape
    _, _, KT, KH, KW = w5.shape
    o = (out_extent2(T, KT, pad3[0], pad_t_back, stride3[0]),
         out_extent(H, KH, pad3[1], stride3[1]),
         out_extent(W, KW, pad3[2], stride3[2]))
    if min(o) < 0:
        raise ValueError("bad geometry")
    return o


def _time_pad_back(p3, nd, pad_t_back):
    """Time padding after the last frame: the pad before it unless given
    (the causal padding of "SeedVR2 NCNN Vulkan", section 7.2, is 0)."""
    if pad_t_back is None:
        return p3[0]
    if nd == 2 or int(pad_t_back) < 0:
        raise ValueError("pad_t_back needs 3-D operands and a non-negative value")
    return int(pad_t_back)


def conv(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray], stride=1, pad=0,
         relu: bool = False, nthreads: int = 0,
         pad_t_back: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 forward convolution.  Returns (y, S), both float64, shaped like y.

    x: NCHW or NCDHW; w: OIHW or OIDHW; b: [C_out] or None.
    stride / pad: an int, or one value per spatial axis ((h, w) or (t, h, w)).
    For 2-D operands the time stride is 1 and the time pad is 0.  For 3-D
    operands the time pad applies before the first frame and, unless
    pad_t_back is given, after the last one.
    """
    x5, w5, nd = _as5d(np.ascontiguousarray(x, np.float64), np.ascontiguousarray(w, np.float64))
    s3 = _norm3(stride, nd)
    p3 = _norm3(pad, nd)
    if nd == 2:
        s3, p3 = (1, s3[1], s3[2]), (0, p3[1], p3[2])
    ptb = _time_pad_back(p3, nd, pad_t_back)
    x5 = np.ascontiguousarray(x5)
    w5 = np.ascontiguousarray(w5)
    bb = None if b is None else np.ascontiguousarray(b, np.float64)
    OT, OH, OW = _spatial(x5, w5, s3, p3, ptb)
    N, CO = x5.shape[0], w5.shape[0]
    y = np.empty((N, CO, OT, OH, OW), np.float64)
    s = np.empty_like(y)
    dims = _dims(x5, w5, s3, p3, ptb)
    rc = _load().oracle_conv(_dp(x5), _dp(w5), _dp(bb), _dp(y), _dp(s),
                             dims.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                             int(bool(relu)), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_conv failed ({rc})")
    if nd == 2:
        y, s = y[:, :, 0], s[:, :, 0]
    return y, s


def conv_points(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray],
                flat_idx: Sequence[int], stride=1, pad=0, relu: bool = False,
                nthreads: int = 0, pad_t_back: Optional[int] = None
                ) -> Tuple[np.ndarray, np.ndarray]:
    """The outputs at flat indices of y (row-major over N, C_out, (OT,) OH, OW)."""
    x5, w5, nd = _as5d(np.ascontiguousarray(x, np.float64), np.ascontiguousarray(w, np.float64))
    s3 = _norm3(stride, nd)
    p3 = _norm3(pad, nd)
    if nd == 2:
        s3, p3 = (1, s3[1], s3[2]), (0, p3[1], p3[2])
    ptb = _time_pad_back(p3, nd, pad_t_back)
    x5 = np.ascontiguousarray(x5)
    w5 = np.ascontiguousarray(w5)
    bb = None if b is None else np.ascontiguousarray(b, np.float64)
    idx = np.ascontiguousarray(np.asarray(flat_idx, dtype=np.int64))
    y = np.empty(idx.shape[0], np.float64)
    s = np.empty_like(y)
    dims = _dims(x5, w5, s3, p3, ptb)
    rc = _load().oracle_conv_points(_dp(x5), _dp(w5), _dp(bb),
                                    idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                    idx.shape[0], _dp(y), _dp(s),
                                    dims.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                                    int(bool(relu)), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_conv_points failed ({rc})")
    return y, s


def fold_batchnorm(w: np.ndarray, b: Optional[np.ndarray], gamma: np.ndarray, beta: np.ndarray,
                   mean: np.ndarray, var: np.ndarray, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Batch normalisation folded into the convolution before it, in fp64 (the
    folding formula of the page "PP-OCR on Vulkan compute shaders": the weights
    scaled by gamma / sqrt(var + eps) per output channel, the bias shifted by
    the mean, scaled likewise, plus beta).  Returns (w_folded, b_folded)."""
    w = np.asarray(w, np.float64)
    co = w.shape[0]
    scale = np.asarray(gamma, np.float64) / np.sqrt(np.asarray(var, np.float64) + float(eps))
    bias = np.zeros(co) if b is None else np.asarray(b, np.float64)
    w_f = w * scale.reshape((co,) + (1,) * (w.ndim - 1))
    b_f = (bias - np.asarray(mean, np.float64)) * scale + np.asarray(beta, np.float64)
    return w_f, b_f


def max_pool2x2(y: np.ndarray) -> np.ndarray:
    """2x2 max pooling with stride 2 over the last two axes, dropping an odd
    last row or column (the pooling the PP-OCR detector fuses after its conv
    and activation, page "PP-OCR on Vulkan compute shaders", section 4.4)."""
    y = np.asarray(y)
    oh, ow = y.shape[-2] // 2, y.shape[-1] // 2
    t = y[..., :2 * oh, :2 * ow]
    return np.maximum(np.maximum(t[..., 0::2, 0::2], t[..., 0::2, 1::2]),
                      np.maximum(t[..., 1::2, 0::2], t[..., 1::2, 1::2]))


def pack_channels(x: np.ndarray, group: int) -> np.ndarray:
    """Channel-packed activations: x [N][C][...spatial] as
    [N][ceil(C/group)][...spatial][group], element [n][c // group][...][c % group]
    = x[n][c][...], and zero in the channels past C of the last group.  The
    channel packing the page "SeedVR2 NCNN Vulkan" plans to keep through the
    whole network (section 9: pack4 kept across layers; groups of 4 channels
    there, one 16-byte vector of channels here).  Written as a loop over
    channels so that the definition is read off directly."""
    x = np.asarray(x)
    n, c = x.shape[:2]
    groups = -(-c // group)
    out = np.zeros((n, groups) + x.shape[2:] + (group,), dtype=x.dtype)
    for ch in range(c):
        out[:, ch // group, ..., ch % group] = x[:, ch]
    return out


def unpack_channels(xp: np.ndarray, channels: int) -> np.ndarray:
    """The inverse of pack_channels: the first `channels` channels of a
    channel-packed tensor, back as [N][C][...spatial]."""
    xp = np.asarray(xp)
    n, group = xp.shape[0], xp.shape[-1]
    out = np.empty((n, channels) + xp.shape[2:-1], dtype=xp.dtype)
    for ch in range(channels):
        out[:, ch] = xp[:, ch // group, ..., ch % group]
    return out
