"""Test-side helpers: run a layer through libconv on the GPU and score it
against the fp64 oracle.

Gates (per layer):
  G1  max_i |y_i - r_i| / (S_i + 1e-6)  <= 1e-5 (f32), 2e-3 (f16, bf16)
      r = the unrounded fp64 oracle, S = |b| + sum of |x*w| over in-bounds taps;
      asserted as written for f32 and f16, and for bf16 on the error beyond
      the final rounding to bf16 (see metrics)
  G2  NRMSE = sqrt(sum (y - r')^2 / sum r'^2) <= 1e-3
      r' = the oracle rounded once (RNE) to the storage dtype for f16/bf16 (the
      correctly rounded result); the fp64 oracle itself for f32.
"""
from __future__ import annotations

import numpy as np

import workloads as W

G1_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
# Workspace bytes to plan with when a test asks which kernel a call will run:
# the tensor-level helpers give every call the workspace its best (or
# forced) plan asks for, so plans are queried as with unlimited room.
BIG_WS = 1 << 40
G2_TOL = 1e-3


def round_to_dtype(a64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return a64.astype(np.float32).astype(np.float64)
    return W.Tensor.quantise(a64, dtype).f64()


_SIG_BITS = {"f16": 11, "bf16": 8}
_MIN_HALF_ULP = {"f16": 2.0 ** -25, "bf16": 2.0 ** -134}


def half_ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the storage dtype at |v|'s binade."""
    _, ex = np.frexp(np.abs(v))           # |v| = m * 2^ex, m in [0.5, 1)
    h = np.ldexp(1.0, ex - 1 - _SIG_BITS[dtype])
    return np.maximum(h, _MIN_HALF_ULP[dtype])


def metrics(y: np.ndarray, ref: np.ndarray, s: np.ndarray, dtype: str) -> dict:
    """G1 as written (``g1_raw``) for f32 and f16: one f16 rounding is at most
    2^-11 of |y| <= S, below the 2e-3 bound, so a correct f16 result always
    passes it.  For bf16 one rounding can reach 2^-8 of |y| (above 2e-3 when
    |y| is close to S), so its G1 counts the error beyond the final rounding
    of y to bf16 (half an ulp at the binade of max(|y|, |r|)): a result that
    is the exact sum rounded once always passes, whatever |r| / S is."""
    y = np.asarray(y, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    s = np.asarray(s, np.float64).ravel()
    err = np.abs(y - ref)
    g1_raw = float(np.max(err / (s + 1e-6))) if y.size else 0.0
    if dtype == "bf16" and y.size:
        err = np.maximum(err - half_ulp(np.maximum(np.abs(y), np.abs(ref)), dtype), 0.0)
    g1 = float(np.max(err / (s + 1e-6))) if y.size else 0.0
    r2 = ref if dtype == "f32" else round_to_dtype(ref, dtype)
    den = float(np.sum(r2 * r2))
    nrmse = float(np.sqrt(np.sum((y - r2) ** 2) / den)) if den > 0 else float(np.sqrt(np.sum((y - r2) ** 2)))
    den_u = float(np.sum(ref * ref))
    nrmse_u = float(np.sqrt(np.sum((y - ref) ** 2) / den_u)) if den_u > 0 else 0.0
    return {"g1": g1, "g1_raw": g1_raw, "nrmse": nrmse, "nrmse_unrounded": nrmse_u,
            "n": int(y.size)}


def assert_gates(m: dict, dtype: str, what: str = "") -> None:
    assert m["g1"] <= G1_TOL[dtype], f"{what} G1 {m['g1']:.3e} > {G1_TOL[dtype]:.0e}  {m}"
    if dtype != "bf16":  # the gate exactly as stated, no rounding allowance
        assert m["g1_raw"] <= G1_TOL[dtype], f"{what} raw G1 {m['g1_raw']:.3e}  {m}"
    assert m["nrmse"] <= G2_TOL, f"{what} NRMSE {m['nrmse']:.3e} > {G2_TOL:.0e}  {m}"


def oracle_args(layer: W.Layer):
    """(stride, pad) in the oracle's per-axis form."""
    if layer.dims == 2:
        return layer.stride[1:], layer.pad[1:]
    return layer.stride, layer.pad


def gpu_forward(layer: W.Layer, x: W.Tensor, w: W.Tensor, b, algo: str = "auto",
                device: str = "cuda:0", workspace: bool = True):
    """Run through libconv; returns the output as a torch device tensor.

    workspace=True: the tensor helper with the workspace the plan asks for
    (weights packed per call, split-K where the dispatcher wants them);
    workspace=False with algo "auto": the spec exports themselves,
    conv2d_forward / conv3d_forward, which take no workspace."""
    import torch
    import direct_implicit_gemm_amd as L
    xt = x.torch(device)
    wt = w.torch(device)
    bt = None if b is None else b.torch(device)
    st, pd = (layer.stride[1:], layer.pad[1:]) if layer.dims == 2 else (layer.stride, layer.pad)
    if workspace or algo != "auto":
        return L.conv_nd(xt, wt, bt, st, pd, layer.act, algo, workspace=workspace)
    o = [L.libconv_out_size(n, k, p, s) for n, k, p, s in
         zip((layer.T, layer.H, layer.W), (layer.KT, layer.KH, layer.KW), layer.pad,
             layer.stride)]
    shape = (layer.N, layer.C_out) + (tuple(o[1:]) if layer.dims == 2 else tuple(o))
    y = torch.empty(shape, dtype=xt.dtype, device=device)
    s = torch.cuda.current_stream(device).cuda_stream
    dt, act = W.DTYPE_CODE[layer.dtype], W.ACT_CODE[layer.act]
    bp = None if bt is None else bt.data_ptr()
    if layer.dims == 2:
        st_ = L.conv2d_forward(xt.data_ptr(), wt.data_ptr(), bp, y.data_ptr(), layer.N,
                               layer.C_in, layer.H, layer.W, layer.C_out, layer.KH, layer.KW,
                               layer.pad[1], layer.pad[2], layer.stride[1], layer.stride[2], dt,
                               act, s)
    else:
        st_ = L.conv3d_forward(xt.data_ptr(), wt.data_ptr(), bp, y.data_ptr(), layer.N,
                               layer.C_in, layer.T, layer.H, layer.W, layer.C_out, layer.KT,
                               layer.KH, layer.KW, *layer.pad, *layer.stride, dt, act, s)
    if st_ != 0:
        raise L.LibconvError(st_, "conv2d_forward" if layer.dims == 2 else "conv3d_forward")
    return y


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
