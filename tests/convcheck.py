"""Test-side helpers: run a layer through libconv on the GPU and score it
against the fp64 oracle.

Gates (per layer):
  G1  max_i |y_i - r_i| / (S_i + 1e-6)  <= 1e-5 (f32), 2e-3 (f16, bf16)
      r = the unrounded fp64 oracle, S = |b| + sum of |x*w| over in-bounds taps
  G2  NRMSE = sqrt(sum (y - r')^2 / sum r'^2) <= 1e-3
      r' = the oracle rounded once (RNE) to the storage dtype for f16/bf16 (the
      correctly rounded result); the fp64 oracle itself for f32.
"""
from __future__ import annotations

import numpy as np

import workloads as W

G1_TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
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
    """G1 for f16/bf16 counts the error beyond the final rounding of y to its
    storage dtype (half an ulp at the binade of max(|y|, |r|)): a result that
    is the exact sum rounded once always passes, whatever |r| / S is."""
    y = np.asarray(y, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    s = np.asarray(s, np.float64).ravel()
    err = np.abs(y - ref)
    g1_raw = float(np.max(err / (s + 1e-6))) if y.size else 0.0
    if dtype != "f32" and y.size:
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
    assert m["nrmse"] <= G2_TOL, f"{what} NRMSE {m['nrmse']:.3e} > {G2_TOL:.0e}  {m}"


def oracle_args(layer: W.Layer):
    """(stride, pad) in the oracle's per-axis form."""
    if layer.dims == 2:
        return layer.stride[1:], layer.pad[1:]
    return layer.stride, layer.pad


def gpu_forward(layer: W.Layer, x: W.Tensor, w: W.Tensor, b, algo: str = "auto",
                device: str = "cuda:0"):
    """Run through libconv; returns the output as a torch device tensor."""
    import direct_implicit_gemm_amd as L
    xt = x.torch(device)
    wt = w.torch(device)
    bt = None if b is None else b.torch(device)
    st, pd = (layer.stride[1:], layer.pad[1:]) if layer.dims == 2 else (layer.stride, layer.pad)
    return L.conv_nd(xt, wt, bt, st, pd, layer.act, algo)


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
