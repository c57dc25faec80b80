"""Split-K (several workgroups share one tile's reduction, then a sum
kernel adds their fp32 partial sums in a fixed order): forced split counts on
small layers against the fp64 oracle, and repeatability bit for bit.

Shapes: channel counts that are not a multiple of a stage's channels (the
last split is shorter and ends in a guarded chunk), ragged output channels
and pixels, batch and frames, with and without ReLU and bias."""
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from convcheck import BIG_WS, assert_gates, metrics, oracle_args, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


# (name, dtype, N, C, T, H, W, K, KT, KH, pad, stride, act, tile or 0, bias)
CASES = [  # channel counts give 10 chunks of a stage, so every split count 2..4 runs
    ("f32_k3s1", "f32", 1, 76, 1, 13, 40, 40, 1, 3, (0, 1, 1), (1, 1, 1), "relu", 244, True),
    ("f32_k3s2", "f32", 2, 76, 1, 21, 44, 70, 1, 3, (0, 1, 1), (1, 2, 2), "none", 245, True),
    ("f16_k3s1", "f16", 2, 152, 1, 11, 40, 72, 1, 3, (0, 1, 1), (1, 1, 1), "relu", 203, True),
    ("bf16_k3s1_packed", "bf16", 1, 156, 1, 9, 48, 136, 1, 3, (0, 1, 1), (1, 1, 1), "none", 271,
     True),
    ("f16_k1", "f16", 2, 600, 1, 7, 40, 130, 1, 1, (0, 0, 0), (1, 1, 1), "relu", 221, False),
    ("f16_k333_packed", "f16", 1, 152, 4, 7, 40, 64, 3, 3, (1, 1, 1), (1, 1, 1), "relu", 262,
     True),
    # eight-wave packed tiles (128 channels x 256 pixels; K ragged over two channel tiles)
    ("bf16_k3s1_packed_8w", "bf16", 1, 156, 1, 9, 48, 136, 1, 3, (0, 1, 1), (1, 1, 1), "relu",
     277, True),
    ("f16_k333_packed_8w", "f16", 1, 152, 4, 7, 40, 136, 3, 3, (1, 1, 1), (1, 1, 1), "none", 259,
     True),
    # 16-row eight-wave tile (64 x 128 per wave, one B fragment set); 19 rows: ragged
    ("f16_k333_packed_8w_16r", "bf16", 1, 152, 4, 19, 40, 136, 3, 3, (1, 1, 1), (1, 1, 1), "none",
     257, True),
    # 12-row eight-wave tile (64 x 96 per wave); 13 rows leave a ragged second row tile
    ("f16_k333_packed_8w_12r", "f16", 1, 152, 4, 13, 40, 136, 3, 3, (1, 1, 1), (1, 1, 1), "relu",
     258, True),
    # OI(D)HW weights through one register set
    ("f16_k3s1_w1", "f16", 2, 152, 1, 11, 40, 72, 1, 3, (0, 1, 1), (1, 1, 1), "none", 207, True),
    ("bf16_k333_w1", "bf16", 1, 152, 4, 7, 40, 64, 3, 3, (1, 1, 1), (1, 1, 1), "relu", 266, True),
]


def _layer(case):
    name, dt, N, C, T, H, Wd, K, KT, KH, pad, stride, act, tile, bias = case
    dims = 3 if KT > 1 or T > 1 else 2
    return W.Layer(name, dt, N, C, T, H, Wd, K, KT, KH, KH, pad, stride, act, dims,
                   "N01", "N01", "U0.05" if bias else "zero"), tile, bias


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("ksplit", [2, 3, 4])
def test_forced_split(case, ksplit, monkeypatch):
    import direct_implicit_gemm_amd as L
    layer, tile, has_bias = _layer(case)
    monkeypatch.setenv("LIBCONV_FORCE_KSPLIT", str(ksplit))
    if tile:
        monkeypatch.setenv("LIBCONV_FORCE_TILE", str(tile))
    q1 = L.libconv_query_plan(layer.N, layer.C_in, layer.T, layer.H, layer.W, layer.C_out,
                              layer.KT, layer.KH, layer.KW, *layer.pad, *layer.stride,
                              W.DTYPE_CODE[layer.dtype], W.ACT_CODE[layer.act], L.ALGO_IGEMM,
                              0, BIG_WS)
    monkeypatch.setenv("LIBCONV_FORCE_KSPLIT", "1")
    q0 = L.libconv_query_plan(layer.N, layer.C_in, layer.T, layer.H, layer.W, layer.C_out,
                              layer.KT, layer.KH, layer.KW, *layer.pad, *layer.stride,
                              W.DTYPE_CODE[layer.dtype], W.ACT_CODE[layer.act], L.ALGO_IGEMM,
                              0, BIG_WS)
    monkeypatch.setenv("LIBCONV_FORCE_KSPLIT", str(ksplit))
    assert q1[0] == 0 and q0[0] == 0
    assert q1[2] == q0[2] and q1[3] == ksplit * q0[3], (q0, q1)  # same tile, S x workgroups
    x, w, b = W.make_inputs(layer, 40 + ksplit)
    bt = b.torch("cuda") if has_bias else None
    note(f"split {ksplit} {layer.name}: x={layer.x_shape} w={layer.w_shape} tile "
         f"{L.libconv_tile_name(q1[2])} grid {q1[3]}")
    st, pd = oracle_args(layer)
    st_, pd_ = (st, pd)
    y1 = L.conv_nd(x.torch("cuda"), w.torch("cuda"), bt, st_, pd_, layer.act, "igemm")
    y2 = L.conv_nd(x.torch("cuda"), w.torch("cuda"), bt, st_, pd_, layer.act, "igemm")
    torch.cuda.synchronize()
    assert torch.equal(y1, y2), "split-K result differs between two identical calls"
    ref, s = oracle.conv(x.f64(), w.f64(), b.f64() if has_bias else None, st, pd,
                         relu=layer.act == "relu")
    m = metrics(to_f64(y1), ref, s, layer.dtype)
    note(f"  {m}")
    assert_gates(m, layer.dtype, f"{layer.name} split {ksplit}")
