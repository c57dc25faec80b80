"""Packed weights on the GPU: the packed layout itself, and convolutions that
read packed weights (explicitly packed, or packed inside conv3d_forward)."""
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


def _expected_packed(w: np.ndarray, se: int, kp_align: int = 128) -> np.ndarray:
    """The layout definition: [round_up(K,128)/64][ceil(C/se)][taps][64][se],
    zero-filled."""
    K, C = w.shape[:2]
    ts = int(np.prod(w.shape[2:]))
    g = -(-C // se)
    kp = -(-K // kp_align) * kp_align
    wf = np.zeros((kp, g * se, ts), dtype=w.dtype)
    wf[:K, :C] = w.reshape(K, C, ts)
    # [co // 64][g][t][co % 64][j]
    return wf.reshape(kp // 64, 64, g, se, ts).transpose(0, 2, 4, 1, 3).copy()


@pytest.mark.parametrize("dt,C,K,ks", [
    ("f16", 16, 128, (3, 3)), ("bf16", 24, 40, (3, 3)), ("f16", 12, 8, (3, 3, 3)),
    ("f32", 8, 130, (3, 3)), ("f32", 6, 5, (1, 1)), ("bf16", 128, 128, (3, 3, 3)),
    ("f16", 3, 7, (1, 1)),
    # several 64-channel blocks and groups (the block-wise packing of whole groups)
    ("f16", 64, 200, (3, 3, 3)), ("f32", 32, 70, (3, 3)), ("bf16", 16, 130, (1, 1)),
    ("bf16", 40, 64, (3, 3)),
])
def test_pack_layout(dt, C, K, ks):
    import direct_implicit_gemm_amd as L
    rng = np.random.default_rng(31)
    w = W.Tensor.quantise(rng.standard_normal((K, C) + ks), dt)
    note(f"pack layout {dt} C={C} K={K} k={ks}")
    pw = L.pack_weights(w.torch("cuda"))
    torch.cuda.synchronize()
    se = 4 if dt == "f32" else 8
    want = _expected_packed(w.storage, se)
    got = pw.data.cpu().numpy().view(want.dtype).reshape(want.shape)
    np.testing.assert_array_equal(got, want)


PACKED_CASES = [
    # (tile, dims, dtype, N, C, spatial, K, relu); tiles reading 16-byte runs
    # need W % 8 == 0, the "_e" tiles (265, 275) take any W
    (260, 3, "f16", 1, 16, (5, 9, 40), 128, False),
    (261, 3, "bf16", 1, 24, (3, 7, 48), 200, True),    # C % 8 != 0 (zero-padded group)
    (262, 3, "f16", 2, 8, (4, 10, 56), 64, False),
    (263, 3, "bf16", 1, 40, (3, 6, 72), 96, True),
    (264, 3, "f16", 1, 16, (2, 9, 88), 130, False),     # K % 128 != 0
    (265, 3, "bf16", 1, 20, (3, 9, 35), 72, True),      # odd W, C % 16 != 0
    (270, 2, "bf16", 1, 32, (11, 40), 128, True),
    (271, 2, "f16", 2, 20, (9, 48), 72, False),        # C % 8 != 0, K % 64 != 0
    (272, 2, "f16", 1, 64, (7, 72), 256, True),
    (275, 2, "f16", 1, 24, (9, 33), 64, False),        # odd W
]


@pytest.mark.parametrize("case", range(len(PACKED_CASES)))
def test_forward_packed_forced_tile(case, monkeypatch):
    import direct_implicit_gemm_amd as L
    tile, dims, dt, N, C, sp, K, relu = PACKED_CASES[case]
    if dims == 2:
        layer = W.Layer("pk", dt, N, C, 1, sp[0], sp[1], K, 1, 3, 3, (0, 1, 1), (1, 1, 1),
                        "relu" if relu else "none", 2, "N01", "N01", "U0.05")
    else:
        layer = W.Layer("pk", dt, N, C, sp[0], sp[1], sp[2], K, 3, 3, 3, (1, 1, 1), (1, 1, 1),
                        "relu" if relu else "none", 3, "N01", "N01", "U0.05")
    x, w, b = W.make_inputs(layer, 700 + case)
    monkeypatch.setenv("LIBCONV_FORCE_TILE", str(tile))
    note(f"packed tile {tile}: {PACKED_CASES[case]}")
    st, pd = (layer.stride[1:], layer.pad[1:]) if dims == 2 else (layer.stride, layer.pad)
    q = L.libconv_query_plan(layer.N, C, layer.T, layer.H, layer.W, K, layer.KT, 3, 3,
                             *layer.pad, *layer.stride, W.DTYPE_CODE[dt], W.ACT_CODE[layer.act], 0,
                             0, BIG_WS)
    assert q[0] == 0 and q[2] == tile, q
    xt, wt, bt = x.torch("cuda"), w.torch("cuda"), b.torch("cuda")
    pw = L.pack_weights(wt)
    y_packed = to_f64(L.conv_nd_packed(xt, pw, bt, st, pd, layer.act))
    y_oihw = to_f64(L.conv_nd(xt, wt, bt, st, pd, layer.act))     # packs inside the call
    ref, s = oracle.conv(x.f64(), w.f64(), b.f64(), *oracle_args(layer), relu=relu)
    m = metrics(y_packed, ref, s, dt)
    note(f"  {m}")
    assert_gates(m, dt, f"packed {tile}")
    np.testing.assert_array_equal(y_oihw, y_packed)


def test_forward_packed_rejects_direct_only_shapes():
    import direct_implicit_gemm_amd as L
    # 5x5 kernels have no packed tiles: packing itself is unsupported
    assert L.libconv_packed_weight_bytes(8, 8, 1, 5, 5, L.F16) == -1
    x = torch.zeros((1, 8, 9, 9), dtype=torch.float16, device="cuda")
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    y = torch.zeros((1, 8, 9, 9), dtype=torch.float16, device="cuda")
    # 3x3 stride 2 16-bit: packed tiles exist only for stride 1
    st = L.libconv_forward_packed(x.data_ptr(), buf.data_ptr(), None, y.data_ptr(), 1, 8, 1, 9, 9,
                                  8, 1, 3, 3, 0, 1, 1, 1, 2, 2, L.F16, 0, None)
    assert st == 6
