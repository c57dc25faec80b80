"""Channel-packed activations on the GPU: the conversions against the
oracle's packing definition (bit for bit), and convolutions that read and
write the packed layout against the fp64 oracle (the outputs are unpacked by
the oracle's own definition, on the host).

Every MFMA tile made for the layout is forced on a small layer of its own
geometry and dtype (ragged channel groups, output-channel and pixel tails,
time padding); the vector-ALU kernel takes the shapes those tiles do not
cover.  The channels past C_out in the last output group must be zero.  The
full-size layers are the video-VAE's and the diffusion UNet's, on sampled
outputs."""
import numpy as np
import pytest

import oracle
import workloads as W
from convcheck import BIG_WS, assert_gates, metrics, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"[gpu] {msg}", flush=True)


def _group(dtype):
    return 4 if dtype == "f32" else 8


def _packed_numpy(xp, dtype):
    """The raw bytes of a packed device tensor as a numpy array of the
    storage type, shaped [N][groups][spatial...][g]."""
    g = _group(dtype)
    n, c = xp.shape[:2]
    raw = xp.data.cpu().numpy()
    np_dt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[dtype]
    return raw.view(np_dt).reshape((n, -(-c // g)) + tuple(xp.shape[2:]) + (g,))


def _to_f64(a, dtype):
    if dtype == "bf16":
        return W.bf16_bits_to_f64(a)
    return a.astype(np.float64)


@pytest.mark.parametrize("dtype,shape", [
    ("f16", (2, 13, 5, 7)), ("bf16", (1, 16, 3, 4, 9)), ("f32", (2, 6, 2, 3, 5)),
    ("f32", (1, 3, 8, 8)), ("bf16", (1, 1, 1, 3)),
])
def test_pack_unpack_match_oracle(dtype, shape):
    import direct_implicit_gemm_amd as L
    rng = np.random.default_rng(40)
    x = W.Tensor.quantise(rng.standard_normal(shape), dtype)
    note(f"pack/unpack {dtype} {shape}")
    xt = x.torch("cuda")
    xp = L.pack_activations(xt)
    back = L.unpack_activations(xp)
    torch.cuda.synchronize()
    want = oracle.pack_channels(x.storage, _group(dtype))
    np.testing.assert_array_equal(_packed_numpy(xp, dtype), want)
    assert torch.equal(back, xt)


# tile, dtype, C, K, T, H, W, (KT, KH, KW), stride (t, h, w), pad (t, h, w), pad_t_back, relu
TILE_CASES = [
    (280, "f16", 16, 72, 4, 9, 40, (3, 3, 3), (1, 1, 1), (1, 1, 1), None, True),
    (280, "bf16", 20, 64, 5, 7, 33, (3, 3, 3), (1, 1, 1), (2, 1, 1), 0, False),  # causal, odd W
    (281, "bf16", 24, 136, 3, 10, 48, (3, 3, 3), (1, 1, 1), (1, 1, 1), None, True),
    # eight waves, 64 x 128 per wave: 19 rows leave a ragged second 16-row tile
    (279, "f16", 24, 136, 3, 19, 40, (3, 3, 3), (1, 1, 1), (1, 1, 1), None, True),
    (279, "bf16", 16, 64, 4, 17, 72, (3, 3, 3), (1, 1, 1), (2, 1, 1), 0, False),  # causal
    (282, "f16", 20, 70, 1, 19, 72, (1, 3, 3), (1, 1, 1), (0, 1, 1), None, True),  # K % 8 != 0
    (283, "bf16", 32, 200, 1, 11, 40, (1, 3, 3), (1, 1, 1), (0, 1, 1), None, False),
    (284, "f16", 16, 72, 1, 21, 75, (1, 3, 3), (1, 2, 2), (0, 1, 1), None, True),
    (285, "f16", 64, 200, 1, 7, 33, (1, 1, 1), (1, 1, 1), (0, 0, 0), None, True),
    (285, "bf16", 40, 96, 3, 5, 16, (1, 1, 1), (1, 1, 1), (0, 0, 0), None, False),  # frames
    (290, "f32", 12, 40, 1, 17, 40, (1, 3, 3), (1, 1, 1), (0, 1, 1), None, True),
    (291, "f32", 8, 70, 1, 19, 67, (1, 3, 3), (1, 2, 2), (0, 1, 1), None, True),
    (292, "f32", 32, 70, 1, 9, 31, (1, 1, 1), (1, 1, 1), (0, 0, 0), None, False),
    # a 3-channel stem (one group, padded) and 5 channels: fewer groups than a stage
    (291, "f32", 3, 32, 1, 40, 64, (1, 3, 3), (1, 2, 2), (0, 1, 1), None, True),
    (290, "f32", 5, 24, 1, 12, 36, (1, 3, 3), (1, 1, 1), (0, 1, 1), None, False),
    (282, "bf16", 3, 16, 1, 10, 33, (1, 3, 3), (1, 1, 1), (0, 1, 1), None, True),
]


def _case_layer(case):
    tid, dt, C, K, T, H, Wd, ks, st, pd, pb, relu = case
    dims = 3 if T > 1 or ks[0] > 1 else 2
    return W.Layer("cpack", dt, 1, C, T, H, Wd, K, *ks, pd, st, "relu" if relu else "none",
                   dims, "N01", "N01", "U0.05", pad_t_back=pb), tid


def _run_cpack(layer, x, w, b, packed_w):
    import direct_implicit_gemm_amd as L
    xt = x.torch("cuda")
    wt = w.torch("cuda")
    wq = L.pack_weights(wt) if packed_w else wt
    xp = L.pack_activations(xt)
    if layer.dims == 2:
        yp = L.conv_cpack(xp, wq, b.torch("cuda"), layer.stride[1:], layer.pad[1:], act=layer.act)
    else:
        pt = None if layer.pad_t_back is None else (layer.pad[0], layer.pad_t_back)
        yp = L.conv_cpack(xp, wq, b.torch("cuda"), layer.stride, layer.pad, pad_t=pt,
                          act=layer.act)
    torch.cuda.synchronize()
    return yp


def _check(layer, x, w, b, yp, what):
    ref, s = oracle.conv(x.f64(), w.f64(), b.f64(), layer.stride if layer.dims == 3 else
                         layer.stride[1:], layer.pad if layer.dims == 3 else layer.pad[1:],
                         relu=layer.act == "relu", pad_t_back=layer.pad_t_back)
    packed = _packed_numpy(yp, layer.dtype)
    y = _to_f64(oracle.unpack_channels(packed, layer.C_out), layer.dtype)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    # the channels past C_out of the last group hold zeros
    k_last = layer.C_out % _group(layer.dtype)
    if k_last:
        assert not _to_f64(packed[:, -1, ..., k_last:], layer.dtype).any(), what
    m = metrics(y, ref, s, layer.dtype)
    note(f"  {m}")
    assert_gates(m, layer.dtype, what)


@pytest.mark.parametrize("case", TILE_CASES, ids=lambda c: f"t{c[0]}_{c[1]}_C{c[2]}_K{c[3]}")
def test_cpack_tiles(case, monkeypatch):
    import direct_implicit_gemm_amd as L
    layer, tid = _case_layer(case)
    monkeypatch.setenv("LIBCONV_FORCE_TILE", str(tid))
    note(f"cpack tile {tid} {L.libconv_tile_name(tid)}: x={layer.x_shape} w={layer.w_shape} "
         f"{layer.dtype} pad={layer.pad} back={layer.pad_t_back} stride={layer.stride} {layer.act}")
    x, w, b = W.make_inputs(layer, 1000 + case[2] + case[3])
    yp = _run_cpack(layer, x, w, b, packed_w=True)
    _check(layer, x, w, b, yp, f"tile {tid}")


# The tiles that read OI(D)HW weights (transposed in registers; no workspace
# to pack them into): C a multiple of the channel group, ragged stages
# (C not a multiple of the stage's 16 / 8 channels), ragged K, odd widths,
# one-sided time padding.
XO_CASES = [
    (286, "f16", 24, 72, 4, 9, 40, (3, 3, 3), (1, 1, 1), (1, 1, 1), None, True),
    (286, "bf16", 16, 64, 5, 7, 33, (3, 3, 3), (1, 1, 1), (2, 1, 1), 0, False),  # causal, odd W
    (287, "f16", 40, 70, 1, 19, 72, (1, 3, 3), (1, 1, 1), (0, 1, 1), None, True),  # K % 8 != 0
    (287, "bf16", 32, 136, 1, 11, 35, (1, 3, 3), (1, 1, 1), (0, 1, 1), None, False),
    (288, "f16", 24, 72, 1, 21, 75, (1, 3, 3), (1, 2, 2), (0, 1, 1), None, True),
    (289, "f16", 64, 200, 1, 7, 33, (1, 1, 1), (1, 1, 1), (0, 0, 0), None, True),
    (289, "bf16", 72, 96, 3, 5, 16, (1, 1, 1), (1, 1, 1), (0, 0, 0), None, False),  # frames
    (293, "f32", 12, 40, 1, 17, 40, (1, 3, 3), (1, 1, 1), (0, 1, 1), None, True),
    (294, "f32", 8, 70, 1, 19, 67, (1, 3, 3), (1, 2, 2), (0, 1, 1), None, True),
    (295, "f32", 36, 70, 1, 9, 31, (1, 1, 1), (1, 1, 1), (0, 0, 0), None, False),
]


@pytest.mark.parametrize("case", XO_CASES, ids=lambda c: f"t{c[0]}_{c[1]}_C{c[2]}_K{c[3]}")
def test_cpack_tiles_unpacked_weights(case, monkeypatch):
    import direct_implicit_gemm_amd as L
    layer, tid = _case_layer(case)
    monkeypatch.setenv("LIBCONV_FORCE_TILE", str(tid))
    note(f"cpack tile {tid} {L.libconv_tile_name(tid)} (OI(D)HW weights): x={layer.x_shape} "
         f"w={layer.w_shape} {layer.dtype} pad={layer.pad} back={layer.pad_t_back} "
         f"stride={layer.stride} {layer.act}")
    x, w, b = W.make_inputs(layer, 1200 + case[2] + case[3])
    yp = _run_cpack(layer, x, w, b, packed_w=False)
    _check(layer, x, w, b, yp, f"tile {tid}")


AUTO_CASES = [
    # shapes no MFMA tile of the layout covers (5x5, 3x3 stride 2 in 3-D):
    # the vector-ALU kernel, with OIHW weights
    ("f16", 8, 12, 1, 12, 20, (1, 5, 5), (1, 1, 1), (0, 2, 2), None, True),
    ("f32", 3, 32, 1, 33, 40, (1, 3, 3), (1, 2, 2), (0, 1, 1), None, True),
    ("bf16", 6, 10, 5, 8, 12, (3, 3, 3), (2, 2, 2), (1, 1, 1), None, False),
    # MFMA shapes with OIHW weights (packed into a temporary by the call)
    ("f16", 32, 64, 3, 8, 32, (3, 3, 3), (1, 1, 1), (1, 1, 1), None, True),
    ("f32", 32, 32, 1, 16, 40, (1, 3, 3), (1, 1, 1), (0, 1, 1), None, True),
]


@pytest.mark.parametrize("case", AUTO_CASES, ids=lambda c: f"{c[0]}_k{c[6][1]}s{c[7][1]}_C{c[1]}")
def test_cpack_dispatched(case):
    dt, C, K, T, H, Wd, ks, st, pd, pb, relu = case
    layer, _ = _case_layer((0,) + case)
    note(f"cpack auto: x={layer.x_shape} w={layer.w_shape} {dt} stride={st}")
    x, w, b = W.make_inputs(layer, 1100 + C + K)
    yp = _run_cpack(layer, x, w, b, packed_w=False)
    _check(layer, x, w, b, yp, "auto")


def test_cpack_chain_stays_packed():
    """Two layers in a row on packed activations (the second reads the
    first's packed output directly) against the oracle applied to the first
    layer's rounded output."""
    import direct_implicit_gemm_amd as L
    l1 = W.Layer("c1", "f16", 1, 16, 3, 12, 40, 40, 3, 3, 3, (1, 1, 1), (1, 1, 1), "relu", 3,
                 "N01", "N01", "U0.05")
    l2 = l1.with_(C_in=40, C_out=24)
    x, w1, b1 = W.make_inputs(l1, 1201)
    _, w2, b2 = W.make_inputs(l2, 1202)
    note("cpack chain of two 3x3x3 layers")
    xp = L.pack_activations(x.torch("cuda"))
    y1 = L.conv_cpack(xp, L.pack_weights(w1.torch("cuda")), b1.torch("cuda"), 1, 1, act="relu")
    y2 = L.conv_cpack(y1, L.pack_weights(w2.torch("cuda")), b2.torch("cuda"), 1, 1, act="relu")
    torch.cuda.synchronize()
    h = _to_f64(oracle.unpack_channels(_packed_numpy(y1, "f16"), 40), "f16")
    ref, s = oracle.conv(h, w2.f64(), b2.f64(), 1, 1, relu=True)
    y = _to_f64(oracle.unpack_channels(_packed_numpy(y2, "f16"), 24), "f16")
    m = metrics(y, ref, s, "f16")
    note(f"  {m}")
    assert_gates(m, "f16", "chain")


@pytest.mark.parametrize("name", ["c5_A", "c5_B", "c4_A"])
def test_cpack_full_size_sampled(name):
    import direct_implicit_gemm_amd as L
    layer = W.ALL_LAYERS[name]
    x, w, b = W.make_inputs(layer)
    note(f"cpack full size {name} x={layer.x_shape} {layer.dtype}")
    xp = L.pack_activations(x.torch("cuda"))
    st, pd = (layer.stride[1:], layer.pad[1:]) if layer.dims == 2 else (layer.stride, layer.pad)
    yp = L.conv_cpack(xp, L.pack_weights(w.torch("cuda")), b.torch("cuda"), st, pd,
                      act=layer.act)
    y = to_f64(L.unpack_activations(yp))
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    idx = np.unique(np.concatenate([rng.integers(0, y.size, 3000),
                                    [0, y.size - 1]]))
    ref, s = oracle.conv_points(x.f64(), w.f64(), b.f64(), idx, st, pd, relu=layer.act == "relu")
    m = metrics(y.ravel()[idx], ref, s, layer.dtype)
    note(f"  sampled {m}")
    assert_gates(m, layer.dtype, name)


@pytest.mark.parametrize("tid,dt,ks", [(282, "f16", 3), (283, "bf16", 2), (290, "f32", 2),
                                       (280, "bf16", 2), (279, "f16", 2)])
def test_cpack_split_k(tid, dt, ks, monkeypatch):
    """Split-K on packed activations: fp32 partial sums, then the sum kernel
    writes the packed output (with zeros past C_out)."""
    import direct_implicit_gemm_amd as L
    monkeypatch.setenv("LIBCONV_FORCE_TILE", str(tid))
    monkeypatch.setenv("LIBCONV_FORCE_KSPLIT", str(ks))
    if tid in (279, 280):
        layer = W.Layer("cpk", dt, 1, 64, 3, 9 if tid == 280 else 19, 40, 70, 3, 3, 3, (1, 1, 1),
                        (1, 1, 1), "relu", 3, "N01", "N01", "U0.05")
    else:
        layer = W.Layer("cpk", dt, 2, 96 if dt != "f32" else 48, 1, 11, 40, 70, 1, 3, 3,
                        (0, 1, 1), (1, 1, 1), "relu", 2, "N01", "N01", "U0.05")
    dims = (layer.N, layer.C_in, layer.T, layer.H, layer.W, layer.C_out, layer.KT, layer.KH,
            layer.KW, *layer.pad, *layer.stride)
    q = L.libconv_query_plan(*dims, W.DTYPE_CODE[dt], 1, 0, L.PLAN_CPACK, BIG_WS)
    assert q[0] == 0 and q[2] == tid and q[4] == ks, q
    note(f"cpack split-K tile {tid} ks={ks}: x={layer.x_shape} w={layer.w_shape} {dt}")
    x, w, b = W.make_inputs(layer, 1300 + tid + ks)
    yp = _run_cpack(layer, x, w, b, packed_w=False)
    _check(layer, x, w, b, yp, f"split {tid}/{ks}")


def test_cpack_batch_no_bias():
    """N = 3, no bias, through a forced packed tile and the vector-ALU kernel."""
    import direct_implicit_gemm_amd as L
    import os
    for tid, ks in ((282, (1, 3, 3)), (None, (1, 5, 5))):
        layer = W.Layer("cpb", "f16", 3, 24, 1, 11, 40, 40, *ks, (0, ks[1] // 2, ks[2] // 2),
                        (1, 1, 1), "none", 2, "N01", "N01", "zero")
        x, w, b = W.make_inputs(layer, 1500 + (tid or 0))
        if tid:
            os.environ["LIBCONV_FORCE_TILE"] = str(tid)
        try:
            note(f"cpack N=3 no bias, tile {tid}, kernel {ks}")
            xp = L.pack_activations(x.torch("cuda"))
            wq = L.pack_weights(w.torch("cuda")) if tid else w.torch("cuda")
            yp = L.conv_cpack(xp, wq, None, 1, layer.pad[1:])
            torch.cuda.synchronize()
        finally:
            os.environ.pop("LIBCONV_FORCE_TILE", None)
        ref, s = oracle.conv(x.f64(), w.f64(), None, 1, layer.pad[1:])
        y = _to_f64(oracle.unpack_channels(_packed_numpy(yp, "f16"), 40), "f16")
        m = metrics(y, ref, s, "f16")
        note(f"  {m}")
        assert_gates(m, "f16", f"cpack N=3 {tid}")
