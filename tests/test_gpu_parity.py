"""GPU parity of libconv against the fp64 oracle.

* every workload layer at a reduced size (same channels, kernel, stride, pad,
  activation, dtype; spatial extents that span several tiles and end in a
  ragged tail): every output compared;
* every workload layer at its full size, in the launch configuration the
  bench times: a sample of outputs (random plus every border row/column/frame
  and every output channel) compared one by one;
* both kernel families forced on every layer they support;
* bit-exact repeatability, untouched guard bands around the output, and
  edge shapes (ragged, 1x1 outputs, stride 3, kernel wider than the input,
  channel counts that are not multiples of the slot width, no bias).
"""
import sys

import numpy as np
import pytest

import oracle
import workloads as W
from convcheck import BIG_WS, assert_gates, gpu_forward, metrics, oracle_args, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import direct_implicit_gemm_amd as L
    assert L.libconv_device_supported(0) == 0, "device 0 is not gfx950"


def note(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


# Reduced versions of the workload layers (seed = 100 + index).
SMALL = {
    "c1": W.ALL_LAYERS["c1"],
    "c2_L1": W.ALL_LAYERS["c2_L1"].with_(H=70, W=83),
    "c2_L2": W.ALL_LAYERS["c2_L2"].with_(H=37, W=45),
    "c2_L3": W.ALL_LAYERS["c2_L3"].with_(H=37, W=45),
    "c2_L4": W.ALL_LAYERS["c2_L4"].with_(H=41, W=70),
    "c3_A": W.ALL_LAYERS["c3_A"].with_(N=2, H=19, W=70),
    "c3_B": W.ALL_LAYERS["c3_B"].with_(N=2, H=12, W=47),
    "c4_A": W.ALL_LAYERS["c4_A"].with_(N=1, H=10, W=36),
    "c4_B": W.ALL_LAYERS["c4_B"].with_(N=1, H=7, W=33),
    "c5_A": W.ALL_LAYERS["c5_A"].with_(T=5, H=9, W=40),
    "c5_B": W.ALL_LAYERS["c5_B"].with_(T=3, H=5, W=36),
}
SMALL_SEED = {name: 100 + i for i, name in enumerate(sorted(SMALL))}


def check_full(layer, seed, algo="auto", workspace=True):
    x, w, b = W.make_inputs(layer, seed)
    note(f"{layer.name} seed={seed} algo={algo} workspace={workspace} x={layer.x_shape} "
         f"w={layer.w_shape}")
    y = to_f64(gpu_forward(layer, x, w, b, algo, workspace=workspace))
    st, pd = oracle_args(layer)
    ref, s = oracle.conv(x.f64(), w.f64(), b.f64(), st, pd, relu=layer.act == "relu")
    assert y.shape == ref.shape
    m = metrics(y, ref, s, layer.dtype)
    note(f"  {m}")
    assert_gates(m, layer.dtype, layer.name)
    return m


@pytest.mark.parametrize("workspace", [True, False], ids=["workspace", "export"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_layer(name, workspace):
    """Every output of each reduced workload layer; `export`: through
    conv2d_forward / conv3d_forward themselves (no workspace)."""
    check_full(SMALL[name], SMALL_SEED[name], workspace=workspace)


def _supports(layer, algo):
    import direct_implicit_gemm_amd as L
    st, *_ = L.libconv_query_plan(layer.N, layer.C_in, layer.T, layer.H, layer.W, layer.C_out,
                                  layer.KT, layer.KH, layer.KW, *layer.pad, *layer.stride,
                                  W.DTYPE_CODE[layer.dtype], W.ACT_CODE[layer.act],
                                  {"direct": 1, "igemm": 2}[algo], 0, BIG_WS)
    return st == 0


@pytest.mark.parametrize("algo", ["direct", "igemm"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_layer_forced(name, algo):
    layer = SMALL[name]
    if not _supports(layer, algo):
        pytest.skip(f"{algo} has no tile for {name}")
    check_full(layer, SMALL_SEED[name], algo)


def _sample_indices(shape, rng, n_random=3000):
    """Random outputs plus every border position of every (n, co)."""
    nd = len(shape) - 2
    idx = [rng.integers(0, np.prod(shape), n_random)]
    grids = []
    N, CO = shape[:2]
    sp = shape[2:]
    for n in {0, N - 1}:
        for co in range(CO):
            # the eight corners / edges of the spatial box (first and last of each axis)
            for d in range(nd):
                for v in {0, sp[d] - 1}:
                    coords = [rng.integers(0, s) for s in sp]
                    coords[d] = v
                    grids.append(np.ravel_multi_index([n, co] + coords, shape))
    idx.append(np.array(grids, dtype=np.int64))
    return np.unique(np.concatenate(idx))


@pytest.mark.parametrize("workspace", [True, False], ids=["workspace", "export"])
@pytest.mark.parametrize("name", sorted(W.ALL_LAYERS))
def test_full_size_sampled(name, workspace):
    layer = W.ALL_LAYERS[name]
    x, w, b = W.make_inputs(layer)
    note(f"{name} full size x={layer.x_shape} w={layer.w_shape} (workload inputs) "
         f"workspace={workspace}")
    y = to_f64(gpu_forward(layer, x, w, b, workspace=workspace))
    rng = np.random.default_rng(7)
    idx = _sample_indices(y.shape, rng)
    st, pd = oracle_args(layer)
    ref, s = oracle.conv_points(x.f64(), w.f64(), b.f64(), idx, st, pd,
                                relu=layer.act == "relu")
    m = metrics(y.ravel()[idx], ref, s, layer.dtype)
    note(f"  sampled {m}")
    assert_gates(m, layer.dtype, name)
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("name", ["c2_L1", "c2_L2", "c3_A", "c5_B"])
def test_bitwise_repeatable(name):
    layer = SMALL[name]
    x, w, b = W.make_inputs(layer, SMALL_SEED[name])
    note(f"repeatability {name}")
    outs = [gpu_forward(layer, x, w, b).cpu() for _ in range(3)]
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16 if o.element_size() == 2 else torch.int32),
                           outs[0].view(torch.int16 if o.element_size() == 2 else torch.int32))


@pytest.mark.parametrize("name,algo", [("c2_L1", "direct"), ("c2_L2", "igemm"),
                                       ("c3_B", "igemm"), ("c5_A", "igemm"),
                                       ("c4_A", "igemm"), ("c2_L3", "direct")])
def test_guard_bands(name, algo):
    """Sentinels right before and after y stay untouched."""
    import direct_implicit_gemm_amd as L
    layer = SMALL[name]
    x, w, b = W.make_inputs(layer, SMALL_SEED[name])
    note(f"guard bands {name} {algo}")
    xt, wt, bt = x.torch("cuda"), w.torch("cuda"), b.torch("cuda")
    st, pd = (layer.stride[1:], layer.pad[1:]) if layer.dims == 2 else (layer.stride, layer.pad)
    ref = L.conv_nd(xt, wt, bt, st, pd, layer.act, algo)
    pad = 4096
    buf = torch.full((ref.numel() + 2 * pad,), -7.0, dtype=ref.dtype, device="cuda")
    out = buf[pad:pad + ref.numel()].view(ref.shape)
    L.conv_nd(xt, wt, bt, st, pd, layer.act, algo, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == -7.0) and torch.all(buf[pad + ref.numel():] == -7.0)
    assert torch.equal(out, ref)


EDGE = [
    # dims, dtype, N, C, (T,) H, W, K, k, stride, pad, act, bias
    (2, "f32", 1, 5, (7, 9), 6, 3, 1, 1, "relu", True),
    (2, "f32", 2, 3, (1, 1), 4, 3, 1, 1, "none", True),       # 1x1 input, pad 1
    (2, "f32", 1, 4, (13, 11), 3, 3, 3, 0, "none", False),     # stride 3, no bias
    (2, "f16", 1, 16, (5, 6), 40, 5, 1, 2, "relu", True),      # 5x5: direct only
    (2, "f16", 1, 12, (9, 40), 24, 3, 1, 1, "none", True),     # C % 8 != 0
    (2, "bf16", 3, 8, (3, 2), 8, 3, 1, 1, "none", True),       # tiny planes
    (2, "f16", 1, 24, (33, 65), 136, 3, 1, 1, "relu", False),  # ragged co and px tiles
    (2, "bf16", 1, 8, (2, 2), 4, 3, 1, 2, "none", True),       # output wider than input
    (2, "f32", 1, 8, (20, 20), 10, 3, 2, 1, "relu", True),     # s2, K not a tile multiple
    (2, "f16", 2, 8, (17, 19), 8, 1, 1, 0, "none", True),      # 1x1 flat, ragged
    (2, "f32", 1, 4, (33, 35), 8, 1, 1, 0, "relu", True),      # 1x1 flat fp32
    (3, "f16", 1, 8, (2, 7, 9), 16, 3, 1, 1, "relu", True),    # T=2
    (3, "bf16", 1, 16, (4, 5, 33), 40, 3, 1, 1, "none", True),
    (3, "f32", 1, 3, (5, 6, 7), 4, 3, 2, 1, "none", True),     # 3-D stride 2: direct
    (3, "f16", 1, 8, (1, 4, 4), 8, 3, 1, 1, "none", True),     # T=1 with time padding
]


@pytest.mark.parametrize("case", range(len(EDGE)))
@pytest.mark.parametrize("algo", ["auto", "direct", "igemm"])
def test_edge_shapes(case, algo):
    dims, dt, N, C, sp, K, k, s, p, act, bias = EDGE[case]
    if dims == 2:
        layer = W.Layer("edge", dt, N, C, 1, sp[0], sp[1], K, 1, k, k, (0, p, p), (1, s, s),
                        act, 2, "N01", "N01", "U0.1" if bias else "zero")
    else:
        layer = W.Layer("edge", dt, N, C, sp[0], sp[1], sp[2], K, k, k, k, (p, p, p),
                        (s, s, s), act, 3, "N01", "N01", "U0.1" if bias else "zero")
    if algo != "auto" and not _supports(layer, algo):
        pytest.skip(f"{algo} has no tile")
    x, w, b = W.make_inputs(layer, 500 + case)
    if not bias:
        b = None
    note(f"edge {case} {algo} {EDGE[case]}")
    y = to_f64(gpu_forward(layer, x, w, b, algo))
    st, pd = oracle_args(layer)
    ref, sm = oracle.conv(x.f64(), w.f64(), None if b is None else b.f64(), st, pd,
                          relu=act == "relu")
    m = metrics(y, ref, sm, dt)
    note(f"  {m}")
    assert_gates(m, dt, f"edge {case}")


def test_empty_batch_touches_nothing():
    import direct_implicit_gemm_amd as L
    y = torch.full((4,), 3.0, device="cuda")
    x = torch.zeros(4, device="cuda")
    w = torch.zeros(4, device="cuda")
    st = L.conv2d_forward(x.data_ptr(), w.data_ptr(), None, y.data_ptr(), 0, 1, 2, 2, 1, 1, 1,
                          0, 0, 1, 1, L.F32, 0, None)
    torch.cuda.synchronize()
    assert st == 0 and torch.all(y == 3.0)


def test_ocr_stack_chained():
    """The OCR stack run layer after layer on the GPU (reduced plane) against the
    oracle run layer after layer on the CPU from the same input."""
    layers = [W.ALL_LAYERS[n].with_(H=h, W=wd) for n, h, wd in
              [("c2_L1", 66, 70), ("c2_L2", 33, 35), ("c2_L3", 33, 35), ("c2_L4", 33, 35)]]
    x, _, _ = W.make_inputs(layers[0], 900)
    xg = x.torch("cuda")
    xr = x.f64()
    for i, layer in enumerate(layers):
        _, w, b = W.make_inputs(layer, 901 + i)
        import direct_implicit_gemm_amd as L
        st, pd = oracle_args(layer)
        note(f"chain layer {i} {layer.name}")
        xg = L.conv_nd(xg, w.torch("cuda"), b.torch("cuda"), st, pd, layer.act)
        xr, s = oracle.conv(xr, w.f64(), b.f64(), st, pd, relu=True)
        xr = xr.astype(np.float32).astype(np.float64)
    m = metrics(to_f64(xg), xr, s, "f32")
    note(f"  chain end {m}")
    assert m["nrmse"] < 1e-5
