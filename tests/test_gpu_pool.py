"""conv2d_forward_pool: convolution, activation and 2x2 stride-2 max pooling
in one MFMA kernel (the conv + activation + pool fusion of the detector in
"PP-OCR on Vulkan compute shaders", section 4.4), against the fp64 oracle's
conv, activation and pooling; and bit-for-bit against the same kernel's
unpooled output pooled on the host (the max is taken before the one
rounding, which commutes with it)."""
import re

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


def _pool_ref(layer, x, w, b):
    st, pd = layer.stride[1:], layer.pad[1:]
    y, s = oracle.conv(x.f64(), w.f64(), b.f64(), st, pd, relu=layer.act == "relu")
    ref = oracle.max_pool2x2(y)
    # error scale of a pooled output: the largest S of its window
    return ref, oracle.max_pool2x2(s)


CASES = [
    # dtype, N, C, H, W, K, stride, act
    ("f32", 1, 32, 40, 72, 40, 1, "relu"),
    ("f32", 2, 16, 21, 45, 24, 1, "none"),     # odd H / W: last row and column dropped
    ("f16", 2, 64, 24, 160, 128, 1, "relu"),   # the text-recognition layer's shape
    ("bf16", 1, 40, 17, 56, 72, 1, "none"),    # ragged channels and rows
    ("f16", 1, 24, 30, 70, 48, 2, "relu"),     # stride 2
    ("f32", 1, 64, 34, 64, 64, 2, "relu"),     # stride 2, fp32
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_conv_pool(case):
    import direct_implicit_gemm_amd as L
    dt, N, C, H, Wd, K, s, act = case
    layer = W.Layer("pool", dt, N, C, 1, H, Wd, K, 1, 3, 3, (0, 1, 1), (1, s, s), act, 2,
                    "N01", "N01", "U0.05")
    x, w, b = W.make_inputs(layer, 500 + H + K)
    q = L.libconv_query_plan(N, C, 1, H, Wd, K, 1, 3, 3, 0, 1, 1, 1, s, s,
                             W.DTYPE_CODE[dt], W.ACT_CODE[act], 0, L.PLAN_POOL2, BIG_WS)
    note(f"pool {case}: tile {L.libconv_tile_name(q[2])}")
    y = to_f64(L.conv2d_pool(x.torch("cuda"), w.torch("cuda"), b.torch("cuda"), s, 1, act))
    ref, sp = _pool_ref(layer, x, w, b)
    assert y.shape == ref.shape
    m = metrics(y, ref, sp, dt)
    note(f"  {m}")
    assert_gates(m, dt, "conv+pool")


def _pool_tiles():
    import direct_implicit_gemm_amd as L
    out = []
    for tid in range(200, 300):
        name = L.libconv_tile_name(tid)
        m = re.match(r"igemm(16|32)(p?)_k3(s(\d))?_m\d+w?_n\d+x\d+", name)
        if m:
            out.append((tid, name, m.group(1) == "16", m.group(2) == "p", int(m.group(4) or 1)))
    return out


def test_every_pool_tile_matches_unfused(monkeypatch):
    """Each tile that can pool, forced: the fused output equals the same
    tile's unpooled output pooled on the host, bit for bit."""
    import direct_implicit_gemm_amd as L
    ran = 0
    for i, (tid, name, wide, packed, s) in enumerate(_pool_tiles()):
        dt = ("bf16" if i % 2 else "f16") if wide else "f32"
        se = 8 if wide else 4
        C = 2 * se * 2
        H, Wd = (19, 72) if s == 1 else (37, 144)
        layer = W.Layer("pt", dt, 1, C, 1, H, Wd, 72, 1, 3, 3, (0, 1, 1), (1, s, s), "relu", 2,
                        "N01", "N01", "U0.05")
        monkeypatch.setenv("LIBCONV_FORCE_TILE", str(tid))
        q = L.libconv_query_plan(1, C, 1, H, Wd, 72, 1, 3, 3, 0, 1, 1, 1, s, s,
                                 W.DTYPE_CODE[dt], 1, 0, L.PLAN_POOL2, BIG_WS)
        if q[0] != 0 or q[2] != tid:
            continue  # this tile does not pool
        x, w, b = W.make_inputs(layer, 600 + i)
        note(f"pool tile {tid} {name} {dt}")
        xt, wt, bt = x.torch("cuda"), w.torch("cuda"), b.torch("cuda")
        if packed:
            wq = L.pack_weights(wt)
            full = L.conv_nd_packed(xt, wq, bt, s, 1, "relu")
        else:
            full = L.conv_nd(xt, wt, bt, s, 1, "relu")
        pooled = L.conv2d_pool(xt, wt, bt, s, 1, "relu")
        torch.cuda.synchronize()
        host = torch.nn.functional.max_pool2d(full.float().cpu(), 2, 2).to(full.dtype)
        assert torch.equal(pooled.cpu(), host), name
        ran += 1
    assert ran >= 8


def test_pool_rejects():
    import direct_implicit_gemm_amd as L
    dev = "cuda"
    x = torch.zeros(1, 3, 32, 32, device=dev)
    w = torch.zeros(8, 3, 3, 3, device=dev)
    with pytest.raises(L.LibconvError) as e:  # 3 input channels: no MFMA tile takes it
        L.conv2d_pool(x, w, None, 1, 1)
    assert e.value.status == 6
    x = torch.zeros(1, 32, 1, 40, device=dev)
    w = torch.zeros(8, 32, 1, 3, device=dev)
    with pytest.raises(L.LibconvError) as e:  # one output row: nothing to pool
        L.conv2d_pool(x, w, None, 1, 0)
    assert e.value.status == 2


def test_ocr_pool_block_full_size():
    """The bench's fused OCR conv + ReLU + pool block at full size (workload
    inputs), every pooled output against the oracle."""
    import direct_implicit_gemm_amd as L
    (layer,) = W.EXTRA_WORKLOADS["ocr_pool_f32"][1]
    x, w, b = W.make_inputs(layer)
    note(f"ocr pool block full size x={layer.x_shape}")
    y = to_f64(L.conv2d_pool(x.torch("cuda"), w.torch("cuda"), b.torch("cuda"), 1, 1, "relu"))
    ref, sp = _pool_ref(layer, x, w, b)
    m = metrics(y, ref, sp, layer.dtype)
    note(f"  {m}")
    assert_gates(m, layer.dtype, "ocr pool block")
