"""Time padding on one side (conv3d_forward_tpad) on the GPU against the fp64
oracle: the causal 3-D convolution of the spatio-temporal VAE ("SeedVR2 NCNN
Vulkan", section 7.2) pads KT-1 frames before the first frame and none after.

Small shapes span several tiles and end in ragged tails; the full-size layers
are the video-VAE workload's layers made causal, checked on sampled outputs."""
import numpy as np
import pytest

import oracle
import workloads as W
from convcheck import assert_gates, metrics, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"[gpu] {msg}", flush=True)


def _run(layer, x, w, b, pf, pb, packed):
    import direct_implicit_gemm_amd as L
    wt = w.torch("cuda")
    wq = L.pack_weights(wt) if packed else wt
    return L.conv3d_tpad(x.torch("cuda"), wq, b.torch("cuda"), (pf, pb), layer.stride,
                         layer.pad[1:], layer.act)


def _check(layer, seed, pf, pb, packed):
    x, w, b = W.make_inputs(layer, seed)
    note(f"tpad {layer.name} x={layer.x_shape} w={layer.w_shape} {layer.dtype} "
         f"pad_t=({pf},{pb}) stride={layer.stride} packed={packed}")
    y = to_f64(_run(layer, x, w, b, pf, pb, packed))
    torch.cuda.synchronize()
    ref, s = oracle.conv(x.f64(), w.f64(), b.f64(), layer.stride, layer.pad,
                         relu=layer.act == "relu", pad_t_back=pb)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    m = metrics(y, ref, s, layer.dtype)
    note(f"  {m}")
    assert_gates(m, layer.dtype, layer.name)


def _small(dtype, C, K, T, H, Wd, st=1, pf=2, relu=True):
    return W.Layer("tpad", dtype, 1, C, T, H, Wd, K, 3, 3, 3, (pf, 1, 1), (st, 1, 1),
                   "relu" if relu else "none", 3, "N01", "N01", "U0.05")


CASES = [
    # dtype, C, K, T, H, W, stride_t, pad front, pad back, packed
    ("f16", 16, 72, 5, 9, 40, 1, 2, 0, False),    # causal, OIDHW weights
    ("bf16", 24, 130, 4, 10, 48, 1, 2, 0, True),  # causal, packed weights
    ("f16", 8, 64, 6, 7, 37, 1, 2, 0, False),     # W not a whole 16-byte run
    ("f32", 12, 20, 5, 6, 24, 1, 2, 0, False),    # fp32: the direct kernel
    ("f16", 16, 40, 7, 8, 32, 2, 2, 0, False),    # time stride 2
    ("bf16", 16, 96, 5, 6, 40, 1, 1, 2, True),    # more padding after than before
    ("f16", 8, 16, 3, 5, 16, 1, 0, 2, False),     # padding only after
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_C{c[1]}_T{c[3]}_s{c[6]}_p{c[7]}{c[8]}{'_pk' if c[9] else ''}")
def test_tpad_small(case):
    dt, C, K, T, H, Wd, st, pf, pb, packed = case
    layer = _small(dt, C, K, T, H, Wd, st, pf)
    _check(layer, 400 + C + T, pf, pb, packed)


def test_causal_frames_depend_only_on_past():
    """Output frame t reads input frames up to t: changing the last input
    frame leaves every earlier output frame bit-for-bit unchanged."""
    import direct_implicit_gemm_amd as L
    layer = _small("f16", 16, 64, 5, 8, 32, 1, 2, relu=False)
    x, w, b = W.make_inputs(layer, 77)
    xt = x.torch("cuda")
    y1 = L.conv3d_tpad(xt, w.torch("cuda"), b.torch("cuda"), (2, 0), 1, 1)
    x2 = xt.clone()
    x2[:, :, -1] += 1
    y2 = L.conv3d_tpad(x2, w.torch("cuda"), b.torch("cuda"), (2, 0), 1, 1)
    torch.cuda.synchronize()
    assert torch.equal(y1[:, :, :-1], y2[:, :, :-1])
    assert not torch.equal(y1[:, :, -1], y2[:, :, -1])


@pytest.mark.parametrize("name", ["c5_A", "c5_B"])
def test_causal_full_size_sampled(name):
    base = W.ALL_LAYERS[name]
    layer = base.with_(pad=(2, 1, 1))
    x, w, b = W.make_inputs(base)
    note(f"causal {name} full size x={layer.x_shape} (workload inputs), pad_t=(2,0)")
    y = to_f64(_run(layer, x, w, b, 2, 0, packed=False))
    rng = np.random.default_rng(8)
    idx = np.unique(np.concatenate([rng.integers(0, y.size, 3000),
                                    # every output frame's first and last row of co 0
                                    [np.ravel_multi_index((0, 0, t, r, c), y.shape)
                                     for t in range(y.shape[2]) for r in (0, y.shape[3] - 1)
                                     for c in (0, y.shape[4] - 1)]]))
    ref, s = oracle.conv_points(x.f64(), w.f64(), b.f64(), idx, layer.stride, layer.pad,
                                relu=layer.act == "relu", pad_t_back=0)
    m = metrics(y.ravel()[idx], ref, s, layer.dtype)
    note(f"  sampled {m}")
    assert_gates(m, layer.dtype, name)
