"""A video convolution computed a few output frames at a time on the GPU
(conv3d_forward_frames) and streamed through the device in chunks
(conv3d_forward_chunked), against the fp64 oracle on the whole video.  The
long-video plan of "SeedVR2 NCNN Vulkan", section 9, cuts a video into
overlapping chunks of frames; per convolution the overlap is the frames
consecutive windows share.

Small shapes span several tiles and ragged tails, with causal, symmetric and
one-sided time padding, time stride 2, host and device tensors; with one
forced MFMA tile the pieces equal the whole-video call bit for bit.  The
full-size case is the video-VAE's 128-channel causal layer over 17 frames,
streamed from pinned host memory in chunks of 5 output frames."""
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


def _layer(dtype, C, K, T, H, Wd, st, pf, relu=True):
    return W.Layer("frames", dtype, 1, C, T, H, Wd, K, 3, 3, 3, (pf, 1, 1), (st, 1, 1),
                   "relu" if relu else "none", 3, "N01", "N01", "U0.05")


def _oracle(layer, x, w, b, pb):
    return oracle.conv(x.f64(), w.f64(), b.f64(), layer.stride, layer.pad,
                       relu=layer.act == "relu", pad_t_back=pb)


CASES = [
    # dtype, C, K, T, H, W, stride_t, pad front, pad back, packed
    ("f16", 16, 72, 7, 9, 40, 1, 2, 0, False),    # causal
    ("bf16", 24, 130, 6, 10, 48, 1, 2, 0, True),  # causal, packed weights
    ("f16", 16, 64, 9, 6, 32, 2, 1, 1, False),    # time stride 2
    ("f32", 12, 20, 6, 6, 24, 1, 1, 1, False),    # fp32: the direct kernel
    ("bf16", 8, 96, 5, 7, 40, 1, 0, 2, True),     # padding only after
    ("f16", 16, 64, 10, 6, 32, 3, 0, 0, False),   # stride = KT: windows share no frame
    ("bf16", 8, 64, 13, 6, 32, 4, 1, 0, True),    # stride > KT: frames between windows unread
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_T{c[3]}_s{c[6]}_p{c[7]}{c[8]}{'_pk' if c[9] else ''}")
@pytest.mark.parametrize("chunk", [1, 2, 3])
def test_frames_windows(case, chunk):
    import direct_implicit_gemm_amd as L
    dt, C, K, T, H, Wd, st, pf, pb, packed = case
    layer = _layer(dt, C, K, T, H, Wd, st, pf)
    x, w, b = W.make_inputs(layer, 600 + C + T)
    ref, s = _oracle(layer, x, w, b, pb)
    ot = ref.shape[2]
    xt = x.torch("cuda")
    wt = w.torch("cuda")
    wq = L.pack_weights(wt) if packed else wt
    bt = b.torch("cuda")
    note(f"frames {dt} C={C} K={K} T={T} st={st} pad_t=({pf},{pb}) packed={packed} chunk={chunk}")
    for o0 in range(0, ot, chunk):
        on = min(chunk, ot - o0)
        status, f0, tw = L.libconv_frame_window(T, 3, pf, pb, st, o0, on)
        assert status == 0
        xw = xt[:, :, f0:f0 + tw].contiguous()
        y = L.conv3d_frames(xw, wq, bt, T, (o0, on), (pf, pb), layer.stride, 1, layer.act)
        torch.cuda.synchronize()
        m = metrics(to_f64(y), ref[:, :, o0:o0 + on], s[:, :, o0:o0 + on], dt)
        note(f"  out frames [{o0}, {o0 + on}) from input frames [{f0}, {f0 + tw}): {m}")
        assert_gates(m, dt, f"frames {o0}+{on}")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}_T{c[3]}_s{c[6]}_p{c[7]}{c[8]}{'_pk' if c[9] else ''}")
@pytest.mark.parametrize("where,chunk", [("host", 2), ("device", 3), ("host", 100)])
def test_chunked_driver(case, where, chunk):
    import direct_implicit_gemm_amd as L
    dt, C, K, T, H, Wd, st, pf, pb, packed = case
    layer = _layer(dt, C, K, T, H, Wd, st, pf)
    x, w, b = W.make_inputs(layer, 700 + C + T)
    ref, s = _oracle(layer, x, w, b, pb)
    wt = w.torch("cuda")
    wq = L.pack_weights(wt) if packed else wt
    if where == "host":
        xs = torch.empty(x.shape, dtype=wt.dtype, pin_memory=True)
        xs.copy_(x.torch("cpu"))
    else:
        xs = x.torch("cuda")
    note(f"chunked {dt} C={C} K={K} T={T} st={st} pad_t=({pf},{pb}) packed={packed} "
         f"x on {where}, chunk={chunk}")
    y = L.conv3d_chunked(xs, wq, b.torch("cuda"), chunk, (pf, pb), layer.stride, 1, layer.act)
    torch.cuda.synchronize()
    assert y.is_cuda == (where == "device")
    m = metrics(to_f64(y), ref, s, dt)
    note(f"  {m}")
    assert_gates(m, dt, "chunked")


@pytest.mark.parametrize("where", ["host", "device"])
def test_chunks_equal_whole_video_one_tile(monkeypatch, where):
    """With one MFMA tile forced, every chunk runs the same kernel as the
    whole-video call, and the results agree bit for bit."""
    import direct_implicit_gemm_amd as L
    monkeypatch.setenv("LIBCONV_FORCE_TILE", "260")
    layer = _layer("f16", 16, 128, 11, 9, 40, 1, 2)
    x, w, b = W.make_inputs(layer, 811)
    wq = L.pack_weights(w.torch("cuda"))
    bt = b.torch("cuda")
    whole = L.conv3d_tpad(x.torch("cuda"), wq, bt, (2, 0), 1, 1, "relu")
    if where == "host":
        xs = torch.empty(x.shape, dtype=torch.float16, pin_memory=True)
        xs.copy_(x.torch("cpu"))
    else:
        xs = x.torch("cuda")
    for chunk in (1, 4, 5):
        note(f"one tile: x on {where}, chunk={chunk}")
        y = L.conv3d_chunked(xs, wq, bt, chunk, (2, 0), 1, 1, "relu")
        torch.cuda.synchronize()
        assert torch.equal(y.cuda(), whole)


def test_chunked_pageable_host_memory():
    """x and y in ordinary (pageable) host memory: the copies block the host
    but the result is the one pinned memory gives, bit for bit, and within
    the oracle gates."""
    import direct_implicit_gemm_amd as L
    layer = _layer("bf16", 16, 72, 8, 8, 40, 1, 2)
    x, w, b = W.make_inputs(layer, 813)
    ref, s = _oracle(layer, x, w, b, 0)
    wt, bt = w.torch("cuda"), b.torch("cuda")
    pinned = torch.empty(x.shape, dtype=torch.bfloat16, pin_memory=True)
    pinned.copy_(x.torch("cpu"))
    plain = x.torch("cpu").clone()
    assert not plain.is_pinned()
    note("chunked, pageable x and y")
    y_pinned = L.conv3d_chunked(pinned, wt, bt, 3, (2, 0), 1, 1, "relu")
    y_plain = L.conv3d_chunked(plain, wt, bt, 3, (2, 0), 1, 1, "relu",
                               out=torch.empty(tuple(y_pinned.shape), dtype=torch.bfloat16))
    torch.cuda.synchronize()
    assert not y_plain.is_pinned()
    assert torch.equal(y_plain, y_pinned)
    m = metrics(to_f64(y_plain), ref, s, "bf16")
    assert_gates(m, "bf16", "pageable")


@pytest.mark.parametrize("streams", ["one", "one_copy"])
def test_chunked_stream_modes(streams):
    """Everything on the compute stream, or both copy directions on one copy
    stream (the next window is copied in before the previous output is
    copied out)."""
    import direct_implicit_gemm_amd as L
    layer = _layer("f16", 16, 64, 6, 8, 32, 1, 2)
    x, w, b = W.make_inputs(layer, 812)
    ref, s = _oracle(layer, x, w, b, 0)
    cur = torch.cuda.current_stream().cuda_stream
    xs = torch.empty(x.shape, dtype=torch.float16, pin_memory=True)
    xs.copy_(x.torch("cpu"))
    side = torch.cuda.Stream().cuda_stream
    pair = (cur, cur) if streams == "one" else (side, side)
    note(f"chunked, streams: {streams}")
    y = L.conv3d_chunked(xs, w.torch("cuda"), b.torch("cuda"), 2, (2, 0), 1, 1, "relu",
                         copy_streams=pair)
    torch.cuda.synchronize()
    m = metrics(to_f64(y), ref, s, "f16")
    assert_gates(m, "f16", streams)


def test_chunked_long_video_full_size():
    """The video-VAE's 128-channel 3x3x3 layer, causal, over 17 frames of
    256x480 (535 MB per tensor in f16), streamed from pinned host memory in
    chunks of 5 output frames; sampled outputs against the oracle and the
    whole result against the whole-video call on the device."""
    import direct_implicit_gemm_amd as L
    base = W.ALL_LAYERS["c5_A"]
    layer = base.with_(T=17, pad=(2, 1, 1))
    x, w, b = W.make_inputs(layer, 17)
    note(f"long video x={layer.x_shape} {layer.dtype}, causal, chunks of 5 frames")
    wt = w.torch("cuda")
    wq = L.pack_weights(wt)
    bt = b.torch("cuda")
    xs = torch.empty(x.shape, dtype=torch.float16, pin_memory=True)
    xs.copy_(x.torch("cpu"))
    y = L.conv3d_chunked(xs, wq, bt, 5, (2, 0), layer.stride, 1, layer.act)
    assert not y.is_cuda
    whole = L.conv3d_tpad(xs.cuda(), wq, bt, (2, 0), layer.stride, 1, layer.act)
    torch.cuda.synchronize()
    yd = to_f64(y)
    # every output element agrees with the whole-video call to about one
    # f16 rounding (the kernels may sum in another order); a frame taken from
    # the wrong place would differ by the size of the values themselves
    diff = (y.cuda().float() - whole.float()).abs()
    tol = whole.float().abs() * 2.0 ** -9 + 2.0 ** -12
    assert bool((diff <= tol).all()), float(diff.max())
    rng = np.random.default_rng(9)
    idx = np.unique(np.concatenate([
        rng.integers(0, yd.size, 3000),
        # first and last row and column of every output frame, channel 0
        [np.ravel_multi_index((0, 0, t, r, c), yd.shape)
         for t in range(yd.shape[2]) for r in (0, yd.shape[3] - 1) for c in (0, yd.shape[4] - 1)]]))
    ref, s = oracle.conv_points(x.f64(), w.f64(), b.f64(), idx, layer.stride, layer.pad,
                                relu=layer.act == "relu", pad_t_back=0)
    m = metrics(yd.ravel()[idx], ref, s, layer.dtype)
    note(f"  sampled {m}")
    assert_gates(m, layer.dtype, "long video")


@pytest.mark.parametrize("where", ["host", "device"])
def test_chunked_batch_of_two_no_bias(where):
    """N = 2 (the copies take N * C rows of frames) and no bias."""
    import direct_implicit_gemm_amd as L
    layer = W.Layer("frames", "bf16", 2, 16, 7, 6, 40, 72, 3, 3, 3, (2, 1, 1), (1, 1, 1),
                    "relu", 3, "N01", "N01", "zero")
    x, w, b = W.make_inputs(layer, 813)
    ref, s = oracle.conv(x.f64(), w.f64(), None, layer.stride, layer.pad, relu=True,
                         pad_t_back=0)
    if where == "host":
        xs = torch.empty(x.shape, dtype=torch.bfloat16, pin_memory=True)
        xs.copy_(x.torch("cpu"))
    else:
        xs = x.torch("cuda")
    note(f"chunked N=2 no bias, x on {where}")
    y = L.conv3d_chunked(xs, w.torch("cuda"), None, 3, (2, 0), 1, 1, "relu")
    torch.cuda.synchronize()
    m = metrics(to_f64(y), ref, s, "bf16")
    note(f"  {m}")
    assert_gates(m, "bf16", "chunked N=2")
    # the window call on its own, batch of two
    st_, f0, tw = L.libconv_frame_window(7, 3, 2, 0, 1, 3, 4)
    assert st_ == 0
    yw = L.conv3d_frames(x.torch("cuda")[:, :, f0:f0 + tw].contiguous(), w.torch("cuda"), None,
                         7, (3, 4), (2, 0), 1, 1, "relu")
    torch.cuda.synchronize()
    m = metrics(to_f64(yw), ref[:, :, 3:7], s[:, :, 3:7], "bf16")
    assert_gates(m, "bf16", "frames N=2")
