"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test states what fixes the expected value: a hand-computed fixture, a
closed form, an identity of the definition, an independent brute force, or
torch's fp64 CPU convolution (the same cross-correlation with zero padding).
The definition is the gather-form direct convolution of the page "PP-OCR on
Vulkan compute shaders" (section 2.2); the 3-D form is the Convolution3D
layer of the page "SeedVR2 NCNN Vulkan" (section 3.2).
"""
import itertools
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- fixtures
def _read_all_ones_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "all_ones.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0], "rows": []}
                cases.append(cur)
            elif key == "shape":
                cur["shape"] = [float(v) for v in vals]
            elif key == "row":
                cur["rows"].append([float(v) for v in vals])
    return cases


@pytest.mark.parametrize("case", _read_all_ones_cases(), ids=lambda c: c["name"])
def test_golden_all_ones(case):
    """Hand-computed all-ones results (page 1, section 5.1's checking method)."""
    N, C, H, W, CO, KH, KW, ph, pw, sh, sw = (int(v) for v in case["shape"][:11])
    bias = case["shape"][11]
    x = np.ones((N, C, H, W))
    w = np.ones((CO, C, KH, KW))
    b = np.full(CO, bias)
    y, s = oracle.conv(x, w, b, (sh, sw), (ph, pw))
    expect = np.array(case["rows"])
    assert y.shape == (N, CO) + expect.shape
    for co in range(CO):
        np.testing.assert_array_equal(y[0, co], expect)
    # all operands >= 0 except possibly bias: S = |b| + taps * C_in
    np.testing.assert_array_equal(s[0, 0], expect - bias + abs(bias))


# ------------------------------------------------------------- output size
@pytest.mark.parametrize("n_in,k,p,s,expect", [
    (640, 3, 1, 2, 320), (320, 3, 1, 2, 160), (320, 3, 1, 1, 320), (320, 1, 0, 1, 320),
    (32, 3, 1, 1, 32), (5, 3, 1, 1, 5), (24, 3, 1, 1, 24), (5, 3, 0, 1, 3),
    (7, 3, 0, 3, 2), (4, 5, 0, 1, 0), (1, 1, 0, 1, 1), (2, 5, 1, 1, 0), (3, 5, 1, 1, 1),
])
def test_out_extent_values(n_in, k, p, s, expect):
    """Extents the workloads fix (640 -> 320 -> 160 at k3 s2 p1) and small cases
    counted by hand."""
    assert oracle.out_extent(n_in, k, p, s) == expect


def test_out_extent_closed_form():
    """The walked count equals floor((I + 2p - k)/s) + 1 when the window fits."""
    for n_in, k, p, s in itertools.product(range(1, 12), range(1, 7), range(0, 4), range(1, 5)):
        expect = (n_in + 2 * p - k) // s + 1 if n_in + 2 * p >= k else 0
        assert oracle.out_extent(n_in, k, p, s) == expect


@pytest.mark.parametrize("args", [(0, 3, 1, 1), (5, 0, 1, 1), (5, 3, -1, 1), (5, 3, 1, 0)])
def test_out_extent_rejects(args):
    assert oracle.out_extent(*args) == -1


# ------------------------------------------------------ all-ones closed form
def _taps_in_bounds(n_in, k, p, s, n_out):
    """Closed form: #{kk < k : 0 <= o*s - p + kk < n_in} for each o."""
    o = np.arange(n_out)
    lo = np.maximum(0, p - o * s)
    hi = np.minimum(k, n_in + p - o * s)
    return np.maximum(0, hi - lo)


@pytest.mark.parametrize("dims", [2, 3])
def test_all_ones_closed_form(dims):
    r = _rng(11)
    for _ in range(40):
        C = int(r.integers(1, 5))
        CO = int(r.integers(1, 4))
        sp = [int(r.integers(1, 10)) for _ in range(dims)]
        ks = [int(r.integers(1, 6)) for _ in range(dims)]
        ps = [int(r.integers(0, k + 1)) for k in ks]
        ss = [int(r.integers(1, 4)) for _ in range(dims)]
        if any(i + 2 * p < k for i, p, k in zip(sp, ps, ks)):
            continue
        b = r.integers(-16, 17, CO) / 8.0   # dyadic: every partial sum is exact
        x = np.ones([2, C] + sp)
        w = np.ones([CO, C] + ks)
        y, s = oracle.conv(x, w, b, ss, ps)
        cnt = None
        for d in range(dims):
            n_out = y.shape[2 + d]
            c = _taps_in_bounds(sp[d], ks[d], ps[d], ss[d], n_out)
            cnt = c if cnt is None else np.multiply.outer(cnt, c)
        expect = C * cnt[None, None] + b.reshape([1, CO] + [1] * dims)
        np.testing.assert_array_equal(y, np.broadcast_to(expect, y.shape))
        sexp = C * cnt[None, None] + np.abs(b).reshape([1, CO] + [1] * dims)
        np.testing.assert_array_equal(s, np.broadcast_to(sexp, s.shape))


# ----------------------------------------------------------- delta kernels
@pytest.mark.parametrize("dims,k", [(2, 1), (2, 3), (2, 5), (3, 3), (3, 1)])
def test_delta_kernel_identity(dims, k):
    """Centre delta, stride 1, pad (k-1)/2: y = x + b, channel by channel."""
    r = _rng(12)
    C = 4
    sp = [5, 7, 6][:dims] if dims == 3 else [7, 6]
    x = r.standard_normal([2, C] + sp)
    w = np.zeros([C, C] + [k] * dims)
    for c in range(C):
        w[(c, c) + (k // 2,) * dims] = 1.0
    b = r.uniform(-1, 1, C)
    y, _ = oracle.conv(x, w, b, 1, (k - 1) // 2)
    np.testing.assert_array_equal(y, x + b.reshape([1, C] + [1] * dims))


def test_delta_kernel_shifted_and_channel_swap():
    """Off-centre delta at tap (ky, kx), pad 1, from channel c to (c+1) % C:
    y[co = (c+1)%C][oh][ow] = x[c][oh - 1 + ky][ow - 1 + kx], zero outside."""
    r = _rng(13)
    C, H, W = 3, 6, 7
    x = r.standard_normal((1, C, H, W))
    for ky, kx in itertools.product(range(3), range(3)):
        w = np.zeros((C, C, 3, 3))
        for c in range(C):
            w[(c + 1) % C, c, ky, kx] = 1.0
        y, _ = oracle.conv(x, w, None, 1, 1)
        xp = np.pad(x, ((0, 0), (0, 0), (1, 1), (1, 1)))
        for c in range(C):
            np.testing.assert_array_equal(y[0, (c + 1) % C], xp[0, c, ky:ky + H, kx:kx + W])


def test_delta_kernel_3d_frame_shift():
    """Delta at time tap kt, centre in space, pad 1: a copy of frame t - 1 + kt."""
    r = _rng(14)
    C, T, H, W = 2, 5, 4, 3
    x = r.standard_normal((1, C, T, H, W))
    for kt in range(3):
        w = np.zeros((C, C, 3, 3, 3))
        for c in range(C):
            w[c, c, kt, 1, 1] = 1.0
        y, _ = oracle.conv(x, w, None, 1, 1)
        xp = np.pad(x, ((0, 0), (0, 0), (1, 1), (0, 0), (0, 0)))
        np.testing.assert_array_equal(y, xp[:, :, kt:kt + T])


# ---------------------------------------------------------------- linearity
@pytest.mark.parametrize("dims", [2, 3])
def test_linearity(dims):
    r = _rng(15)
    sp = [6, 9] if dims == 2 else [4, 6, 5]
    x1, x2 = r.standard_normal([2, 3] + sp), r.standard_normal([2, 3] + sp)
    w1, w2 = r.standard_normal([4, 3] + [3] * dims), r.standard_normal([4, 3] + [3] * dims)
    a, bb = 0.75, -1.25
    st, pd = 2, 1
    y_x = oracle.conv(a * x1 + bb * x2, w1, None, st, pd)[0]
    ref_x = a * oracle.conv(x1, w1, None, st, pd)[0] + bb * oracle.conv(x2, w1, None, st, pd)[0]
    np.testing.assert_allclose(y_x, ref_x, rtol=0, atol=1e-12 * np.abs(ref_x).max())
    y_w = oracle.conv(x1, a * w1 + bb * w2, None, st, pd)[0]
    ref_w = a * oracle.conv(x1, w1, None, st, pd)[0] + bb * oracle.conv(x1, w2, None, st, pd)[0]
    np.testing.assert_allclose(y_w, ref_w, rtol=0, atol=1e-12 * np.abs(ref_w).max())


# ------------------------------------------------- brute-force im2col x matmul
def _im2col_conv(x, w, b, stride, pad):
    """Independent reference: zero-pad x, cut every window, one matmul."""
    dims = x.ndim - 2
    N, C = x.shape[:2]
    CO = w.shape[0]
    ks = w.shape[2:]
    xp = np.pad(x, [(0, 0), (0, 0)] + [(p, p) for p in pad])
    outs = [(xp.shape[2 + d] - ks[d]) // stride[d] + 1 for d in range(dims)]
    cols = []
    for o in itertools.product(*[range(n) for n in outs]):
        sl = tuple(slice(o[d] * stride[d], o[d] * stride[d] + ks[d]) for d in range(dims))
        cols.append(xp[(slice(None), slice(None)) + sl].reshape(N, -1))
    cols = np.stack(cols, axis=1)                      # N x P x (C*taps)
    y = cols @ w.reshape(CO, -1).T                     # N x P x CO
    if b is not None:
        y = y + b
    return np.moveaxis(y, 2, 1).reshape([N, CO] + outs)


@pytest.mark.parametrize("dims", [2, 3])
def test_bruteforce_im2col(dims):
    r = _rng(16)
    done = 0
    while done < 60:
        C = int(r.integers(1, 6))
        CO = int(r.integers(1, 5))
        ks = [int(r.choice([1, 2, 3, 5])) for _ in range(dims)]
        ps = [int(r.integers(0, k + 1)) for k in ks]
        ss = [int(r.integers(1, 4)) for _ in range(dims)]
        sp = [int(r.integers(1, 10)) for _ in range(dims)]
        if any(i + 2 * p < k for i, p, k in zip(sp, ps, ks)):
            continue
        x = r.standard_normal([int(r.integers(1, 3)), C] + sp)
        w = r.standard_normal([CO, C] + ks)
        b = r.standard_normal(CO) if r.integers(0, 2) else None
        y, s = oracle.conv(x, w, b, ss, ps)
        ref = _im2col_conv(x, w, b, ss, ps)
        assert y.shape == ref.shape
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
        # S is the same brute force on |x| and |w| (plus |b|)
        sref = _im2col_conv(np.abs(x), np.abs(w), None if b is None else np.abs(b), ss, ps)
        np.testing.assert_allclose(s, sref, rtol=1e-12, atol=1e-12)
        done += 1


# ------------------------------------------------ torch fp64 CPU (library)
@pytest.mark.parametrize("shape", [
    # (dims, N, C, spatial, CO, k, stride, pad, relu)
    (2, 1, 3, (32, 32), 8, 3, 1, 1, False),
    (2, 1, 3, (40, 36), 32, 3, 2, 1, True),
    (2, 2, 32, (20, 18), 16, 3, 1, 1, True),
    (2, 1, 32, (11, 13), 64, 1, 1, 0, True),
    (2, 1, 16, (21, 20), 24, 3, 2, 1, False),
    (2, 3, 8, (9, 10), 5, 5, 1, 2, False),
    (3, 1, 8, (5, 12, 10), 8, 3, 1, 1, False),
    (3, 2, 4, (4, 7, 9), 6, 3, 2, 1, True),
])
def test_torch_fp64(shape):
    dims, N, C, sp, CO, k, st, pd, relu = shape
    r = _rng(17)
    x = r.standard_normal((N, C) + sp)
    w = r.standard_normal((CO, C) + (k,) * dims)
    b = r.standard_normal(CO)
    y, _ = oracle.conv(x, w, b, st, pd, relu=relu)
    f = torch.nn.functional.conv2d if dims == 2 else torch.nn.functional.conv3d
    ref = f(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b), stride=st, padding=pd)
    if relu:
        ref = torch.relu(ref)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- identities
@pytest.mark.parametrize("dims", [2, 3])
def test_stride_subsamples(dims):
    """Stride-s output = stride-1 output taken at every s-th position."""
    r = _rng(18)
    sp = [13, 11] if dims == 2 else [7, 9, 8]
    x = r.standard_normal([1, 3] + sp)
    w = r.standard_normal([2, 3] + [3] * dims)
    y1, _ = oracle.conv(x, w, None, 1, 1)
    for s in (2, 3):
        ys, _ = oracle.conv(x, w, None, s, 1)
        sl = (slice(None), slice(None)) + (slice(None, None, s),) * dims
        np.testing.assert_array_equal(ys, y1[sl])


def test_conv3d_single_frame_is_conv2d():
    r = _rng(19)
    x = r.standard_normal((2, 3, 1, 8, 7))
    w = r.standard_normal((4, 3, 1, 3, 3))
    b = r.standard_normal(4)
    y3, s3 = oracle.conv(x, w, b, (1, 2, 1), (0, 1, 1))
    y2, s2 = oracle.conv(x[:, :, 0], w[:, :, 0], b, (2, 1), (1, 1))
    np.testing.assert_array_equal(y3[:, :, 0], y2)
    np.testing.assert_array_equal(s3[:, :, 0], s2)


def test_conv3d_is_sum_of_conv2d_over_time_taps():
    """y[t] = b + sum_kt conv2d(x[t*s - p + kt], w[:, :, kt]), missing frames = 0."""
    r = _rng(20)
    C, T, CO = 3, 5, 4
    x = r.standard_normal((1, C, T, 6, 5))
    w = r.standard_normal((CO, C, 3, 3, 3))
    b = r.standard_normal(CO)
    for st in (1, 2):
        y3, _ = oracle.conv(x, w, b, (st, 1, 1), 1)
        for t in range(y3.shape[2]):
            acc = np.broadcast_to(b[None, :, None, None], (1, CO, 6, 5)).copy()
            for kt in range(3):
                it = t * st - 1 + kt
                if 0 <= it < T:
                    acc += oracle.conv(x[:, :, it], w[:, :, kt], None, 1, 1)[0]
            np.testing.assert_allclose(y3[:, :, t], acc, rtol=1e-13, atol=1e-13)


def test_pointwise_is_matmul_and_relu_is_max0():
    r = _rng(21)
    x = r.standard_normal((2, 6, 5, 4))
    w = r.standard_normal((7, 6, 1, 1))
    b = r.standard_normal(7)
    y, _ = oracle.conv(x, w, b, 1, 0)
    ref = np.einsum("oc,nchw->nohw", w[:, :, 0, 0], x) + b[None, :, None, None]
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)
    yr, _ = oracle.conv(x, w, b, 1, 0, relu=True)
    np.testing.assert_array_equal(yr, np.maximum(y, 0.0))


def test_magnitude_sum_properties():
    """S >= |y| (no activation); S is even in x; S == y for non-negative data."""
    r = _rng(22)
    x = r.standard_normal((1, 4, 7, 6))
    w = r.standard_normal((3, 4, 3, 3))
    b = r.standard_normal(3)
    y, s = oracle.conv(x, w, b, 1, 1)
    assert np.all(s >= np.abs(y) - 1e-12)
    _, s_neg = oracle.conv(-x, w, b, 1, 1)
    np.testing.assert_array_equal(s, s_neg)
    yp, sp = oracle.conv(np.abs(x), np.abs(w), np.abs(b), 1, 1)
    np.testing.assert_allclose(sp, yp, rtol=1e-14, atol=0)


# --------------------------------------------------------- sampled outputs
@pytest.mark.parametrize("dims", [2, 3])
def test_points_match_torch(dims):
    """The sampled-output entry point agrees with torch at the same indices."""
    r = _rng(23)
    sp = (17, 19) if dims == 2 else (4, 9, 11)
    x = r.standard_normal((2, 5) + sp)
    w = r.standard_normal((6, 5) + (3,) * dims)
    b = r.standard_normal(6)
    f = torch.nn.functional.conv2d if dims == 2 else torch.nn.functional.conv3d
    ref = torch.relu(f(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b),
                       stride=2, padding=1)).numpy().ravel()
    idx = r.choice(ref.size, 200, replace=False)
    idx = np.concatenate([idx, [0, ref.size - 1]])
    y, _ = oracle.conv_points(x, w, b, idx, 2, 1, relu=True)
    np.testing.assert_allclose(y, ref[idx], rtol=1e-12, atol=1e-12)


def test_points_rejects_out_of_range():
    x = np.ones((1, 1, 4, 4))
    w = np.ones((1, 1, 3, 3))
    with pytest.raises(ValueError):
        oracle.conv_points(x, w, None, [16], 1, 1)


def test_thread_count_does_not_change_result():
    r = _rng(24)
    x = r.standard_normal((1, 8, 12, 12))
    w = r.standard_normal((8, 8, 3, 3))
    y1, s1 = oracle.conv(x, w, None, 1, 1, nthreads=1)
    y4, s4 = oracle.conv(x, w, None, 1, 1, nthreads=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(s1, s4)


# ------------------------------------------- padding only before / after in time
# The causal 3-D convolution of the spatio-temporal VAE ("SeedVR2 NCNN Vulkan",
# section 7.2) pads the frame axis on one side only (the page builds it from
# Concat/Crop around a plain Convolution3D).


def test_out_extent2_closed_form():
    """Walked count against floor((in + lo + hi - k) / s) + 1."""
    for n_in, k, lo, hi, s in itertools.product(range(1, 12), range(1, 6), range(0, 4),
                                               range(0, 4), range(1, 4)):
        span = n_in + lo + hi - k
        want = span // s + 1 if span >= 0 else 0
        assert oracle.out_extent2(n_in, k, lo, hi, s) == want, (n_in, k, lo, hi, s)
        if lo == hi:
            assert oracle.out_extent2(n_in, k, lo, hi, s) == oracle.out_extent(n_in, k, lo, s)


@pytest.mark.parametrize("dims", [
    # N, C, T, H, W, CO, KT, KH, KW, pf, pb, ph, pw, st, sh, sw
    (1, 2, 5, 4, 6, 3, 3, 3, 3, 2, 0, 1, 1, 1, 1, 1),
    (2, 3, 4, 5, 3, 2, 2, 1, 3, 1, 0, 0, 1, 1, 1, 1),
    (1, 1, 7, 3, 3, 2, 3, 3, 3, 0, 2, 1, 1, 2, 1, 1),
    (1, 2, 6, 4, 4, 1, 3, 2, 2, 3, 1, 1, 0, 2, 2, 1),
])
def test_all_ones_closed_form_time_pads(dims):
    """x = w = 1: y = C * cnt_t(ot) * cnt_h(oh) * cnt_w(ow) + b, with cnt_t
    counting the taps kt whose frame ot*st - pf + kt lies in [0, T)."""
    N, C, T, H, W, CO, KT, KH, KW, pf, pb, ph, pw, st, sh, sw = dims
    b = np.arange(CO) * 0.25 - 0.5
    y, s = oracle.conv(np.ones((N, C, T, H, W)), np.ones((CO, C, KT, KH, KW)), b,
                       (st, sh, sw), (pf, ph, pw), pad_t_back=pb)
    OT = (T + pf + pb - KT) // st + 1
    OH = (H + 2 * ph - KH) // sh + 1
    OW = (W + 2 * pw - KW) // sw + 1
    assert y.shape == (N, CO, OT, OH, OW)

    def cnt(o, s_, p_, k, n):
        return sum(1 for t in range(k) if 0 <= o * s_ - p_ + t < n)

    for ot, oh, ow in itertools.product(range(OT), range(OH), range(OW)):
        taps = C * cnt(ot, st, pf, KT, T) * cnt(oh, sh, ph, KH, H) * cnt(ow, sw, pw, KW, W)
        np.testing.assert_array_equal(y[0, :, ot, oh, ow], taps + b)
        np.testing.assert_array_equal(s[0, :, ot, oh, ow], taps + np.abs(b))


@pytest.mark.parametrize("dims", [
    (1, 3, 5, 6, 7, 4, 3, 3, 3, 2, 0, 1, 1, 1, 1, 1),
    (2, 2, 6, 5, 5, 3, 3, 3, 3, 1, 2, 1, 1, 2, 1, 2),
    (1, 4, 4, 4, 6, 2, 2, 3, 1, 0, 1, 1, 0, 1, 2, 1),
])
def test_time_pads_match_torch_explicit_padding(dims):
    """Padding (pf, pb) in time = torch's fp64 conv3d of the input with pf
    zero frames concatenated before it and pb after it (the Concat of the page)."""
    N, C, T, H, W, CO, KT, KH, KW, pf, pb, ph, pw, st, sh, sw = dims
    r = _rng(77)
    x = r.standard_normal((N, C, T, H, W))
    w = r.standard_normal((CO, C, KT, KH, KW))
    b = r.standard_normal(CO)
    y, _ = oracle.conv(x, w, b, (st, sh, sw), (pf, ph, pw), pad_t_back=pb)
    xt = torch.nn.functional.pad(torch.from_numpy(x), (0, 0, 0, 0, pf, pb))
    ref = torch.nn.functional.conv3d(xt, torch.from_numpy(w), torch.from_numpy(b),
                                     stride=(st, sh, sw), padding=(0, ph, pw)).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_causal_is_symmetric_cropped():
    """Causal padding (KT-1 frames before, none after, stride 1) keeps the
    first T frames of the symmetric KT-1 padding (the Crop of the page)."""
    r = _rng(78)
    N, C, T, H, W, CO, KT = 1, 3, 5, 6, 4, 2, 3
    x = r.standard_normal((N, C, T, H, W))
    w = r.standard_normal((CO, C, KT, 3, 3))
    y, _ = oracle.conv(x, w, None, 1, (KT - 1, 1, 1), pad_t_back=0)
    full = torch.nn.functional.conv3d(torch.from_numpy(x), torch.from_numpy(w),
                                      padding=(KT - 1, 1, 1)).numpy()
    assert y.shape[2] == T
    np.testing.assert_allclose(y, full[:, :, :T], rtol=1e-12, atol=1e-12)
    # output frame t sees input frames t-KT+1 .. t only: changing frame T-1
    # changes only the last output frame
    x2 = x.copy()
    x2[:, :, T - 1] += 1.0
    y2, _ = oracle.conv(x2, w, None, 1, (KT - 1, 1, 1), pad_t_back=0)
    np.testing.assert_array_equal(y2[:, :, :T - 1], y[:, :, :T - 1])
    assert np.abs(y2[:, :, T - 1] - y[:, :, T - 1]).max() > 0


def test_time_pads_points_match_full():
    r = _rng(79)
    x = r.standard_normal((1, 2, 6, 5, 5))
    w = r.standard_normal((3, 2, 3, 3, 3))
    y, s = oracle.conv(x, w, None, (2, 1, 1), (2, 1, 1), pad_t_back=0)
    idx = r.choice(y.size, 40, replace=False)
    yp, sp = oracle.conv_points(x, w, None, idx, (2, 1, 1), (2, 1, 1), pad_t_back=0)
    np.testing.assert_array_equal(yp, y.reshape(-1)[idx])
    np.testing.assert_array_equal(sp, s.reshape(-1)[idx])


# ----------------------------------------- batch normalisation folded into the conv
def test_fold_batchnorm_matches_torch_batch_norm_after_conv():
    """conv(x, w_f) + b_f = BN(conv(x, w) + b) with BN in inference form,
    evaluated by torch's fp64 batch_norm (not the folding formula)."""
    r = _rng(90)
    x = r.standard_normal((2, 5, 9, 11))
    w = r.standard_normal((6, 5, 3, 3))
    b = r.standard_normal(6)
    gamma, beta = r.uniform(0.5, 2.0, 6), r.standard_normal(6)
    mean, var, eps = r.standard_normal(6), r.uniform(0.1, 3.0, 6), 1e-5
    wf, bf = oracle.fold_batchnorm(w, b, gamma, beta, mean, var, eps)
    y_fold, _ = oracle.conv(x, wf, bf, 1, 1)
    conv = torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(w),
                                      torch.from_numpy(b), padding=1)
    ref = torch.nn.functional.batch_norm(conv, torch.from_numpy(mean), torch.from_numpy(var),
                                         torch.from_numpy(gamma), torch.from_numpy(beta),
                                         training=False, eps=eps).numpy()
    np.testing.assert_allclose(y_fold, ref, rtol=1e-12, atol=1e-12)


def test_fold_batchnorm_identity_and_no_bias():
    """gamma = sqrt(var + eps), beta = mean: the fold leaves w and b unchanged;
    a missing conv bias is a zero bias."""
    r = _rng(91)
    w = r.standard_normal((4, 3, 1, 3, 3))
    b = r.standard_normal(4)
    var, eps = r.uniform(0.5, 2.0, 4), 1e-3
    mean = r.standard_normal(4)
    wf, bf = oracle.fold_batchnorm(w, b, np.sqrt(var + eps), mean, mean, var, eps)
    np.testing.assert_allclose(wf, w, rtol=1e-15)
    np.testing.assert_allclose(bf, b, rtol=1e-14, atol=1e-14)
    g, be = r.uniform(0.5, 2, 4), r.standard_normal(4)
    w0, b0 = oracle.fold_batchnorm(w, None, g, be, mean, var, eps)
    w1, b1 = oracle.fold_batchnorm(w, np.zeros(4), g, be, mean, var, eps)
    np.testing.assert_array_equal(w0, w1)
    np.testing.assert_array_equal(b0, b1)


def test_max_pool2x2_matches_torch():
    """The pooling after conv + activation against torch's max_pool2d (2x2,
    stride 2, floor), on even and odd extents."""
    r = _rng(95)
    for shape in [(2, 3, 8, 10), (1, 4, 7, 9), (1, 1, 2, 3)]:
        y = r.standard_normal(shape)
        ref = torch.nn.functional.max_pool2d(torch.from_numpy(y), 2, 2).numpy()
        np.testing.assert_array_equal(oracle.max_pool2x2(y), ref)


def test_pack_channels_matches_torch_reshape():
    """Channel packing against torch's route (zero-pad the channel axis, split
    it into groups, move the in-group index last), 2-D and 3-D, with and
    without a partial last group."""
    r = _rng(96)
    for shape, g in [((2, 8, 3, 5), 8), ((1, 13, 4, 6), 8), ((1, 6, 2, 3, 4), 4), ((2, 3, 5, 7), 4)]:
        x = r.standard_normal(shape)
        c = shape[1]
        gs = -(-c // g)
        t = torch.nn.functional.pad(torch.from_numpy(x).movedim(1, -1), (0, gs * g - c))
        t = t.reshape(t.shape[:-1] + (gs, g)).movedim(-2, 1)
        np.testing.assert_array_equal(oracle.pack_channels(x, g), t.numpy())


def test_pack_channels_index_rule_and_roundtrip():
    """Element [n][c // g][h][w][c % g] holds x[n][c][h][w]: an iota tensor
    shows every element in its place; the pad channels are zero; unpacking
    returns x."""
    x = np.arange(2 * 11 * 3 * 4, dtype=np.float64).reshape(2, 11, 3, 4)
    p = oracle.pack_channels(x, 8)
    assert p.shape == (2, 2, 3, 4, 8)
    for n, c, h, w in itertools.product(range(2), range(11), range(3), range(4)):
        assert p[n, c // 8, h, w, c % 8] == x[n, c, h, w]
    assert not p[:, 1, :, :, 3:].any()
    np.testing.assert_array_equal(oracle.unpack_channels(p, 11), x)
