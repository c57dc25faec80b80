"""Frame windows of a long video (host logic, no GPU): which input frames a
range of output frames reads, the chunked driver's workspace size, and the
argument errors the window and chunked calls return before touching a
device.

The window is pinned to the oracle's convolution itself: an input frame
belongs to the window of a range of output frames exactly when changing it
changes one of those outputs (one-hot frames through the fp64 oracle)."""
import ctypes
import itertools

import numpy as np
import pytest

import direct_implicit_gemm_amd as L
import oracle


def _dependency(T, KT, pf, pb, st):
    """dep[o] = input frames output frame o depends on, by the oracle."""
    ot = oracle.out_extent2(T, KT, pf, pb, st)
    w = np.ones((1, 1, KT, 1, 1))
    dep = [set() for _ in range(ot)]
    for f in range(T):
        x = np.zeros((1, 1, T, 1, 1))
        x[0, 0, f] = 1.0
        y, _ = oracle.conv(x, w, None, (st, 1, 1), (pf, 0, 0), pad_t_back=pb)
        for o in np.nonzero(y[0, 0, :, 0, 0])[0]:
            dep[o].add(f)
    return dep


GEOMS = [(T, KT, pf, pb, st)
         for T, KT, st in itertools.product((1, 2, 5, 9), (1, 2, 3), (1, 2, 3))
         for pf, pb in ((0, 0), (KT - 1, 0), (1, 1), (0, KT - 1), (KT + 1, 0), (2, 3))
         if oracle.out_extent2(T, KT, pf, pb, st) >= 1]


@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: "T%d_k%d_p%d%d_s%d" % g)
def test_frame_window_matches_oracle_dependency(geom):
    T, KT, pf, pb, st = geom
    dep = _dependency(T, KT, pf, pb, st)
    ot = len(dep)
    for o0 in range(ot):
        for on in range(1, ot - o0 + 1):
            frames = set().union(*dep[o0:o0 + on])
            status, f0, tw = L.libconv_frame_window(T, KT, pf, pb, st, o0, on)
            if not frames:   # those outputs read padding only
                assert status == 2, (o0, on)
                continue
            assert status == 0, (o0, on)
            assert (f0, tw) == (min(frames), max(frames) - min(frames) + 1), (o0, on, frames)
            # every frame in between is read by some output of the range
            # unless the time stride skips it
            if st <= KT:
                assert frames == set(range(f0, f0 + tw))


def test_frame_window_errors():
    lib = L.load()
    f0, tw = ctypes.c_int(), ctypes.c_int()
    assert lib.libconv_frame_window(5, 3, 1, 1, 1, 0, 1, None, ctypes.byref(tw)) == 1
    assert lib.libconv_frame_window(5, 3, 1, 1, 1, 0, 1, ctypes.byref(f0), None) == 1
    for args in [(5, 3, 1, 1, 1, -1, 1), (5, 3, 1, 1, 1, 0, 0), (5, 3, 1, 1, 1, 4, 2),
                 (5, 3, 1, 1, 1, 5, 1), (5, 3, -1, 1, 1, 0, 1), (2, 3, 0, 0, 1, 0, 1),
                 (5, 3, 1, 1, 0, 0, 1)]:
        assert L.libconv_frame_window(*args)[0] == 2, args


def _ws_expected(N, C, T, H, W, K, KT, KH, KW, pf, pb, ph, pw, st, sh, sw, chunk, eb):
    ot = oracle.out_extent2(T, KT, pf, pb, st)
    oh = oracle.out_extent(H, KH, ph, sh)
    ow = oracle.out_extent(W, KW, pw, sw)
    chunk = min(chunk, ot)
    tw_max = 0
    for o0 in range(0, ot, chunk):
        on = min(chunk, ot - o0)
        lo = max(0, o0 * st - pf)
        hi = min(T, (o0 + on - 1) * st - pf + KT)
        tw_max = max(tw_max, hi - lo)
    r = lambda v: -(-v // 256) * 256
    # room for the weights packed once (the packed layout of libconv.h: groups
    # of 16 bytes of input channels, output channels padded to 128), for the
    # kernel sizes the packed kernels take
    taps = KT * KH * KW
    packed = (-(-C // (16 // eb)) * taps * (-(-K // 128) * 128) * 16) if taps in (1, 9, 27) else 0
    return 2 * (r(N * C * tw_max * H * W * eb) + r(N * K * chunk * oh * ow * eb)) + r(packed)


@pytest.mark.parametrize("case", [
    # N, C, T, H, W, K, KT, KH, KW, pf, pb, ph, pw, st, sh, sw, chunk, dtype
    (1, 128, 17, 256, 480, 128, 3, 3, 3, 2, 0, 1, 1, 1, 1, 1, 5, L.F16),
    (2, 16, 9, 10, 12, 8, 3, 3, 3, 1, 1, 1, 1, 2, 1, 1, 2, L.BF16),
    (1, 3, 4, 7, 7, 5, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 10, L.F32),
    (1, 8, 33, 6, 6, 8, 3, 3, 3, 2, 0, 1, 1, 1, 2, 2, 17, L.F32),
])
def test_chunked_workspace_bytes(case):
    *shape, dt = case
    eb = 4 if dt == L.F32 else 2
    assert L.libconv_chunked_workspace_bytes(*shape, dt) == _ws_expected(*shape, eb)


def test_chunked_workspace_rejects():
    base = [1, 8, 9, 6, 6, 8, 3, 3, 3, 2, 0, 1, 1, 1, 1, 1, 4, L.F16]
    assert L.libconv_chunked_workspace_bytes(*base) > 0
    for i, v in [(9, 3), (10, 3), (9, -1), (16, 0), (17, 7), (2, 0)]:
        a = list(base)
        a[i] = v
        assert L.libconv_chunked_workspace_bytes(*a) == -1, (i, v)


def test_frames_and_chunked_errors_without_gpu():
    """Rejected before any device access (this host has none: a valid call
    reaches the device check and reports it)."""
    fake = 1 << 40
    y = fake + (1 << 32)
    geo = (1, 8, 9, 6, 6, 8, 3, 3, 3, 2, 0, 1, 1, 1, 1, 1)
    # frames: both or neither weight form; an out-of-range output window
    assert L.conv3d_forward_frames(fake, fake, fake, None, y, *geo, 0, 2, L.F16, 0, None) == 1
    assert L.conv3d_forward_frames(fake, None, None, None, y, *geo, 0, 2, L.F16, 0, None) == 1
    assert L.conv3d_forward_frames(fake, fake, None, None, y, *geo, 8, 2, L.F16, 0, None) == 2
    assert L.conv3d_forward_frames(fake, fake, None, None, y, *geo, 0, 2, 7, 0, None) == 3
    assert L.conv3d_forward_frames(fake, fake, None, None, y, *geo, 0, 2, L.F16, 0, None) == 7
    ws = fake + (1 << 34)
    need = L.libconv_chunked_workspace_bytes(*geo, 4, L.F16)
    call = lambda w, pw, chunk, wsb, act=0, x=fake: L.conv3d_forward_chunked(
        x, w, pw, None, y, *geo, chunk, ws, wsb, L.F16, act, None, None, None)
    assert call(fake, fake, 4, need) == 1
    assert call(None, None, 4, need) == 1
    assert call(fake, None, 0, need) == 2
    assert call(fake, None, 4, need - 1) == 2
    assert call(fake, None, 4, need, act=5) == 4
    assert call(fake, None, 4, need, x=None) == 1
    assert call(fake, None, 4, need, x=y) == 5        # x overlaps y
    assert call(fake, None, 4, need) == 7
