"""Host-side checks of the libconv C ABI that need no GPU: the library loads
and exports every function its header declares, the output-extent rule, the
status strings, argument validation (which returns before any launch), and
the dispatcher's choices."""
import itertools

import numpy as np
import pytest

import direct_implicit_gemm_amd as L
import oracle
import workloads as W


def test_library_loads_and_exports_header_symbols():
    lib = L.load()
    names = L.header_functions()
    assert {"conv2d_forward", "conv3d_forward", "libconv_forward_algo", "libconv_query_algo",
            "libconv_out_size", "libconv_status_string", "libconv_device_supported",
            "libconv_tile_name", "libconv_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_out_size_matches_oracle_extent():
    """The library's closed form against the oracle's walked count."""
    for n_in, k, p, s in itertools.product(range(1, 14), range(1, 8), range(0, 4), range(1, 5)):
        want = oracle.out_extent(n_in, k, p, s)
        got = L.libconv_out_size(n_in, k, p, s)
        assert got == (want if want >= 1 else -1), (n_in, k, p, s)
    for args in [(0, 3, 1, 1), (5, 0, 1, 1), (5, 3, -1, 1), (5, 3, 1, 0)]:
        assert L.libconv_out_size(*args) == -1


def test_status_strings():
    for code in range(11):
        assert L.libconv_status_string(code)
    assert L.libconv_status_string(12345) == "unknown status"


# A valid 2-D argument set (pointers are fake, non-null, non-overlapping:
# validation never dereferences them and returns before any launch).
X, Wp, B, Y = 0x10000000, 0x20000000, 0x30000000, 0x40000000
GOOD2 = dict(N=1, C_in=4, H=8, W=8, C_out=8, KH=3, KW=3, pad_h=1, pad_w=1, stride_h=1,
             stride_w=1, dtype=L.F32, act=L.ACT_NONE)


def call2(x=X, w=Wp, b=B, y=Y, **kw):
    a = dict(GOOD2)
    a.update(kw)
    return L.conv2d_forward(x, w, b, y, a["N"], a["C_in"], a["H"], a["W"], a["C_out"], a["KH"],
                            a["KW"], a["pad_h"], a["pad_w"], a["stride_h"], a["stride_w"],
                            a["dtype"], a["act"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(w=None), 1), (dict(y=None), 1),
    (dict(C_in=0), 2), (dict(H=0), 2), (dict(C_out=0), 2), (dict(KH=0), 2), (dict(N=-1), 2),
    (dict(stride_h=0), 2), (dict(pad_w=-1), 2), (dict(H=2, KH=5, pad_h=0), 2),
    (dict(dtype=7), 3), (dict(dtype=-1), 3), (dict(act=2), 4), (dict(act=-3), 4),
    (dict(y=X + 16), 5), (dict(y=Wp - 64), 5), (dict(b=Y + 4), 5),
    (dict(H=70000, W=70000), 10),
])
def test_validation_errors(kw, code):
    assert call2(**kw) == code


def test_bad_algo():
    st = L.libconv_forward_algo(X, Wp, B, Y, 1, 4, 1, 8, 8, 8, 1, 3, 3, 0, 1, 1, 1, 1, 1,
                                L.F32, 0, 3, None)
    assert st == 9


def test_null_bias_is_allowed_and_empty_batch_is_a_no_op():
    # N = 0 returns OK without touching the device (works with no GPU)
    assert call2(b=None, N=0) == 0


def test_no_device_is_reported():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call2() == 7
    assert L.libconv_device_supported(0) == 7


def test_query_algo_validation():
    st, *_ = L.libconv_query_algo(1, 4, 1, 8, 8, 8, 1, 3, 3, 0, 1, 1, 1, 1, 1, 5, 0, 0)
    assert st == 3


EXPECTED_ALGO = {  # the dispatcher's choice per workload layer
    "c1": L.ALGO_DIRECT, "c2_L1": L.ALGO_DIRECT, "c2_L2": L.ALGO_IGEMM,
    "c2_L3": L.ALGO_IGEMM, "c2_L4": L.ALGO_IGEMM, "c3_A": L.ALGO_IGEMM,
    "c3_B": L.ALGO_IGEMM, "c4_A": L.ALGO_IGEMM, "c4_B": L.ALGO_IGEMM,
    "c5_A": L.ALGO_IGEMM, "c5_B": L.ALGO_IGEMM,
}


@pytest.mark.parametrize("name", sorted(W.ALL_LAYERS))
def test_dispatch_choice(name):
    l = W.ALL_LAYERS[name]
    st, algo, tile, grid = L.libconv_query_algo(
        l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH, l.KW, *l.pad, *l.stride,
        W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act], L.ALGO_AUTO)
    assert st == 0
    assert algo == EXPECTED_ALGO[name]
    assert L.libconv_tile_name(tile) != "?"
    assert grid >= 1


def test_forced_algorithms():
    # 3x3 stride-1 fp32 with C_in = 32: both families can run it
    args = (1, 32, 1, 20, 20, 32, 1, 3, 3, 0, 1, 1, 1, 1, 1, L.F32, 0)
    assert L.libconv_query_algo(*args, L.ALGO_DIRECT)[1] == L.ALGO_DIRECT
    assert L.libconv_query_algo(*args, L.ALGO_IGEMM)[1] == L.ALGO_IGEMM
    # 5x5: the MFMA family has no tile -> UNSUPPORTED when forced, direct otherwise
    args5 = (1, 32, 1, 20, 20, 32, 1, 5, 5, 0, 2, 2, 1, 1, 1, L.F16, 0)
    assert L.libconv_query_algo(*args5, L.ALGO_IGEMM)[0] == 6
    assert L.libconv_query_algo(*args5, L.ALGO_AUTO)[1] == L.ALGO_DIRECT
    # fp16 with C_in not a multiple of 8: only the packed-weight MFMA tiles
    # (whose channel groups are zero-padded) or the direct kernel can run it
    args7 = (1, 12, 1, 20, 20, 32, 1, 3, 3, 0, 1, 1, 1, 1, 1, L.F16, 0)
    st, algo, tile, _ = L.libconv_query_algo(*args7, L.ALGO_AUTO)
    assert st == 0
    assert algo == L.ALGO_DIRECT or L.libconv_tile_name(tile).startswith("igemm16p_")
    # a pointwise layer with 16 input channels: too short a reduction for MFMA
    args1 = (1, 16, 1, 64, 64, 64, 1, 1, 1, 0, 0, 0, 1, 1, 1, L.F32, 0)
    assert L.libconv_query_algo(*args1, L.ALGO_AUTO)[1] == L.ALGO_DIRECT


def test_packed_weight_bytes():
    # [round_up(K,128)/64][ceil(C/g)][taps][64][g] x 16 bytes
    assert L.libconv_packed_weight_bytes(128, 128, 3, 3, 3, L.F16) == 16 * 27 * 128 * 16
    assert L.libconv_packed_weight_bytes(12, 200, 1, 3, 3, L.BF16) == 2 * 9 * 256 * 16
    assert L.libconv_packed_weight_bytes(6, 5, 1, 1, 1, L.F32) == 2 * 1 * 128 * 16
    assert L.libconv_packed_weight_bytes(8, 8, 1, 5, 5, L.F16) == -1      # no packed kernels
    assert L.libconv_packed_weight_bytes(0, 8, 1, 3, 3, L.F16) == -1
    assert L.libconv_packed_weight_bytes(8, 8, 1, 3, 3, 9) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(w=None), 1), (dict(packed=None), 1), (dict(dtype=5), 3), (dict(C_in=0), 2),
    (dict(packed_bytes=100), 2), (dict(KH=5, KW=5), 6), (dict(packed=X + 64), 5),
])
def test_pack_weights_validation(kw, code):
    a = dict(w=X, packed=Y, packed_bytes=1 << 22, C_in=16, C_out=32, KT=1, KH=3, KW=3,
             dtype=L.F16)
    a.update(kw)
    st = L.libconv_pack_weights(a["w"], a["packed"], a["packed_bytes"], a["C_in"], a["C_out"],
                                a["KT"], a["KH"], a["KW"], a["dtype"], None)
    assert st == code


def test_forward_packed_validation():
    # null packed pointer; bad dtype; 16-bit 3-D layer on the CPU host: no device
    assert L.libconv_forward_packed(X, None, None, Y, 1, 8, 3, 8, 8, 8, 3, 3, 3, 1, 1, 1, 1, 1,
                                    1, L.F16, 0, None) == 1
    assert L.libconv_forward_packed(X, Wp, None, Y, 1, 8, 3, 8, 8, 8, 3, 3, 3, 1, 1, 1, 1, 1, 1,
                                    4, 0, None) == 3


def _layer_args(name):
    l = W.ALL_LAYERS[name]
    return (l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH, l.KW, *l.pad, *l.stride,
            W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act], L.ALGO_AUTO)


def _ws_size(name, flags=0):
    l = W.ALL_LAYERS[name]
    return L.libconv_workspace_size(l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH, l.KW,
                                    l.pad[0], l.pad[0], l.pad[1], l.pad[2], *l.stride,
                                    W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act], L.ALGO_AUTO, flags)


def test_3d_layers_dispatch_to_mfma_tiles_with_and_without_workspace():
    """conv3d_forward (no workspace) runs the video-VAE layers on the MFMA
    tiles that read OIDHW weights; given the workspace libconv_workspace_size
    names, on the tiles that read weights packed into it."""
    for name in ("c5_A", "c5_B"):
        args = _layer_args(name)
        st, algo, tile, grid = L.libconv_query_algo(*args)
        assert st == 0 and algo == L.ALGO_IGEMM
        assert L.libconv_tile_name(tile).startswith("igemm16_k333"), L.libconv_tile_name(tile)
        ws = _ws_size(name)
        assert ws > 0
        st, algo, tile, grid, ks = L.libconv_query_plan(*args, 0, ws)
        assert st == 0 and L.libconv_tile_name(tile).startswith("igemm16p_k333")


WIDE_LAYERS = ("c3_A", "c4_A", "c4_B", "c5_A", "c5_B")


@pytest.mark.parametrize("cpack", [False, True])
@pytest.mark.parametrize("name", WIDE_LAYERS)
def test_wide_layers_stay_on_the_matrix_cores_without_a_workspace(name, cpack):
    """Without a workspace (so with OI(D)HW weights and no split) every
    wide workload layer still plans an MFMA tile, in the plain layout and in
    the channel-packed one: the tiles that transpose the weights in
    registers, never the vector-ALU kernel."""
    flags = L.PLAN_CPACK if cpack else 0
    st, algo, tile, grid, ks = L.libconv_query_plan(*_layer_args(name), flags, 0)
    nm = L.libconv_tile_name(tile)
    assert st == 0 and algo == L.ALGO_IGEMM and ks == 1, (name, cpack, nm)
    assert nm.startswith(("igemm16xo_",) if cpack else ("igemm16_",)), (name, cpack, nm)


def test_tile_occupancy_query_without_gpu():
    """The cost model's occupancy column is a host query; unknown ids and
    dtypes a tile does not run give -1."""
    for tid in range(200, 300):
        name = L.libconv_tile_name(tid)
        if name == "?":
            assert L.libconv_tile_occupancy(tid, 0, 0) == -1
            continue
        wide = name.startswith("igemm16")
        for dt in (0, 1, 2):
            occ = L.libconv_tile_occupancy(tid, dt, 0)
            if (dt == 0) == (not wide):
                assert 1 <= occ <= 8, (name, dt, occ)
            else:
                assert occ == -1, (name, dt, occ)


CONFIG_LAYERS = ("c1", "c2_L1", "c2_L2", "c2_L3", "c2_L4", "c3_A", "c3_B", "c4_A", "c4_B",
                 "c5_A", "c5_B")


@pytest.mark.parametrize("name", CONFIG_LAYERS)
def test_query_plan_does_not_depend_on_capture(name):
    """A call plans the same kernel, grid and split whether or not its stream
    is being captured into a graph, with no workspace and with the one
    libconv_workspace_size names; the no-workspace plan agrees with
    libconv_query_algo and neither packs weights nor splits."""
    args = _layer_args(name)
    ws = _ws_size(name)
    assert ws >= 0
    for wsb in (0, ws):
        eager = L.libconv_query_plan(*args, 0, wsb)
        captured = L.libconv_query_plan(*args, L.PLAN_CAPTURING, wsb)
        assert eager[0] == 0 and eager == captured, (name, wsb, eager, captured)
    st, algo, tile, grid, ks = L.libconv_query_plan(*args, 0, 0)
    assert L.libconv_query_algo(*args)[1:] == (algo, tile, grid)
    assert ks == 1
    nm = L.libconv_tile_name(tile)
    assert "16p" not in nm and "32p" not in nm, (name, nm)
    # the best plan fits exactly the workspace it asked for, and more changes nothing
    assert L.libconv_query_plan(*args, 0, ws) == L.libconv_query_plan(*args, 0, ws + (1 << 30))


def test_workspace_enables_split_and_packing():
    """The UNet 1280-channel layer (few tiles for the CUs) splits its reduction
    when given a workspace; the partial sums and the packed weights are what
    the workspace holds."""
    args = _layer_args("c4_B")
    ws = _ws_size("c4_B")
    st, algo, tile, grid, ks = L.libconv_query_plan(*args, 0, ws)
    assert st == 0 and ks > 1
    l = W.ALL_LAYERS["c4_B"]
    partials = ks * l.N * l.C_out * l.H * l.W * 4
    packed = L.libconv_packed_weight_bytes(l.C_in, l.C_out, 1, 3, 3, L.BF16)
    want = (-(-packed // 256) * 256 if "16p" in L.libconv_tile_name(tile) else 0) \
        + -(-partials // 256) * 256
    assert ws == want
    # a workspace too small for the split: the best plan that fits
    st2, _, tile2, _, ks2 = L.libconv_query_plan(*args, 0, ws - 256)
    assert st2 == 0 and (ks2, tile2) != (ks, tile)
    out = L.libconv_query_plan(1, 4, 1, 8, 8, 8, 1, 3, 3, 0, 1, 1, 1, 1, 1, 5, 0, 0, 0, 0)
    assert out[0] == 3  # bad dtype
    assert L.libconv_query_plan(*args, 0, -1)[0] == 2
    assert L.libconv_workspace_size(1, 4, 1, 8, 8, 8, 1, 3, 3, 0, 0, 1, 1, 1, 1, 1, 5, 0, 0,
                                    0) == -1
    # layers that need nothing (the vector-ALU stem) ask for nothing
    assert _ws_size("c2_L1") == 0


def test_workspace_argument_errors_without_gpu():
    """Workspace checks come before any device access: a workspace that is not
    256-byte aligned, that overlaps an operand, or a negative size."""
    fake = 1 << 40
    y = fake + (1 << 32)
    ws = fake + (1 << 34)
    geo = (1, 16, 5, 8, 32, 24, 3, 3, 3, 1, 1, 1, 1, 1, 1, 1)
    ex = lambda x, w, pw, yy, wsp, wsb, flags=0: L.libconv_forward_ex(
        x, w, pw, None, yy, 1, 16, 5, 8, 32, 24, 3, 3, 3, 1, 1, 1, 1, 1, 1, 1, L.F16, 0,
        L.ALGO_AUTO, flags, wsp, wsb, None)
    assert ex(fake, fake + 64, None, y, ws + 16, 1 << 20) == 12
    assert ex(fake, fake + 64, None, y, y, 1 << 20) == 5
    assert ex(fake, fake + 64, None, y, ws, -5) == 2
    assert ex(fake, fake + 64, fake + 64, y, ws, 1 << 20) == 1
    assert ex(fake, fake + 64, None, y, ws, 1 << 20) == 7  # valid: reaches the device check
    assert ex(fake, fake + 64, None, y, None, 0) == 7
    assert L.conv3d_forward_ws(fake, fake + 64, None, y, *geo[:6], 3, 3, 3, 1, 1, 1, 1, 1, 1,
                               L.F16, 0, ws + 8, 1 << 20, None) == 12
    assert L.conv2d_forward_ws(fake, fake + 64, None, y, 1, 16, 8, 32, 24, 3, 3, 1, 1, 1, 1,
                               L.F16, 0, ws, 1 << 20, None) == 7


def test_out_size2_matches_oracle():
    for n_in, k, lo, hi, s in itertools.product(range(1, 10), range(1, 5), range(0, 3),
                                               range(0, 3), range(1, 4)):
        want = oracle.out_extent2(n_in, k, lo, hi, s)
        assert L.libconv_out_size2(n_in, k, lo, hi, s) == (want if want >= 1 else -1)
    assert L.libconv_out_size2(5, 3, -1, 0, 1) == -1


def test_tpad_argument_errors_without_gpu():
    """Weights: exactly one of w and packed_w; negative pads are a bad shape.
    Both are rejected before any device access."""
    args = (4, 1, 5, 8, 8, 8, 3, 3, 3)
    fake = 1 << 40
    st = L.conv3d_forward_tpad(fake, fake, fake, None, fake + (1 << 30), *args, 2, 0, 1, 1,
                               1, 1, 1, 1, 0, None)
    assert st == 1  # both weight forms
    st = L.conv3d_forward_tpad(fake, None, None, None, fake + (1 << 30), *args, 2, 0, 1, 1,
                               1, 1, 1, 1, 0, None)
    assert st == 1  # neither
    st = L.conv3d_forward_tpad(fake, fake, None, None, fake + (1 << 30), *args, -1, 0, 1, 1,
                               1, 1, 1, 1, 0, None)
    assert st == 2
    st = L.conv3d_forward_tpad(fake, fake, None, None, fake + (1 << 30), *args, 0, -2, 1, 1,
                               1, 1, 1, 1, 0, None)
    assert st == 2


def test_fold_batchnorm_host_function():
    """libconv's host fold against the oracle's fp64 fold: each value is the
    fp64 result rounded once to fp32 (within one fp32 ulp), in place too."""
    r = np.random.default_rng(92)
    w = r.standard_normal((8, 3, 3, 3)).astype(np.float32)
    b = r.standard_normal(8).astype(np.float32)
    g, be = r.uniform(0.5, 2, 8).astype(np.float32), r.standard_normal(8).astype(np.float32)
    mu, var = r.standard_normal(8).astype(np.float32), r.uniform(0.1, 2, 8).astype(np.float32)
    wf, bf = L.fold_batchnorm(w, b, g, be, mu, var, 1e-5)
    rw, rb = oracle.fold_batchnorm(w, b, g, be, mu, var, np.float32(1e-5))
    np.testing.assert_allclose(wf, rw, rtol=2 ** -23, atol=0)
    np.testing.assert_allclose(bf, rb, rtol=2 ** -23, atol=1e-7)
    wn, bn = L.fold_batchnorm(w, None, g, be, mu, var, 1e-5)
    np.testing.assert_array_equal(wn, wf)
    _, rb0 = oracle.fold_batchnorm(w, None, g, be, mu, var, np.float32(1e-5))
    np.testing.assert_allclose(bn, rb0, rtol=2 ** -23, atol=1e-7)
    # in place: output pointers equal to the inputs
    import ctypes
    w2, b2 = w.copy(), b.copy()
    fp = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    st = L.load().libconv_fold_batchnorm(fp(w2), fp(b2), fp(g), fp(be), fp(mu), fp(var),
                                         1e-5, 8, 27, fp(w2), fp(b2))
    assert st == 0
    np.testing.assert_array_equal(w2, wf)
    np.testing.assert_array_equal(b2, bf)


def test_fold_batchnorm_errors():
    import ctypes
    w = np.ones((2, 4), np.float32)
    v = np.ones(2, np.float32)
    fp = lambda a: None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
    lib = L.load()
    wo, bo = np.empty_like(w), np.empty(2, np.float32)
    assert lib.libconv_fold_batchnorm(fp(w), None, None, fp(v), fp(v), fp(v), 1e-5, 2, 4,
                                      fp(wo), fp(bo)) == 1
    assert lib.libconv_fold_batchnorm(fp(w), None, fp(v), fp(v), fp(v), fp(v), 1e-5, 0, 4,
                                      fp(wo), fp(bo)) == 2
    neg = np.array([1.0, -1.0], np.float32)
    wo[:] = 7
    assert lib.libconv_fold_batchnorm(fp(w), None, fp(v), fp(v), fp(v), fp(neg), 1e-5, 2, 4,
                                      fp(wo), fp(bo)) == 2
    assert np.all(wo == 7)  # nothing written


def test_cpack_bytes():
    # [N][ceil(C/g)][T][H][W] x 16 bytes, g = 16 bytes of channels
    assert L.libconv_cpack_bytes(2, 13, 1, 5, 7, L.F16) == 2 * 2 * 5 * 7 * 16
    assert L.libconv_cpack_bytes(1, 13, 3, 5, 7, L.F32) == 1 * 4 * 3 * 5 * 7 * 16
    assert L.libconv_cpack_bytes(1, 8, 1, 1, 1, L.BF16) == 16
    assert L.libconv_cpack_bytes(0, 8, 1, 4, 4, L.F16) == 0
    assert L.libconv_cpack_bytes(1, 0, 1, 4, 4, L.F16) == -1
    assert L.libconv_cpack_bytes(1, 8, 1, 4, 4, 9) == -1
    assert L.libconv_cpack_bytes(1, 1 << 20, 1, 1 << 10, 1 << 10, L.F32) == -1


def test_cpack_argument_errors_without_gpu():
    """Rejected before any device access; a valid call reaches the device
    check (this host has none)."""
    fake = 1 << 40
    y = fake + (1 << 32)
    geo = (1, 16, 5, 8, 32, 24, 3, 3, 3, 1, 1, 1, 1, 1, 1, 1)
    assert L.conv3d_forward_cpack(fake, fake, fake, None, y, *geo, L.F16, 0, None) == 1
    assert L.conv3d_forward_cpack(fake, None, None, None, y, *geo, L.F16, 0, None) == 1
    assert L.conv3d_forward_cpack(fake, fake, None, None, y, *geo, 7, 0, None) == 3
    assert L.conv3d_forward_cpack(fake, fake, None, None, y, *geo, L.F16, 3, None) == 4
    assert L.conv3d_forward_cpack(fake, fake, None, None, fake, *geo, L.F16, 0, None) == 5
    assert L.conv3d_forward_cpack(fake, fake, None, None, y, *geo, L.F16, 0, None) == 7
    assert L.libconv_pack_activations(fake, y, 1, 16, 5, 8, 32, 5, None) == 3
    assert L.libconv_pack_activations(fake, y, 1, 0, 5, 8, 32, L.F16, None) == 2
    assert L.libconv_pack_activations(None, y, 1, 16, 5, 8, 32, L.F16, None) == 1
    assert L.libconv_pack_activations(fake, fake + 64, 1, 16, 5, 8, 32, L.F16, None) == 5
    assert L.libconv_unpack_activations(fake, y, 1, 16, 5, 8, 32, L.F16, None) == 7



def test_query_plan_packed_weights_and_cpack_flags():
    """PLAN_PACKED_W plans as a call given packed weights (packed MFMA tiles,
    no split without a workspace); PLAN_CPACK plans the channel-packed
    layout's own tiles: those that read packed weights when the weights are
    packed or a workspace can hold them packed, else those that transpose
    OIDHW weights in registers."""
    vae = (1, 512, 5, 64, 120, 512, 3, 3, 3, 1, 1, 1, 1, 1, 1, L.F16, 1, L.ALGO_AUTO)
    st, algo, tile, grid, ks = L.libconv_query_plan(*vae, L.PLAN_PACKED_W)
    assert st == 0 and algo == L.ALGO_IGEMM and ks == 1
    assert L.libconv_tile_name(tile).startswith("igemm16p_")
    st, algo, tile, grid, ks = L.libconv_query_plan(*vae, L.PLAN_CPACK)
    assert st == 0 and algo == L.ALGO_IGEMM
    assert L.libconv_tile_name(tile).startswith("igemm16xo_")
    ws = L.libconv_workspace_size(1, 512, 5, 64, 120, 512, 3, 3, 3, 1, 1, 1, 1, 1, 1, 1,
                                  L.F16, 1, L.ALGO_AUTO, L.PLAN_CPACK)
    assert ws >= L.libconv_packed_weight_bytes(512, 512, 3, 3, 3, L.F16)
    st, algo, tile, grid, ks = L.libconv_query_plan(*vae, L.PLAN_CPACK, ws)
    assert st == 0 and L.libconv_tile_name(tile).startswith("igemm16x_")
    st, algo, tile, grid, ks = L.libconv_query_plan(*vae, L.PLAN_CPACK | L.PLAN_PACKED_W)
    assert st == 0 and L.libconv_tile_name(tile).startswith("igemm16x_")
    # a 5x5 layer: no packed kernels at all
    k5 = (1, 16, 1, 32, 32, 16, 1, 5, 5, 0, 2, 2, 1, 1, 1, L.F16, 0, L.ALGO_AUTO)
    assert L.libconv_query_plan(*k5, L.PLAN_PACKED_W)[0] == 6
    # the channel-packed layout without packed weights: the vector-ALU kernel
    st, algo, tile, grid, ks = L.libconv_query_plan(*k5, L.PLAN_CPACK)
    assert st == 0 and algo == L.ALGO_DIRECT and not L.libconv_tile_name(tile).startswith("tap_")


def test_new_calls_with_an_empty_batch_do_nothing():
    """N = 0: nothing to compute, OK without touching a device (this host has
    none) for the window, chunked, packed-layout and conversion calls."""
    fake = 1 << 40
    y = fake + (1 << 32)
    geo = (0, 16, 5, 8, 32, 24, 3, 3, 3, 2, 0, 1, 1, 1, 1, 1)
    assert L.conv3d_forward_cpack(fake, fake, None, None, y, *geo, L.F16, 0, None) == 0
    assert L.conv3d_forward_frames(fake, fake, None, None, y, *geo, 1, 2, L.F16, 0, None) == 0
    need = L.libconv_chunked_workspace_bytes(*geo, 2, L.F16)
    assert need >= 0
    assert L.conv3d_forward_chunked(fake, fake, None, None, y, *geo, 2, fake + (1 << 34),
                                    max(need, 1), L.F16, 0, None, None, None) == 0
    assert L.libconv_pack_activations(fake, y, 0, 16, 5, 8, 32, L.F16, None) == 0
    assert L.libconv_unpack_activations(fake, y, 0, 16, 5, 8, 32, L.F16, None) == 0


def test_noalloc_rejects_plans_beyond_its_scratch():
    """conv3d_forward_noalloc refuses, before any device access, a call whose
    best plan needs more than the library's 64 MiB scratch array (here the
    UNet 1280-channel layer at 64x64: 113 MB of packed weights and partial
    sums); within the limit a valid call reaches the device check."""
    fake = 1 << 40
    args = (2, 1280, 1, 64, 64, 1280, 1, 3, 3, 0, 1, 1, 1, 1, 1, L.BF16, 0)
    need = L.libconv_workspace_size(2, 1280, 1, 64, 64, 1280, 1, 3, 3, 0, 0, 1, 1, 1, 1, 1,
                                    L.BF16, 0, L.ALGO_AUTO, 0)
    assert need > L.SCRATCH_BYTES
    assert L.conv3d_forward_noalloc(fake, fake + (1 << 30), None, fake + (1 << 33), *args,
                                    None) == 13
    assert L.libconv_status_string(13).startswith("the call needs more workspace")
    small = (1, 64, 5, 8, 40, 64, 3, 3, 3, 1, 1, 1, 1, 1, 1, L.F16, 0)
    assert L.conv3d_forward_noalloc(fake, fake + (1 << 30), None, fake + (1 << 33), *small,
                                    None) == 7
    assert L.conv3d_forward_noalloc(fake, fake + (1 << 30), None, fake + (1 << 33), *small[:15],
                                    9, 0, None) == 3
