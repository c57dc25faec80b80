"""Every implicit-GEMM tile of the library, forced on a small layer of its own
geometry and dtype, against the fp64 oracle.

The shapes span several tiles in every direction and end in ragged tails
(pixels, output channels); half of them have a channel count that is not a
multiple of a stage's channels, which takes the guarded-read path.  Tiles
that read the input as aligned 16-byte runs get W % 8 == 0, the others
("_e" tiles) an odd W."""
import re
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


def _tiles(plain_layout_only: bool = False):
    """The MFMA tiles; plain_layout_only drops the channel-packed ones
    ("igemm16x" / "igemm32x", tested with their own layout elsewhere)."""
    import direct_implicit_gemm_amd as L
    out = []
    for tid in range(1, 400):
        name = L.libconv_tile_name(tid)
        if name.startswith("igemm") and not (plain_layout_only and name[7:8] == "x"):
            out.append((tid, name))
    return out


def _one_stage_width(tid: int, kdig: str, wide: bool) -> int:
    """The most input channels a single-stage tile takes: the widest C that
    the tile (forced through LIBCONV_FORCE_TILE) accepts for its geometry."""
    import direct_implicit_gemm_amd as L
    k = 1 if kdig == "1" else 3
    for c in ((128, 64, 32) if wide else (32, 16)):
        q = L.libconv_query_plan(1, c, 1, 12, 64, 16, 1, k, k, 0, k // 2, k // 2, 1, 1, 1,
                                 1 if wide else 0, 0, 0, 0, BIG_WS)
        if q[0] == 0 and q[2] == tid:
            return c
    raise AssertionError(f"no channel count fits tile {tid}")


def _layer_for(tid: int, name: str, ragged: bool) -> W.Layer:
    """A small layer that the tile `name` fits."""
    m = re.match(r"igemm(16|32)(p?)_k(\d+)(s(\d))?_m(\d+)w?_n(\d+)x?(\d+)?(_c8)?(_e)?(_one)?(_w1)?(_8w)?$", name)
    assert m, name
    wide, packed, kdig = m.group(1) == "16", m.group(2) == "p", m.group(3)
    stride, bm = m.group(5), int(m.group(6))
    elem = m.group(10) is not None
    one = m.group(11) is not None
    dtype = ("bf16" if tid % 2 else "f16") if wide else "f32"
    se = 8 if wide else 4
    c = (3 * se if ragged else 4 * se) if not packed else (3 * se - 4 if ragged else 4 * se)
    if one:  # single-stage tiles: every input channel in the one stage
        c = 5 * se if ragged else _one_stage_width(tid, kdig, wide)  # the stage's full width
    k = bm + bm // 2 + 8                       # ragged output-channel tiles
    w_ = 72 if not elem else 67               # ragged pixel tiles; odd W for "_e" tiles
    relu = "relu" if tid % 3 else "none"
    if kdig == "1":                            # 1x1, stride 1, pad 0 (flattened planes)
        hw = (9, 56) if not elem else (9, 51)
        return W.Layer("t", dtype, 2, c, 1, hw[0], hw[1], k, 1, 1, 1, (0, 0, 0), (1, 1, 1),
                       relu, 2, "N01", "N01", "U0.05")
    if kdig == "333":
        return W.Layer("t", dtype, 1, c, 4, 9, w_, k, 3, 3, 3,
                       (1, 1, 1), (1, 1, 1), relu, 3, "N01", "N01", "U0.05")
    s = int(stride)
    h = 19 if s == 1 else 37
    return W.Layer("t", dtype, 1, c, 1, h, w_ if s == 1 else 2 * w_ + (0 if not elem else 1),
                   k, 1, 3, 3, (0, 1, 1), (1, s, s), relu, 2, "N01", "N01", "U0.05")


@pytest.mark.parametrize("ragged", [False, True])
def test_every_tile(ragged, monkeypatch):
    import direct_implicit_gemm_amd as L
    tiles = _tiles(plain_layout_only=True)
    assert len(tiles) >= 20
    for i, (tid, name) in enumerate(tiles):
        monkeypatch.setenv("LIBCONV_FORCE_TILE", str(tid))
        layer = _layer_for(tid, name, ragged)
        q = L.libconv_query_plan(layer.N, layer.C_in, layer.T, layer.H, layer.W, layer.C_out,
                                 layer.KT, layer.KH, layer.KW, *layer.pad, *layer.stride,
                                 W.DTYPE_CODE[layer.dtype], W.ACT_CODE[layer.act], 0, 0,
                                 BIG_WS)
        assert q[0] == 0 and q[2] == tid, (name, layer, q)
        note(f"tile {tid} {name} ragged={ragged}: x={layer.x_shape} w={layer.w_shape} "
             f"{layer.dtype} {layer.act}")
        x, w, b = W.make_inputs(layer, 900 + 2 * i + ragged)
        st, pd = (layer.stride[1:], layer.pad[1:]) if layer.dims == 2 else (layer.stride,
                                                                           layer.pad)
        y = L.conv_nd(x.torch("cuda"), w.torch("cuda"), b.torch("cuda"), st, pd, layer.act)
        torch.cuda.synchronize()
        ref, s = oracle.conv(x.f64(), w.f64(), b.f64(), *oracle_args(layer),
                             relu=layer.act == "relu")
        m = metrics(to_f64(y), ref, s, layer.dtype)
        note(f"  {m}")
        assert_gates(m, layer.dtype, name)


def _tap_tiles():
    import direct_implicit_gemm_amd as L
    out = []
    for tid in range(100, 200):
        name = L.libconv_tile_name(tid)
        if name.startswith("tap_"):
            out.append((tid, name))
    return out


def _tap_layer_for(i: int, name: str, ragged: bool) -> W.Layer:
    """A small layer that the tap tile `name` fits: ragged output rows,
    columns and channels; some with frames (3-D, one frame tap), some with
    more input channels than one LDS stage holds."""
    m = re.match(r"tap_k(\d)(s(\d))?_cot(\d+)_r(\d+)(_e)?$", name)
    assert m, name
    k, s = int(m.group(1)), int(m.group(3) or 1)
    cot, elem = int(m.group(4)), m.group(6) is not None
    dtype = ("f32", "f16", "bf16")[i % 3]
    c = 3 if not ragged else 5
    kout = cot + cot // 2 + 1 if ragged else 2 * cot
    wd = 72 * s if not elem else 67 * s + 1
    h = 13 * s + 1 if ragged else 16 * s
    pad = (k - 1) // 2
    relu = "relu" if i % 2 else "none"
    if ragged:  # frames: a 3-D layer with one frame tap
        return W.Layer("t", dtype, 1, c, 2, h, wd, kout, 1, k, k, (0, pad, pad), (1, s, s),
                       relu, 3, "N01", "N01", "U0.05")
    return W.Layer("t", dtype, 2, c, 1, h, wd, kout, 1, k, k, (0, pad, pad), (1, s, s),
                   relu, 2, "N01", "N01", "U0.05")


@pytest.mark.parametrize("ragged", [False, True])
def test_every_tap_tile(ragged, monkeypatch):
    import direct_implicit_gemm_amd as L
    tiles = _tap_tiles()
    assert len(tiles) >= 6
    for i, (tid, name) in enumerate(tiles):
        layer = _tap_layer_for(i, name, ragged)
        monkeypatch.setenv("LIBCONV_FORCE_TILE", str(tid))
        q = L.libconv_query_algo(layer.N, layer.C_in, layer.T, layer.H, layer.W, layer.C_out,
                                 layer.KT, layer.KH, layer.KW, *layer.pad, *layer.stride,
                                 W.DTYPE_CODE[layer.dtype], W.ACT_CODE[layer.act], 1)
        assert q[0] == 0 and q[2] == tid, (name, layer, q)
        note(f"tap tile {tid} {name} ragged={ragged}: x={layer.x_shape} w={layer.w_shape} "
             f"{layer.dtype} {layer.act}")
        x, w, b = W.make_inputs(layer, 700 + 2 * i + ragged)
        st, pd = (layer.stride[1:], layer.pad[1:]) if layer.dims == 2 else (layer.stride,
                                                                           layer.pad)
        y = L.conv_nd(x.torch("cuda"), w.torch("cuda"), b.torch("cuda"), st, pd, layer.act,
                      "direct")
        torch.cuda.synchronize()
        ref, s = oracle.conv(x.f64(), w.f64(), b.f64(), *oracle_args(layer),
                             relu=layer.act == "relu")
        m = metrics(to_f64(y), ref, s, layer.dtype)
        note(f"  {m}")
        assert_gates(m, layer.dtype, name)


def test_tile_occupancy_table_matches_runtime():
    """The dispatcher's per-tile workgroups-per-CU figures against the HIP
    runtime's occupancy query for the built kernels."""
    import direct_implicit_gemm_amd as L
    for tid, name in _tiles():
        for dt in (0, 1, 2):
            table = L.libconv_tile_occupancy(tid, dt, False)
            if table < 0:
                continue
            measured = L.libconv_tile_occupancy(tid, dt, True)
            note(f"occupancy {tid} {name} dtype {dt}: table {table} runtime {measured}")
            assert measured == table, (name, dt, table, measured)
