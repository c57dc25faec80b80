"""Seeded random geometries through the dispatcher against the fp64 oracle:
2-D and 3-D, every dtype, kernel sizes 1-5 (height and width independent),
strides 1-3, symmetric spatial padding, time padding that may differ before
and after the frames, odd channel counts and extents, batch 1-3, with and
without bias and ReLU; a subset in the channel-packed layout.  The shapes
are small enough for the oracle to take milliseconds each."""
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


def _geometry(i):
    r = np.random.default_rng(2000 + i)
    while True:
        dims = 3 if r.random() < 0.35 else 2
        dt = ("f32", "f16", "bf16")[r.integers(0, 3)]
        N = int(r.integers(1, 4))
        C = int(r.choice([1, 3, 4, 7, 8, 13, 16, 24, 32, 40]))
        K = int(r.choice([1, 5, 8, 16, 24, 33, 64, 70]))
        KH, KW = int(r.integers(1, 6)), int(r.integers(1, 6))
        sh, sw = int(r.integers(1, 4)), int(r.integers(1, 4))
        ph, pw = int(r.integers(0, KH)), int(r.integers(0, KW))
        H, Wd = int(r.integers(1, 30)), int(r.integers(1, 70))
        if dims == 3:
            T = int(r.integers(1, 6))
            KT = int(r.integers(1, 4))
            st = int(r.integers(1, 3))
            pf, pb = int(r.integers(0, KT)), int(r.integers(0, KT))
        else:
            T, KT, st, pf, pb = 1, 1, 1, 0, 0
        if i % 2:  # the matrix-core geometries: 3x3(x3) stride 1 or 2, 1x1
            C = int(r.choice([8, 16, 24, 32, 48, 64, 96]))
            K = int(r.choice([8, 24, 40, 64, 72, 128, 130]))
            H, Wd = int(r.integers(4, 40)), int(r.integers(8, 90))
            if r.random() < 0.3:
                KH = KW = 1
                sh = sw = 1
                ph = pw = 0
                KT, st, pf, pb = 1, 1, 0, 0
            else:
                KH = KW = 3
                sh = sw = int(r.choice([1, 1, 2])) if dims == 2 else 1
                ph = pw = 1
                if dims == 3:
                    KT, st = 3, 1
                    pf, pb = (2, 0) if r.random() < 0.5 else (1, 1)
        if (oracle.out_extent2(T, KT, pf, pb, st) < 1 or oracle.out_extent(H, KH, ph, sh) < 1
                or oracle.out_extent(Wd, KW, pw, sw) < 1):
            continue
        macs = N * K * C * KT * KH * KW * T * H * Wd
        if macs > 6e7:
            continue
        relu = bool(r.random() < 0.5)
        bias = bool(r.random() < 0.8)
        return dict(dims=dims, dt=dt, N=N, C=C, K=K, T=T, H=H, W=Wd, KT=KT, KH=KH, KW=KW,
                    st=st, sh=sh, sw=sw, pf=pf, pb=pb, ph=ph, pw=pw, relu=relu, bias=bias)


def _inputs(g, seed):
    layer = W.Layer("rnd", g["dt"], g["N"], g["C"], g["T"], g["H"], g["W"], g["K"], g["KT"],
                    g["KH"], g["KW"], (g["pf"], g["ph"], g["pw"]), (g["st"], g["sh"], g["sw"]),
                    "relu" if g["relu"] else "none", g["dims"], "N01", "N01",
                    "U0.05" if g["bias"] else "zero", pad_t_back=g["pb"] if g["dims"] == 3 else None)
    x, w, b = W.make_inputs(layer, seed)
    return layer, x, w, (b if g["bias"] else None)


def _oracle(layer, x, w, b):
    if layer.dims == 3:
        return oracle.conv(x.f64(), w.f64(), None if b is None else b.f64(), layer.stride,
                           layer.pad, relu=layer.act == "relu", pad_t_back=layer.pad_t_back)
    return oracle.conv(x.f64(), w.f64(), None if b is None else b.f64(), layer.stride[1:],
                       layer.pad[1:], relu=layer.act == "relu")


@pytest.mark.parametrize("i", range(128))
def test_random_geometry(i):
    import direct_implicit_gemm_amd as L
    g = _geometry(i)
    layer, x, w, b = _inputs(g, 3000 + i)
    note(f"random {i}: {g}")
    bt = None if b is None else b.torch("cuda")
    if layer.dims == 3:
        y = L.conv3d_tpad(x.torch("cuda"), w.torch("cuda"), bt, (g["pf"], g["pb"]),
                          layer.stride, layer.pad[1:], layer.act)
    else:
        y = L.conv_nd(x.torch("cuda"), w.torch("cuda"), bt, layer.stride[1:], layer.pad[1:],
                      layer.act)
    torch.cuda.synchronize()
    ref, s = _oracle(layer, x, w, b)
    m = metrics(to_f64(y), ref, s, g["dt"])
    note(f"  {m}")
    assert_gates(m, g["dt"], f"random {i}")


@pytest.mark.parametrize("i", range(48))
def test_random_geometry_channel_packed(i):
    import direct_implicit_gemm_amd as L
    g = _geometry(100 + i)
    layer, x, w, b = _inputs(g, 3100 + i)
    note(f"random packed {i}: {g}")
    xp = L.pack_activations(x.torch("cuda"))
    bt = None if b is None else b.torch("cuda")
    if layer.dims == 3:
        yp = L.conv_cpack(xp, w.torch("cuda"), bt, layer.stride, layer.pad,
                          pad_t=(g["pf"], g["pb"]), act=layer.act)
    else:
        yp = L.conv_cpack(xp, w.torch("cuda"), bt, layer.stride[1:], layer.pad[1:], act=layer.act)
    y = L.unpack_activations(yp)
    torch.cuda.synchronize()
    ref, s = _oracle(layer, x, w, b)
    m = metrics(to_f64(y), ref, s, g["dt"])
    note(f"  {m}")
    assert_gates(m, g["dt"], f"random packed {i}")
