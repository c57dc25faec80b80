"""conv3d_forward_noalloc: the convolution with the library's own static
scratch array as its workspace (no allocation anywhere).  Through the C ABI it
must give exactly what conv3d_forward_ws gives with the workspace
libconv_workspace_size names (the same plan, hence bit for bit), and pass the
oracle gates, on two calls in a row, the second on a smaller input (the
scratch keeps the first call's contents)."""
import sys

import pytest

import oracle
import workloads as W
from convcheck import assert_gates, metrics, oracle_args, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _shape_args(l):
    return (l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH, l.KW, *l.pad, *l.stride)


def _out_shape(L, l):
    o = [L.libconv_out_size(n, k, p, s) for n, k, p, s in
         zip((l.T, l.H, l.W), (l.KT, l.KH, l.KW), l.pad, l.stride)]
    return (l.N, l.C_out) + (tuple(o[1:]) if l.dims == 2 else tuple(o))


def _both(L, l, seed):
    """(y from conv3d_forward_noalloc, y from conv3d_forward_ws, inputs, tile)."""
    x, w, b = W.make_inputs(l, seed)
    dev = "cuda:0"
    xt, wt, bt = x.torch(dev), w.torch(dev), b.torch(dev)
    dt, act = W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act]
    need = L.libconv_workspace_size(l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH, l.KW,
                                    l.pad[0], l.pad[0], l.pad[1], l.pad[2], *l.stride, dt, act,
                                    L.ALGO_AUTO, 0)
    assert 0 < need <= L.SCRATCH_BYTES, need
    q = L.libconv_query_plan(*_shape_args(l), dt, act, L.ALGO_AUTO, 0, need)
    assert q[0] == 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    y_ws = torch.empty(_out_shape(L, l), dtype=xt.dtype, device=dev)
    y_na = torch.full(_out_shape(L, l), float("nan"), dtype=xt.dtype, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    st = L.conv3d_forward_ws(xt.data_ptr(), wt.data_ptr(), bt.data_ptr(), y_ws.data_ptr(),
                             *_shape_args(l), dt, act, ws.data_ptr(), need, s)
    assert st == 0, st
    st = L.conv3d_forward_noalloc(xt.data_ptr(), wt.data_ptr(), bt.data_ptr(), y_na.data_ptr(),
                                  *_shape_args(l), dt, act, s)
    assert st == 0, st
    torch.cuda.synchronize()
    return y_na, y_ws, (x, w, b), L.libconv_tile_name(q[2]) + f" ksplit={q[4]}"


CASES = [
    # a 3-D f16 layer whose plan packs the weights into the scratch, then a
    # smaller one whose plan splits the reduction (partial sums in the scratch)
    ("3d", W.Layer("na3", "f16", 1, 128, 5, 64, 120, 128, 3, 3, 3, (1, 1, 1), (1, 1, 1), "relu",
                   3, "N01", "N01", "U0.05"),
     W.Layer("na3s", "f16", 1, 128, 5, 16, 96, 128, 3, 3, 3, (1, 1, 1), (1, 1, 1), "none", 3,
             "N01", "N01", "U0.05")),
    # the UNet 1280-channel bf16 layer (its plan splits the reduction 3 ways),
    # then a smaller 2-D layer
    ("2d", W.Layer("na2", "bf16", 2, 1280, 1, 32, 32, 1280, 1, 3, 3, (0, 1, 1), (1, 1, 1), "none",
                   2, "N01", "N01", "U0.05"),
     W.Layer("na2s", "bf16", 1, 256, 1, 9, 40, 96, 1, 3, 3, (0, 1, 1), (1, 1, 1), "relu", 2,
             "N01", "N01", "U0.05")),
]


def test_noalloc_plans_use_the_scratch():
    """The cases really put packed weights or partial sums in the scratch."""
    import direct_implicit_gemm_amd as L
    for _, big, small in CASES:
        for l in (big, small):
            dt, act = W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act]
            need = L.libconv_workspace_size(*_shape_args(l)[:9], l.pad[0], l.pad[0], l.pad[1],
                                            l.pad[2], *l.stride, dt, act, L.ALGO_AUTO, 0)
            q = L.libconv_query_plan(*_shape_args(l), dt, act, L.ALGO_AUTO, 0, need)
            name = L.libconv_tile_name(q[2])
            note(f"{l.name}: {name} ksplit={q[4]} scratch {need} bytes")
            assert q[0] == 0 and 0 < need <= L.SCRATCH_BYTES
            assert q[4] > 1 or "16p" in name, (l.name, name, q)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_call(case):
    import direct_implicit_gemm_amd as L
    _, big, small = case
    for i, l in enumerate((big, small)):
        note(f"noalloc {l.name}: x={l.x_shape} w={l.w_shape} {l.dtype}")
        y_na, y_ws, (x, w, b), plan = _both(L, l, 1700 + 10 * i + len(l.name))
        note(f"  plan {plan}")
        assert torch.equal(y_na, y_ws), f"{l.name}: noalloc differs from the workspace call"
        ref, s = oracle.conv(x.f64(), w.f64(), b.f64(), *oracle_args(l), relu=l.act == "relu")
        m = metrics(to_f64(y_na), ref, s, l.dtype)
        note(f"  {m}")
        assert_gates(m, l.dtype, l.name)
