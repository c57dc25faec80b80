"""libconv calls recorded into a HIP graph (through torch's graph capture,
whose capture stream is the stream libconv enqueues on) and replayed: every
replay, with the program's own eager work and synchronisations between
replays, must give exactly the eager result (the kernels are deterministic,
so bit for bit).  Covers a chained fp32 stack, layers given a workspace
(split-K partial sums, weights packed per call) and the two north-star
exports called directly."""
import sys

import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def note(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _stack(specs, seed):
    """Device inputs and outputs for a list of (layer, chained) specs."""
    dev = "cuda:0"
    xs, ws, bs, outs = [], [], [], []
    for i, layer in enumerate(specs):
        x, w, b = W.make_inputs(layer, seed + i)
        xs.append(x.torch(dev))
        ws.append(w.torch(dev))
        bs.append(b.torch(dev))
    return xs, ws, bs


def _run(L, specs, xs, ws, bs, outs, chained):
    for i, l in enumerate(specs):
        x_in = outs[i - 1] if (chained and i > 0) else xs[i]
        st, pd = (l.stride[1:], l.pad[1:]) if l.dims == 2 else (l.stride, l.pad)
        L.conv_nd(x_in, ws[i], bs[i], st, pd, l.act, out=outs[i])


def _check_graph(specs, chained, seed):
    import direct_implicit_gemm_amd as L
    xs, ws, bs = _stack(specs, seed)
    outs = []
    for l in specs:
        full = tuple(L.libconv_out_size(n, k, p, s) for n, k, p, s in
                     zip((l.T, l.H, l.W), (l.KT, l.KH, l.KW), l.pad, l.stride))
        shape = (l.N, l.C_out) + (full[1:] if l.dims == 2 else full)
        outs.append(torch.empty(shape, dtype=xs[len(outs)].dtype, device="cuda:0"))
    _run(L, specs, xs, ws, bs, outs, chained)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run(L, specs, xs, ws, bs, outs, chained)
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda:0")
    for r in range(4):
        for o in outs:
            o.fill_(float("nan") if o.dtype == torch.float32 else 0.0)  # the replay must rewrite
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o, eager[i]), f"replay {r}, layer {i}: differs from eager"
        # the program's own eager work between replays
        junk.mul_(1.0001).add_(0.5)
        _run(L, specs[:1], xs, ws, bs, [torch.empty_like(outs[0])] + outs[1:], False)
        torch.cuda.synchronize()
        note(f"replay {r}: all {len(outs)} outputs equal the eager result")


def test_graph_chained_fp32_stack():
    l1 = W.Layer("g1", "f32", 1, 3, 1, 66, 96, 16, 1, 3, 3, (0, 1, 1), (1, 2, 2), "relu", 2,
                 "U01", "U11", "U0.1")
    l2 = W.Layer("g2", "f32", 1, 16, 1, 33, 48, 32, 1, 3, 3, (0, 1, 1), (1, 1, 1), "relu", 2,
                 "U01", "U11", "U0.1")
    l3 = W.Layer("g3", "f32", 1, 32, 1, 33, 48, 64, 1, 1, 1, (0, 0, 0), (1, 1, 1), "none", 2,
                 "U01", "U11", "U0.1")
    _check_graph([l1, l2, l3], True, 500)


def test_graph_layers_with_a_workspace(monkeypatch):
    """Calls given a workspace: split-K partial sums (forced here) and weights
    packed per call on a 3-D layer, both in the workspace.  The plan does not
    depend on capture, so the replays run the eager kernels: every replay
    must equal the eager result bit for bit, and the eager result must pass
    the oracle gates.  A forward on weights packed beforehand is recorded
    alongside."""
    import direct_implicit_gemm_amd as L
    import oracle
    from convcheck import assert_gates, metrics, oracle_args, to_f64
    monkeypatch.setenv("LIBCONV_FORCE_KSPLIT", "2")
    specs = [
        W.Layer("g4", "bf16", 1, 160, 1, 9, 48, 72, 1, 3, 3, (0, 1, 1), (1, 1, 1), "relu", 2,
                "N01", "N01", "U0.05"),
        W.Layer("g5", "f16", 1, 64, 3, 6, 40, 64, 3, 3, 3, (1, 1, 1), (1, 1, 1), "none", 3,
                "N01", "N01", "U0.05"),
    ]
    ins = [W.make_inputs(l, 600 + i) for i, l in enumerate(specs)]
    dev = "cuda:0"
    xs = [x.torch(dev) for x, _, _ in ins]
    ws = [w.torch(dev) for _, w, _ in ins]
    bs = [b.torch(dev) for _, _, b in ins]
    packed = L.pack_weights(ws[1])          # before any capture
    # one workspace per call, allocated before capture (a model keeps its own)
    need = []
    for l in specs:
        pt_ = l.pad[0]
        need.append(L.libconv_workspace_size(l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH,
                                             l.KW, pt_, pt_, l.pad[1], l.pad[2], *l.stride,
                                             W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act], 0, 0))
    assert need[0] > 0 and need[1] > 0, need
    wsp = [torch.empty(n, dtype=torch.uint8, device=dev) for n in need]
    torch.cuda.synchronize()

    def run(outs):
        for i, l in enumerate(specs):
            st, pd = oracle_args(l)
            L.conv_nd(xs[i], ws[i], bs[i], st, pd, l.act, out=outs[i], workspace=wsp[i])
        st, pd = oracle_args(specs[1])
        L.conv_nd_packed(xs[1], packed, bs[1], st, pd, specs[1].act, out=outs[2])

    def fresh():
        return [torch.empty((1, 72, 9, 48), dtype=xs[0].dtype, device=dev),
                torch.empty((1, 64, 3, 6, 40), dtype=xs[1].dtype, device=dev),
                torch.empty((1, 64, 3, 6, 40), dtype=xs[1].dtype, device=dev)]

    def gates(outs, what):
        for i, l in enumerate(specs + [specs[1]]):
            x, w, b = ins[min(i, 1)]
            ref, s = oracle.conv(x.f64(), w.f64(), b.f64(), *oracle_args(l),
                                 relu=l.act == "relu")
            m = metrics(to_f64(outs[i]), ref, s, l.dtype)
            note(f"{what} output {i}: {m}")
            assert_gates(m, l.dtype, f"{what} {i}")

    eager = fresh()
    run(eager)
    torch.cuda.synchronize()
    gates(eager, "eager")
    outs = fresh()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(outs)
    torch.cuda.synchronize()
    for r in range(4):
        for o in outs:
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert torch.equal(o, eager[i]), f"replay {r}, output {i} differs from eager"
        run(fresh())  # the program's own eager work between replays (same workspaces)
        torch.cuda.synchronize()
        note(f"replay {r} ok")


def test_graph_north_star_entry_points():
    """conv3d_forward and conv2d_forward themselves (no workspace), with data,
    recorded into a graph: every replay equals the eager call bit for bit and
    both pass the oracle gates; the captured calls run the MFMA kernels the
    eager ones run (a 3x3x3 f16 layer and a 3x3 bf16 layer)."""
    import direct_implicit_gemm_amd as L
    import oracle
    from convcheck import assert_gates, metrics, oracle_args, to_f64
    dev = "cuda:0"
    l3 = W.Layer("ns3", "f16", 1, 64, 4, 9, 40, 72, 3, 3, 3, (1, 1, 1), (1, 1, 1), "relu", 3,
                 "N01", "N01", "U0.05")
    l2 = W.Layer("ns2", "bf16", 2, 96, 1, 11, 40, 80, 1, 3, 3, (0, 1, 1), (1, 1, 1), "none", 2,
                 "N01", "N01", "U0.05")
    for l in (l3, l2):
        q = L.libconv_query_plan(l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH, l.KW,
                                 *l.pad, *l.stride, W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act],
                                 0, 0, 0)
        assert q[0] == 0 and q[1] == L.ALGO_IGEMM, (l.name, q)
        note(f"{l.name}: {L.libconv_tile_name(q[2])}")
    i3, i2 = W.make_inputs(l3, 620), W.make_inputs(l2, 621)
    t3 = [t.torch(dev) for t in i3]
    t2 = [t.torch(dev) for t in i2]
    y3 = torch.empty((1, 72, 4, 9, 40), dtype=torch.float16, device=dev)
    y2 = torch.empty((2, 80, 11, 40), dtype=torch.bfloat16, device=dev)

    def run():
        s = torch.cuda.current_stream().cuda_stream
        st = L.conv3d_forward(t3[0].data_ptr(), t3[1].data_ptr(), t3[2].data_ptr(),
                              y3.data_ptr(), 1, 64, 4, 9, 40, 72, 3, 3, 3, 1, 1, 1, 1, 1, 1,
                              L.F16, L.ACT_RELU, s)
        assert st == 0, st
        st = L.conv2d_forward(t2[0].data_ptr(), t2[1].data_ptr(), t2[2].data_ptr(),
                              y2.data_ptr(), 2, 96, 11, 40, 80, 3, 3, 1, 1, 1, 1, L.BF16,
                              L.ACT_NONE, s)
        assert st == 0, st

    run()
    torch.cuda.synchronize()
    eager = [y3.clone(), y2.clone()]
    for l, (x, w, b), y in ((l3, i3, eager[0]), (l2, i2, eager[1])):
        ref, sm = oracle.conv(x.f64(), w.f64(), b.f64(), *oracle_args(l), relu=l.act == "relu")
        m = metrics(to_f64(y), ref, sm, l.dtype)
        note(f"{l.name} eager: {m}")
        assert_gates(m, l.dtype, l.name)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        y3.fill_(float("nan"))
        y2.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y3, eager[0]) and torch.equal(y2, eager[1]), f"replay {r}"
        run()  # eager work between replays
        torch.cuda.synchronize()
        note(f"replay {r}: conv3d_forward and conv2d_forward equal the eager calls")


def test_graph_packed_layout_frames_and_causal():
    """Channel-packed layers (packed weights: MFMA tiles, nothing allocated),
    a causal layer and a frame-window call, recorded into one graph: every
    replay equals the eager result bit for bit."""
    import direct_implicit_gemm_amd as L
    dev = "cuda:0"
    l1 = W.Layer("gp1", "f16", 1, 16, 4, 8, 40, 40, 3, 3, 3, (1, 1, 1), (1, 1, 1), "relu", 3,
                 "N01", "N01", "U0.05")
    l2 = l1.with_(C_in=40, C_out=24)
    x, w1, b1 = W.make_inputs(l1, 610)
    _, w2, b2 = W.make_inputs(l2, 611)
    xt = x.torch(dev)
    p1, p2 = L.pack_weights(w1.torch(dev)), L.pack_weights(w2.torch(dev))
    bt1, bt2 = b1.torch(dev), b2.torch(dev)
    xp = L.pack_activations(xt)
    y1 = L.conv_cpack(xp, p1, bt1, 1, 1, act="relu")           # allocate outputs eagerly
    y2 = L.conv_cpack(y1, p2, bt2, 1, 1, act="relu")
    yc = L.conv3d_tpad(xt, p1, bt1, (2, 0), 1, 1, "relu")        # causal
    st_, f0, tw = L.libconv_frame_window(4, 3, 2, 0, 1, 2, 2)
    assert st_ == 0
    xw = xt[:, :, f0:f0 + tw].contiguous()
    yf = L.conv3d_frames(xw, p1, bt1, 4, (2, 2), (2, 0), 1, 1, "relu")

    def run():
        L.conv_cpack(xp, p1, bt1, 1, 1, act="relu", out=y1)
        L.conv_cpack(y1, p2, bt2, 1, 1, act="relu", out=y2)
        L.conv3d_tpad(xt, p1, bt1, (2, 0), 1, 1, "relu", out=yc)
        L.conv3d_frames(xw, p1, bt1, 4, (2, 2), (2, 0), 1, 1, "relu", out=yf)

    run()
    torch.cuda.synchronize()
    eager = [y1.data.clone(), y2.data.clone(), yc.clone(), yf.clone()]
    # the window's frames equal those frames of the causal whole-clip call
    assert torch.equal(yf, yc[:, :, 2:4]) or torch.allclose(yf.float(), yc[:, :, 2:4].float(),
                                                            rtol=2 ** -9, atol=2 ** -12)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        for t in (y1.data, y2.data):
            t.zero_()
        yc.fill_(float("nan"))
        yf.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, t in enumerate((y1.data, y2.data, yc, yf)):
            assert torch.equal(t, eager[i]), f"replay {r}, output {i}"
        note(f"replay {r}: packed, causal and window outputs equal the eager ones")
