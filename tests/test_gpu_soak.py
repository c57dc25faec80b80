"""Soak: ten thousand calls over the workload layers and the other call forms,
with device memory and host memory sampled.  No call allocates device memory
and none keeps anything between calls, so after the warm-up neither may grow
(the method of "OpenCL-101 issue 52": a leak is found by looping each API step
many times and watching memory).  The loop stops at the first failed call."""
import os
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


def _rss_bytes() -> int:
    with open("/proc/self/status") as f:
        for line in f:
            if line.startswith("VmRSS:"):
                return int(line.split()[1]) * 1024
    return 0


CONFIG_LAYERS = ("c1", "c2_L1", "c2_L2", "c2_L3", "c2_L4", "c3_A", "c3_B", "c4_A", "c4_B",
                 "c5_A", "c5_B")


def _calls(L, dev):
    """A list of (name, fn) issuing one libconv call each on preallocated
    tensors: every config layer through its spec export and through the
    workspace call, plus a causal call on packed weights, a channel-packed
    call, a split-K call and the no-allocation call."""
    s = torch.cuda.current_stream(dev).cuda_stream
    calls = []
    keep = []
    for name in CONFIG_LAYERS:
        l = W.ALL_LAYERS[name]
        x, w, b = (t.torch(dev) for t in W.make_inputs(l, 2000 + len(calls)))
        o = [L.libconv_out_size(n, k, p, st) for n, k, p, st in
             zip((l.T, l.H, l.W), (l.KT, l.KH, l.KW), l.pad, l.stride)]
        shape = (l.N, l.C_out) + (tuple(o[1:]) if l.dims == 2 else tuple(o))
        y = torch.empty(shape, dtype=x.dtype, device=dev)
        dt, act = W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act]
        dims = (l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH, l.KW)
        need = L.libconv_workspace_size(*dims, l.pad[0], l.pad[0], l.pad[1], l.pad[2],
                                        *l.stride, dt, act, L.ALGO_AUTO, 0)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        keep += [x, w, b, y, ws]
        p = (x.data_ptr(), w.data_ptr(), b.data_ptr(), y.data_ptr())
        if l.dims == 2:
            exp = (lambda p=p, l=l, dt=dt, act=act: L.conv2d_forward(
                *p, l.N, l.C_in, l.H, l.W, l.C_out, l.KH, l.KW, l.pad[1], l.pad[2], l.stride[1],
                l.stride[2], dt, act, s))
        else:
            exp = (lambda p=p, l=l, dt=dt, act=act, dims=dims: L.conv3d_forward(
                *p, *dims, *l.pad, *l.stride, dt, act, s))
        calls.append((f"{name} export", exp))
        calls.append((f"{name} workspace", lambda p=p, l=l, dt=dt, act=act, dims=dims,
                      ws=ws, need=need: L.conv3d_forward_ws(
                          *p, *dims, *l.pad, *l.stride, dt, act,
                          ws.data_ptr() if need > 0 else None, need, s)))
        if name == "c5_B":
            calls.append((f"{name} noalloc", lambda p=p, l=l, dt=dt, act=act, dims=dims:
                          L.conv3d_forward_noalloc(*p, *dims, *l.pad, *l.stride, dt, act, s)))
            pw = L.pack_weights(w)
            keep.append(pw)
            calls.append((f"{name} causal packed", lambda p=p, l=l, dt=dt, act=act, dims=dims,
                          pw=pw: L.conv3d_forward_tpad(
                              p[0], None, pw.data.data_ptr(), p[2], p[3], *dims, 2, 0, 1, 1,
                              *l.stride, dt, act, s)))
            xp = L.pack_activations(x)
            nb = L.libconv_cpack_bytes(l.N, l.C_out, *o, dt)
            yp = torch.empty(nb, dtype=torch.uint8, device=dev)
            keep += [xp, yp]
            calls.append((f"{name} channel-packed", lambda l=l, dt=dt, act=act, dims=dims,
                          pw=pw, xp=xp, yp=yp, b=b: L.conv3d_forward_cpack(
                              xp.data.data_ptr(), None, pw.data.data_ptr(), b.data_ptr(),
                              yp.data_ptr(), *dims, 1, 1, 1, 1, *l.stride, dt, act, s)))
    return calls, keep


def test_soak_ten_thousand_calls():
    import direct_implicit_gemm_amd as L
    dev = torch.device("cuda:0")
    calls, keep = _calls(L, dev)
    torch.cuda.synchronize()
    total = 10_000
    warm = len(calls) * 20
    samples = []
    for i in range(total):
        name, fn = calls[i % len(calls)]
        st = fn()
        assert st == 0, f"call {i} ({name}) returned {st}"
        if i == warm or (i > warm and i % 1000 == 0) or i == total - 1:
            torch.cuda.synchronize()
            free, _ = torch.cuda.mem_get_info(dev)
            samples.append((i, free, _rss_bytes()))
            note(f"call {i}: device free {free >> 20} MiB, host RSS {samples[-1][2] >> 20} MiB")
    torch.cuda.synchronize()
    free0, rss0 = samples[0][1], samples[0][2]
    for i, free, rss in samples[1:]:
        assert free >= free0, f"device memory fell by {free0 - free} bytes by call {i}"
        assert rss - rss0 < (16 << 20), f"host RSS grew by {rss - rss0} bytes by call {i}"
    del keep
