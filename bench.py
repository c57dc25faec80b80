"""Forward-convolution benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one pass of the workload's convolution layers over one batch of
synthetic input, chained on the GPU (layer k reads layer k-1's output), with
every layer through libconv.  The default workload is the fp32 OCR-detection
stack (N=1, 3x640x640; conv3x3/s2 3->32 +ReLU, conv3x3 32->32 +ReLU,
conv1x1 32->64 +ReLU, conv3x3/s2 64->64 +ReLU).

Printed: ONE JSON line.  ``value`` is the step's effective TFLOP/s
(2*N*C_out*out_spatial*C_in*taps summed over layers, divided by the time of a
step); per-layer figures (µs, TFLOP/s, GB/s, binding roofline and fraction)
are in ``layers``; ``roofline`` describes the layer whose kernel takes the most
time; ``cpu_baseline`` is the fp64 oracle timed on the host cores.

The step is timed twice, K eager steps and K replays of the step captured
once as a HIP graph (no host launch overhead; ``--no-graph`` skips it), and
the faster is reported (``config.step_mode``; both times are in ``config``).
Per-layer times: ``us_b2b``, one event pair around R back-to-back launches of
the layer alone, divided by R (for short kernels this is bounded by the host's
call rate); ``us_graph``, the same R launches captured once as a HIP graph and
replayed between one event pair (no host in the timed region; only when the
call plans the same kernel under capture).  ``us`` is the smaller, and the
roofline fractions use it; it matches the kernel durations of a rocprofv3
kernel trace.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}   # dense MFMA
METRIC = "conv fwd effective TFLOP/s + HBM GB/s per layer, % of binding MI355X roofline"

WORKLOAD_TEXT = {
    "conv1": "single conv2d fp32 N=1 3x32x32 -> 8, 3x3 s1 p1, bias",
    "ocr_stack": ("OCR-detection fp32 stack N=1 3x640x640: conv3x3 s2 p1 3->32 +ReLU, "
                  "conv3x3 s1 p1 32->32 +ReLU, conv1x1 32->64 +ReLU, conv3x3 s2 p1 64->64 +ReLU"),
    "textrec_f16": ("text-recognition f16 N=16: conv3x3 64->128 on 24x160 +ReLU; "
                    "conv1x1 128->256 on 12x80"),
    "unet_bf16": "diffusion-UNet bf16 N=2: conv3x3 640->640 on 64x64; conv3x3 1280->1280 on 32x32",
    "vae3d_f16": ("video-VAE f16 conv3d N=1 T=5: 3x3x3 128->128 on 256x480; "
                  "3x3x3 512->512 on 64x120 +ReLU"),
    "ocr_pool_f32": ("OCR-detector conv3x3 s1 p1 32->32 +ReLU +2x2 max pool (fused) on 1x32x320x320 "
                     "-> 1x32x160x160, fp32"),
    "vae3d_causal_f16": ("video-VAE f16 causal conv3d N=1 T=5 (2 frames of time padding "
                         "before the first frame, none after): 3x3x3 128->128 on 256x480; "
                         "3x3x3 512->512 on 64x120 +ReLU"),
    "vae3d_cpack_f16": ("the video-VAE f16 conv3d layers on channel-packed activations "
                        "([N][C/8][T][H][W][8], packed once before timing)"),
    "ocr_cpack_f32": ("the OCR-detection fp32 stack (chained) on channel-packed activations "
                      "([N][C/4][H][W][4]) and packed weights, both packed once before timing"),
    "unet_cpack_bf16": ("the diffusion-UNet bf16 layers on channel-packed activations "
                        "([N][C/8][H][W][8], packed once before timing)"),
}
ALL_WORKLOADS = {**W.WORKLOADS, **W.EXTRA_WORKLOADS}


def time_pads(layer: W.Layer):
    """(before, after) padding of the frame axis."""
    return layer.pad[0], layer.pad[0] if layer.pad_t_back is None else layer.pad_t_back


def out_shape(layer: W.Layer, lib):
    o = [lib.libconv_out_size2(layer.T, layer.KT, *time_pads(layer), layer.stride[0]),
         lib.libconv_out_size(layer.H, layer.KH, layer.pad[1], layer.stride[1]),
         lib.libconv_out_size(layer.W, layer.KW, layer.pad[2], layer.stride[2])]
    return o


def layer_work(layer: W.Layer, lib):
    ot, oh, ow = out_shape(layer, lib)
    out_spatial = ot * oh * ow
    flops = 2 * layer.N * layer.C_out * out_spatial * layer.C_in * layer.taps
    stored = ot * (oh // 2) * (ow // 2) if layer.pool else out_spatial  # fused pooling
    e = W.DTYPE_BYTES[layer.dtype]
    nbytes = e * (int(np.prod(layer.x_shape)) + int(np.prod(layer.w_shape)) + layer.C_out
                  + layer.N * layer.C_out * stored)
    return flops, nbytes


def roofline_of(layer, flops, nbytes, seconds):
    t_mfma = flops / (PEAK_TFLOPS[layer.dtype] * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    tflops = flops / seconds / 1e12
    gbs = nbytes / seconds / 1e9
    frac = (tflops / PEAK_TFLOPS[layer.dtype]) if bound == "mfma" else (gbs / PEAK_HBM_GBS)
    return bound, tflops, gbs, frac


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("direct.hip", "igemm.hip", "device_common.h"):
        with open(os.path.join(ROOT, "direct_implicit_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, layer: str, tile_name: str):
    """HBM bytes per launch of a layer from committed rocprofv3 counter runs
    (profiles/traffic.json), if they were taken on the current kernel sources
    and the same kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(workload, {}).get(layer)
    if not e or e.get("source_sha") != kernel_source_sha() or e.get("kernel") != tile_name:
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(layers, inputs, budget_s: float):
    """The oracle (as it stands) on the same step, repeated to ~budget_s."""
    import oracle
    threads = oracle.threads(len(os.sched_getaffinity(0)))
    total_flops = 0
    runs = 0
    t0 = time.perf_counter()
    while True:
        x = inputs[0][0].f64()
        for layer, (_, w, b) in zip(layers, inputs):
            st, pd = (layer.stride[1:], layer.pad[1:]) if layer.dims == 2 else (layer.stride, layer.pad)
            y, _ = oracle.conv(x, w.f64(), b.f64(), st, pd, relu=layer.act == "relu")
            x = W.Tensor.quantise(y, layer.dtype).f64()
        runs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return el / runs, threads, runs


def long_video(args, torch, L, dev):
    """A long causal clip through one video-VAE layer (128 -> 128 channels,
    3x3x3, 256x480, f16): the whole clip on the device against the chunked
    driver, from device memory and from pinned host memory (two copy
    streams), with the plain whole-tensor host copies for scale.  Times are
    means over --steps calls after --warmup, by events on the current stream
    (which the chunked driver makes wait for its copies)."""
    T = args.long_video
    layer = W.ALL_LAYERS["c5_A"].with_(T=T, pad=(2, 1, 1))
    x, w, b = W.make_inputs(layer, 17)
    wq = L.pack_weights(w.torch(dev))
    bt = b.torch(dev)
    xd = x.torch(dev)
    shape = (1, 128, T, 256, 480)
    yd = torch.empty(shape, dtype=torch.float16, device=dev)
    xh = torch.empty(x.shape, dtype=torch.float16, pin_memory=True)
    xh.copy_(x.torch("cpu"))
    yh = torch.empty(shape, dtype=torch.float16, pin_memory=True)
    # effective work: taps on frames inside the clip only
    frame_taps = sum(1 for o in range(T) for kt in range(3) if 0 <= o - 2 + kt < T)
    flop = 2.0 * 128 * 128 * 9 * 256 * 480 * frame_taps

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(args.steps):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / args.steps

    c = args.chunk
    ms = {
        "whole_device": timed(lambda: L.conv3d_tpad(xd, wq, bt, (2, 0), 1, 1, out=yd)),
        "chunked_device": timed(lambda: L.conv3d_chunked(xd, wq, bt, c, (2, 0), 1, 1, out=yd)),
        "chunked_host_pinned": timed(lambda: L.conv3d_chunked(xh, wq, bt, c, (2, 0), 1, 1,
                                                              out=yh)),
        "copy_x_host_to_device": timed(lambda: xd.copy_(xh, non_blocking=True)),
        "copy_y_device_to_host": timed(lambda: yh.copy_(yd, non_blocking=True)),
    }
    print(json.dumps({
        "long_video": {"frames": T, "chunk_out_frames": c, "layer": "128->128 3x3x3 256x480 f16, "
                       "time pads (2, 0)", "effective_gflop": round(flop / 1e9, 1),
                       "tensor_mb": round(x.storage.nbytes / 1e6, 1)},
        "ms": {k: round(v, 3) for k, v in ms.items()},
        "tflops_effective": {k: round(flop / v / 1e9, 1) for k, v in ms.items()
                             if not k.startswith("copy")},
        "note": "host-pinned rates include both PCIe directions; not the bench value"}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ocr_stack", choices=sorted(ALL_WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager steps instead of replays of the step captured as a HIP graph")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the workload, copy MIB MiB device-to-device --steps times "
                         "(a plain copy of known size, to scale HBM byte counters)")
    ap.add_argument("--long-video", type=int, default=0, metavar="FRAMES",
                    help="instead of the workload, the video-VAE 128-channel causal layer over "
                         "FRAMES frames: whole on the device, and streamed in chunks of "
                         "--chunk output frames from device and from pinned host memory")
    ap.add_argument("--chunk", type=int, default=3)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import direct_implicit_gemm_amd as L

    lib = L.load()
    if L.libconv_device_supported(0) != 0:
        print("cuda:0 is not a gfx950 device", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                          "copies": args.steps,
                          "GBps_read_plus_write": round(2 * n * 4 * args.steps / el / 1e9, 1)}))
        return

    if args.long_video:
        long_video(args, torch, L, dev)
        return

    _, layers = ALL_WORKLOADS[args.workload]
    # Inputs: the workload's seeded tensors; the stack is chained, so only the
    # first layer's x is used when layers feed each other.
    inputs = [W.make_inputs(l) for l in layers]
    chained = args.workload in ("ocr_stack", "ocr_cpack_f32")
    xs, ws, bs = [], [], []
    for l, (x, w, b) in zip(layers, inputs):
        # channel-packed layers: the network is kept in the packed form, so the
        # input is packed once at its edge, before timing; prepacked layers
        # get their weights packed once at load (as the pages reorder weights
        # at export / load), the others pass OI(D)HW weights on every call
        xs.append(L.pack_activations(x.torch(dev)) if l.cpack else x.torch(dev))
        ws.append(L.pack_weights(w.torch(dev)) if l.prepacked else w.torch(dev))
        bs.append(b.torch(dev))
    outs = []
    for i, l in enumerate(layers):
        ot, oh, ow = out_shape(l, lib)
        if l.pool:
            oh, ow = oh // 2, ow // 2
        shape = (l.N, l.C_out, oh, ow) if l.dims == 2 else (l.N, l.C_out, ot, oh, ow)
        if l.cpack:
            nb = lib.libconv_cpack_bytes(l.N, l.C_out, ot, oh, ow, W.DTYPE_CODE[l.dtype])
            outs.append(L.PackedActivations(torch.empty(nb, dtype=torch.uint8, device=dev),
                                            shape, xs[i].dtype))
        else:
            outs.append(torch.empty(shape, dtype=xs[i].dtype, device=dev))

    def sp(l):
        return (l.stride[1:], l.pad[1:]) if l.dims == 2 else (l.stride, l.pad)

    def conv(l, x_in, w, b, out):
        if l.cpack:  # channel-packed activations in and out
            s, p = sp(l)
            L.conv_cpack(x_in, w, b, s, p, time_pads(l) if l.dims == 3 else None, l.act, out=out)
        elif l.pool:  # conv + activation + 2x2 max pool in one call
            L.conv2d_pool(x_in, w, b, l.stride[1:], l.pad[1:], l.act, out=out)
        elif l.pad_t_back is not None:  # time padding differs before / after the frames
            L.conv3d_tpad(x_in, w, b, time_pads(l), l.stride, l.pad[1:], l.act, out=out)
        else:
            s, p = sp(l)
            L.conv_nd(x_in, w, b, s, p, l.act, out=out)

    def step():
        for i, l in enumerate(layers):
            x_in = outs[i - 1] if (chained and i > 0) else xs[i]
            conv(l, x_in, ws[i], bs[i], outs[i])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # The step as a HIP graph (captured once through torch's graph capture, on
    # torch's capture stream, which is the stream libconv launches on): a
    # replay issues the layers back to back without host launch overhead.
    # Under capture libconv plans without temporaries (no split-K, no weight
    # packing per call), which can be slower for some layers, so both the
    # eager step and the replayed step are timed over K steps and the faster
    # is reported (both are in `config`).
    graph, graph_note = None, "off"
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            graph, graph_note = g, "captured"
        except Exception as e:  # a layer whose call cannot be captured: eager steps
            graph, graph_note = None, f"capture failed ({type(e).__name__})"
            torch.cuda.synchronize()

    K = args.steps

    def timed(run_one):
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        t_start.record()
        for _ in range(K):
            run_one()
        t_end.record()
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / K, time.perf_counter() - w0

    ms_eager, wall_eager = timed(step)
    ms_graph, wall_graph = timed(graph.replay) if graph is not None else (None, None)
    if ms_graph is not None and ms_graph < ms_eager:
        ms_per_step, wall, mode = ms_graph, wall_graph, "graph replay"
    else:
        ms_per_step, wall, mode = ms_eager, wall_eager, "eager"

    # Each layer alone, R launches back to back, timed two ways on the launch
    # stream: (1) issued eagerly between one event pair -- for short kernels
    # this is bounded by the host's call rate (Python, ctypes, planning,
    # launch); (2) the same R launches captured once as a HIP graph and
    # replayed between one event pair, which removes the host from the timed
    # region.  (2) is taken only when the call plans the same kernel under
    # capture as eagerly (libconv_query_plan), so both time one kernel.
    R = max(10, K)
    GRAPH_REPLAYS = 3

    def plan_of(l, capturing):
        # the query takes one time pad: one-sided padding is asked as the
        # symmetric padding with the same number of output frames
        pad = (sum(time_pads(l)) // 2,) + tuple(l.pad[1:])
        st_, algo, tile, grid, ks = L.libconv_query_plan(
            l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH, l.KW, *pad, *l.stride,
            W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act], L.ALGO_AUTO,
            (L.PLAN_CAPTURING if capturing else 0) | (L.PLAN_POOL2 if l.pool else 0)
            | (L.PLAN_CPACK if l.cpack else 0) | (L.PLAN_PACKED_W if l.prepacked else 0))
        return algo, tile, grid, ks

    b2b, b2b_graph = [], []
    for i, l in enumerate(layers):
        x_in = outs[i - 1] if (chained and i > 0) else xs[i]

        def launch_r():
            for _ in range(R):
                conv(l, x_in, ws[i], bs[i], outs[i])

        conv(l, x_in, ws[i], bs[i], outs[i])
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        launch_r()
        e1.record()
        torch.cuda.synchronize()
        b2b.append(1000.0 * e0.elapsed_time(e1) / R)
        ug = None
        if not args.no_graph and plan_of(l, False) == plan_of(l, True):
            try:
                gl = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gl):
                    launch_r()
                gl.replay()
                torch.cuda.synchronize()
                e0.record()
                for _ in range(GRAPH_REPLAYS):
                    gl.replay()
                e1.record()
                torch.cuda.synchronize()
                ug = 1000.0 * e0.elapsed_time(e1) / (R * GRAPH_REPLAYS)
                del gl
            except Exception:  # capture refused: keep the eager figure
                torch.cuda.synchronize()
                ug = None
        b2b_graph.append(ug)

    per_layer = []
    step_flops = 0
    for i, l in enumerate(layers):
        ue, ug = b2b[i], b2b_graph[i]
        us, mode = (ug, "graph") if ug is not None and ug < ue else (ue, "eager")
        flops, nbytes = layer_work(l, lib)
        step_flops += flops
        bound, tflops, gbs, frac = roofline_of(l, flops, nbytes, us * 1e-6)
        algo, tile, grid, ks = plan_of(l, False)
        per_layer.append({
            "layer": l.name, "kernel": L.libconv_tile_name(tile), "grid": grid, "ksplit": ks,
            "us": round(us, 3), "timing": mode,
            "us_b2b": round(ue, 3), "us_graph": None if ug is None else round(ug, 3),
            "b2b_reps": R,
            "gflop": round(flops / 1e9, 4), "mbytes": round(nbytes / 1e6, 3),
            "tflops": round(tflops, 3), "gbs": round(gbs, 1),
            "bound": bound, "frac": round(frac, 4),
        })

    dom = max(range(len(layers)), key=lambda i: per_layer[i]["us"])
    dl = per_layer[dom]
    flops, nbytes = layer_work(layers[dom], lib)
    if dl["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dl["tflops"], "peak": PEAK_TFLOPS[layers[dom].dtype],
                "unit": "TFLOP/s", "frac": dl["frac"]}
    else:
        roof = {"bound": "hbm", "achieved": dl["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": dl["frac"]}
    traffic = measured_traffic(args.workload, dl["layer"], dl["kernel"])
    roof["traffic"] = traffic
    roof["layer"] = dl["layer"]
    roof["kernel"] = dl["kernel"]
    roof["algorithmic"] = flops if dl["bound"] == "mfma" else nbytes

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu:
        sec, threads, runs = cpu_baseline(layers, inputs, args.cpu_budget) if chained else (None, None, None)
        if sec is None:  # unchained workloads: each layer on its own input
            import oracle
            threads = oracle.threads(len(os.sched_getaffinity(0)))
            t0 = time.perf_counter()
            runs = 0
            while True:  # whole steps, repeated to about the CPU budget
                for l, (x, w, b) in zip(layers, inputs):
                    s, p = sp(l)
                    y, _ = oracle.conv(x.f64(), w.f64(), b.f64(), s, p, relu=l.act == "relu",
                                       pad_t_back=l.pad_t_back)
                    if l.pool:
                        oracle.max_pool2x2(y)
                runs += 1
                if time.perf_counter() - t0 >= args.cpu_budget:
                    break
            sec = (time.perf_counter() - t0) / runs
        cpu = {"value": round(step_flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the whole step ({len(layers)} layers, fp64, incl. the |x*w| sum), "
                         f"{runs} run(s), {sec:.3f} s per step",
               "cpu": platform.processor() or platform.machine()}

    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": layers[0].dtype,
        "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": args.workload, "description": WORKLOAD_TEXT[args.workload],
                   "chained": chained, "step_mode": mode, "graph": graph_note,
                   "ms_per_step_eager": round(ms_eager, 5),
                   "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 5),
                   "wall_s_timed": round(wall, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layers": per_layer,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
