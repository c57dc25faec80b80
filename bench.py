"""Forward-convolution benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one pass of the workload's convolution layers over one batch of
synthetic input, every layer through libconv with OI(D)HW weights given on
every call.  The default workload is the largest configuration, the video-VAE
3-D convolutions in f16 (N=1, T=5: 3x3x3 128->128 on 256x480, and 3x3x3
512->512 on 64x120 +ReLU), 1087 effective GFLOP per step.

Timing (cold protocol, the primary figures): before every timed call a 512 MB
scratch buffer is written (evicting the 256 MB Infinity Cache and the L2s),
outside the event pair; one event pair on the launch stream brackets each call.
K steps (at least 20; layers under 10 us get at least 200 reps) give the median
and the minimum.  `ms_per_step` is the median cold step (the sum of its layers'
times), `value` = effective FLOP per step / that time.  Warm figures, labelled
as such: K steps back to back between one event pair, eagerly and as replays of
the step captured once as a HIP graph.

Per layer, three calls of the same convolution, each timed cold:
  * `step`: libconv_forward_ex with the OI(D)HW weights and the workspace
    libconv_workspace_size names (what conv3d_forward_ws / conv2d_forward_ws
    do): the weights are packed into the workspace on every call when the
    chosen kernel reads packed weights, and a split reduction keeps its
    partial sums there.  This is the call the step times.
  * `kernel`: the same call on weights packed beforehand, which runs the
    convolution kernel alone (plus the split-K sum when the plan splits):
    the `roofline` figures of the dominant layer come from it.
  * `export`: conv2d_forward / conv3d_forward themselves (no workspace: no
    per-call packing, no split).

Printed: ONE JSON line (see the keys below).  `cpu_baseline` is the fp64 oracle
timed on the host cores on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
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
FLUSH_MB = 512
SPIN_CYCLES = 300_000   # GPU spin after the scratch write (cycles of torch.cuda._sleep)

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
CHAINED = ("ocr_stack", "ocr_cpack_f32")


def time_pads(layer: W.Layer):
    """(before, after) padding of the frame axis."""
    return layer.pad[0], layer.pad[0] if layer.pad_t_back is None else layer.pad_t_back


def out_shape(layer: W.Layer, lib):
    return [lib.libconv_out_size2(layer.T, layer.KT, *time_pads(layer), layer.stride[0]),
            lib.libconv_out_size(layer.H, layer.KH, layer.pad[1], layer.stride[1]),
            lib.libconv_out_size(layer.W, layer.KW, layer.pad[2], layer.stride[2])]


def layer_work(layer: W.Layer, lib):
    """Effective FLOP (padded taps included) and algorithmic bytes (x, w, b, y once)."""
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
    csrc = os.path.join(ROOT, "direct_implicit_gemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".def")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, layer: str, tile_name: str):
    """HBM bytes per launch of a layer's kernel from committed rocprofv3 counter
    runs (profiles/traffic.json), if they were taken on the current kernel
    sources and the same kernel; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(workload, {}).get(layer)
    if not e or e.get("source_sha") != kernel_source_sha() or e.get("kernel") != tile_name:
        return None
    return e.get("bytes_per_launch")


def sp(l):
    return (l.stride[1:], l.pad[1:]) if l.dims == 2 else (l.stride, l.pad)


def cpu_baseline(layers, inputs, budget_s: float, chained: bool):
    """The oracle (as it stands, fp64, with its |x*w| pass) on a bounded sample
    of the step: for every layer, the same fraction of its output rows (all
    batches, channels, frames and columns), computed from the input rows they
    read; the fraction starts at about 2 GFLOP of work and is doubled (up to
    the whole step) while one pass takes under budget_s / 8, then the pass is
    repeated to about budget_s.  The rate is the effective FLOP of the outputs
    computed, over the time."""
    import oracle
    threads = oracle.threads(len(os.sched_getaffinity(0)))

    def sample(frac, build=True):
        jobs, flops, rows_taken = [], 0, []
        for layer, (x, w, b) in zip(layers, inputs):
            s_, p_ = sp(layer)
            sh, ph, kh = layer.stride[1], layer.pad[1], layer.KH
            oh_all = (layer.H + 2 * ph - kh) // sh + 1
            rows = max(1, int(round(oh_all * frac)))
            h_in = min(layer.H, (rows - 1) * sh + kh - ph)   # rows those outputs read
            pf, pb = time_pads(layer)
            o_t = (layer.T + pf + pb - layer.KT) // layer.stride[0] + 1 if layer.dims == 3 else 1
            o_h = (h_in + 2 * ph - kh) // sh + 1
            o_w = (layer.W + 2 * layer.pad[2] - layer.KW) // layer.stride[2] + 1
            flops += 2 * layer.N * layer.C_out * o_t * o_h * o_w * layer.C_in * layer.taps
            rows_taken.append(f"{layer.name}: {o_h} of {oh_all} rows")
            if build:
                xs = W.Tensor(x.dtype, np.ascontiguousarray(x.storage[..., :h_in, :])).f64()
                jobs.append((layer, xs, w.f64(), b.f64(), s_, p_))
        return jobs, flops, rows_taken

    def run(jobs):
        for layer, xs, w, b, s_, p_ in jobs:
            y, _ = oracle.conv(xs, w, b, s_, p_, relu=layer.act == "relu",
                               pad_t_back=layer.pad_t_back)
            if layer.pool:
                oracle.max_pool2x2(y)

    _, whole, _ = sample(1.0, build=False)
    frac = min(1.0, 2e9 / max(whole, 1))
    while True:
        jobs, flops, rows_taken = sample(frac)
        t0 = time.perf_counter()
        run(jobs)
        one = time.perf_counter() - t0
        if one >= budget_s / 8 or frac >= 1.0:
            break
        frac = min(1.0, frac * 2)
    runs, t0 = 0, time.perf_counter()
    while True:
        run(jobs)
        runs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    note = (f"the first output rows of every layer ({'; '.join(rows_taken)}; all batches, "
            f"channels, frames, columns; {flops / 1e9:.2f} effective GFLOP per pass), fp64 with "
            f"the |x*w| sum, {runs} pass(es) in {el:.1f} s")
    return flops * runs / el, threads, note


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


class LayerCalls:
    """The three calls of one layer (step / kernel / export) on device tensors."""

    def __init__(self, L, lib, torch, dev, layer, x, w, b):
        self.L, self.lib, self.torch, self.layer = L, lib, torch, layer
        l = layer
        self.dt, self.act = W.DTYPE_CODE[l.dtype], W.ACT_CODE[l.act]
        self.flags = (L.PLAN_POOL2 if l.pool else 0) | (L.PLAN_CPACK if l.cpack else 0)
        pf, pb = time_pads(l)
        self.dims = (l.N, l.C_in, l.T, l.H, l.W, l.C_out, l.KT, l.KH, l.KW)
        self.pads = (pf, pb, l.pad[1], l.pad[2])
        self.strides = tuple(l.stride)
        self.x = L.pack_activations(x.torch(dev)) if l.cpack else x.torch(dev)
        self.xp = self.x.data.data_ptr() if l.cpack else self.x.data_ptr()
        self.w = w.torch(dev)
        self.b = b.torch(dev)
        ot, oh, ow = out_shape(l, lib)
        if l.pool:
            oh, ow = oh // 2, ow // 2
        shape = (l.N, l.C_out, oh, ow) if l.dims == 2 else (l.N, l.C_out, ot, oh, ow)
        if l.cpack:
            nb = lib.libconv_cpack_bytes(l.N, l.C_out, ot, oh, ow, self.dt)
            self.y = L.PackedActivations(torch.empty(nb, dtype=torch.uint8, device=dev), shape,
                                         self.x.dtype)
            self.yp = self.y.data.data_ptr()
        else:
            self.y = torch.empty(shape, dtype=self.x.dtype, device=dev)
            self.yp = self.y.data_ptr()
        self.ws_n = lib.libconv_workspace_size(*self.dims, *self.pads, *self.strides, self.dt,
                                               self.act, L.ALGO_AUTO, self.flags)
        assert self.ws_n >= 0, l.name
        self.ws = torch.empty(max(self.ws_n, 1), dtype=torch.uint8, device=dev)
        self.plan_step = self.plan(self.ws_n, packed=False)
        # The kernel-only call: weights packed once beforehand (as a runtime
        # with fixed weights does), when the layer has a tile that reads
        # packed weights; else the step's own call.
        self.packed = None
        self.plan_kernel = self.plan_step
        kw_n = lib.libconv_workspace_size(*self.dims, *self.pads, *self.strides, self.dt,
                                          self.act, L.ALGO_AUTO, self.flags | L.PLAN_PACKED_W)
        if kw_n >= 0:
            kws_n = max(kw_n, 0)
            plan_k = self.plan(kws_n, packed=True, must=False)
            if plan_k is not None and L.libconv_tile_name(plan_k[1]).startswith(
                    ("igemm16p", "igemm32p", "igemm16x_", "igemm32x_")):
                self.packed = L.pack_weights(self.w)
                self.kws_n = kws_n
                self.kws = torch.empty(max(self.kws_n, 1), dtype=torch.uint8, device=dev)
                self.plan_kernel = plan_k
        self.plan_export = self.plan(0, packed=False)

    def plan(self, ws_bytes, packed, must=True):
        l = self.layer
        pad = (sum(self.pads[:2]) // 2,) + self.pads[2:]   # the query takes one time pad
        st, algo, tile, grid, ks = self.L.libconv_query_plan(
            *self.dims, *pad, *self.strides, self.dt, self.act, self.L.ALGO_AUTO,
            self.flags | (self.L.PLAN_PACKED_W if packed else 0), ws_bytes)
        if st != 0 and not must:
            return None
        assert st == 0, (l.name, st)
        return algo, tile, grid, ks

    def _ex(self, x_ptr, w_ptr, pw_ptr, ws, ws_n, stream):
        st = self.lib.libconv_forward_ex(x_ptr, w_ptr, pw_ptr, self.b.data_ptr(), self.yp,
                                         *self.dims, *self.pads, *self.strides, self.dt,
                                         self.act, self.L.ALGO_AUTO, self.flags, ws, ws_n,
                                         stream)
        if st != 0:
            raise self.L.LibconvError(st, f"{self.layer.name} libconv_forward_ex")

    def step(self, stream, x_ptr=None):
        self._ex(x_ptr or self.xp, self.w.data_ptr(), None,
                 self.ws.data_ptr() if self.ws_n > 0 else None, self.ws_n, stream)

    def kernel(self, stream):
        if self.packed is None:
            return self.step(stream)
        self._ex(self.xp, None, self.packed.data.data_ptr(),
                 self.kws.data_ptr() if self.kws_n > 0 else None, self.kws_n, stream)

    def export(self, stream):
        l = self.layer
        if l.cpack or l.pool or l.pad_t_back is not None:
            self._ex(self.xp, self.w.data_ptr(), None, None, 0, stream)
            return
        if l.dims == 2:
            st = self.lib.conv2d_forward(self.xp, self.w.data_ptr(), self.b.data_ptr(), self.yp,
                                         l.N, l.C_in, l.H, l.W, l.C_out, l.KH, l.KW, l.pad[1],
                                         l.pad[2], l.stride[1], l.stride[2], self.dt, self.act,
                                         stream)
        else:
            st = self.lib.conv3d_forward(self.xp, self.w.data_ptr(), self.b.data_ptr(), self.yp,
                                         *self.dims, *l.pad, *l.stride, self.dt, self.act,
                                         stream)
        if st != 0:
            raise self.L.LibconvError(st, f"{l.name} conv_forward")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="vae3d_f16", choices=sorted(ALL_WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-graph", action="store_true", help="skip the warm graph-replay figures")
    ap.add_argument("--no-export", action="store_true",
                    help="skip timing the no-workspace export calls")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
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
        print("bench.py measures one GPU only: this library has no multi-GPU path "
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
    chained = args.workload in CHAINED
    inputs = [W.make_inputs(l) for l in layers]
    calls = [LayerCalls(L, lib, torch, dev, l, *inp) for l, inp in zip(layers, inputs)]
    scratch = torch.empty(FLUSH_MB << 20, dtype=torch.uint8, device=dev)

    def x_of(i):  # a chained stack feeds each layer the previous layer's output
        return calls[i - 1].yp if (chained and i > 0) else None

    def step_eager(stream):
        for i, c in enumerate(calls):
            c.step(stream, x_of(i))

    stream = torch.cuda.current_stream(dev).cuda_stream   # the stream libconv launches on
    for _ in range(args.warmup):
        step_eager(stream)
        for c in calls:
            c.kernel(stream)
            if not args.no_export:
                c.export(stream)
    torch.cuda.synchronize()

    Ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def evict():
        """The cold protocol's scratch write, then a GPU spin of about 150 us:
        both outside the event pair.  The spin keeps the GPU busy while the host
        enqueues the first event and the call, so that the event pair times the
        GPU's work and not the host's enqueue latency (a workspace call's pack
        and convolution kernels otherwise showed 7-20 us of idle GPU between
        them and the first event)."""
        scratch.zero_()
        torch.cuda._sleep(SPIN_CYCLES)

    def cold(fn, reps):
        """reps timed calls of fn, each after the scratch write, events on the
        launch stream; returns the per-call times in microseconds."""
        pairs = []
        for _ in range(reps):
            evict()                               # outside the event pair
            e0, e1 = Ev(), Ev()
            e0.record()
            fn()
            e1.record()
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        return [1000.0 * a.elapsed_time(b) for a, b in pairs]

    K = max(args.steps, 20)
    # ---- the timed steps (cold): each layer's call after its own scratch write
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    step_pairs = []
    for _ in range(K):
        lp = []
        for i, c in enumerate(calls):
            evict()
            e0, e1 = Ev(), Ev()
            e0.record()
            c.step(stream, x_of(i))
            e1.record()
            lp.append((e0, e1))
        step_pairs.append(lp)
    torch.cuda.synchronize()
    wall_timed = time.perf_counter() - wall0
    layer_step_us = [[1000.0 * p[i][0].elapsed_time(p[i][1]) for p in step_pairs]
                     for i in range(len(calls))]
    step_us = [sum(layer_step_us[i][k] for i in range(len(calls))) for k in range(K)]
    ms_per_step = statistics.median(step_us) / 1000.0

    # ---- per layer: more reps for short layers; kernel-only and export calls
    per_layer = []
    step_flops = 0
    for i, c in enumerate(calls):
        us_step = layer_step_us[i]
        if statistics.median(us_step) < 10.0 and K < 200:
            us_step = us_step + cold(lambda: c.step(stream, x_of(i)), 200 - K)
        us_kernel = us_step if c.packed is None else cold(lambda: c.kernel(stream), len(us_step))
        us_export = None if args.no_export else cold(lambda: c.export(stream), len(us_step))
        # warm: the same call back to back
        for _ in range(3):
            c.step(stream, x_of(i))
        torch.cuda.synchronize()
        e0, e1 = Ev(), Ev()
        e0.record()
        for _ in range(K):
            c.step(stream, x_of(i))
        e1.record()
        torch.cuda.synchronize()
        warm_b2b = 1000.0 * e0.elapsed_time(e1) / K
        flops, nbytes = layer_work(c.layer, lib)
        step_flops += flops
        med_k = statistics.median(us_kernel)
        bound, tflops, gbs, frac = roofline_of(c.layer, flops, nbytes, med_k * 1e-6)
        med_s = statistics.median(us_step)
        _, tf_s, gb_s, fr_s = roofline_of(c.layer, flops, nbytes, med_s * 1e-6)
        ent = {
            "layer": c.layer.name,
            "kernel": L.libconv_tile_name(c.plan_kernel[1]), "grid": c.plan_kernel[2],
            "ksplit": c.plan_kernel[3],
            "kernel_us_median": round(med_k, 3), "kernel_us_min": round(min(us_kernel), 3),
            "kernel_reps": len(us_kernel),
            "tflops": round(tflops, 3), "gbs": round(gbs, 1), "bound": bound,
            "frac": round(frac, 4),
            "step_call": ("OI(D)HW weights + workspace (" +
                          ("weights packed on the call, " if c.packed is not None else "") +
                          f"{c.ws_n} bytes)"),
            "step_kernel": L.libconv_tile_name(c.plan_step[1]), "step_ksplit": c.plan_step[3],
            "step_us_median": round(med_s, 3), "step_us_min": round(min(us_step), 3),
            "step_frac": round(fr_s, 4),
            "warm_b2b_us": round(warm_b2b, 3),
            "gflop": round(flops / 1e9, 4), "mbytes": round(nbytes / 1e6, 3),
        }
        if us_export is not None:
            me = statistics.median(us_export)
            ent.update({"export_kernel": L.libconv_tile_name(c.plan_export[1]),
                        "export_us_median": round(me, 3), "export_us_min": round(min(us_export), 3),
                        "export_frac": round(roofline_of(c.layer, flops, nbytes, me * 1e-6)[3], 4)})
        per_layer.append(ent)

    # ---- warm steps: eager back to back, and replays of the step as a HIP graph
    e0, e1 = Ev(), Ev()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        step_eager(stream)
    e1.record()
    torch.cuda.synchronize()
    warm_eager = e0.elapsed_time(e1) / K
    warm_graph, graph_note = None, "off"
    if not args.no_graph:
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step_eager(torch.cuda.current_stream(dev).cuda_stream)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(K):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            warm_graph, graph_note = e0.elapsed_time(e1) / K, "captured"
            del g
        except Exception as e:  # a call that cannot be captured: no graph figure
            graph_note = f"capture failed ({type(e).__name__}: {e})"
            torch.cuda.synchronize()

    dom = max(range(len(calls)), key=lambda i: per_layer[i]["kernel_us_median"])
    dl = per_layer[dom]
    flops, nbytes = layer_work(layers[dom], lib)
    if dl["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dl["tflops"], "peak": PEAK_TFLOPS[layers[dom].dtype],
                "unit": "TFLOP/s", "frac": dl["frac"]}
    else:
        roof = {"bound": "hbm", "achieved": dl["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": dl["frac"]}
    roof["traffic"] = measured_traffic(args.workload, dl["layer"], dl["kernel"])
    roof.update({"layer": dl["layer"], "kernel": dl["kernel"],
                 "algorithmic": flops if dl["bound"] == "mfma" else nbytes,
                 "algorithmic_unit": "FLOP per launch" if dl["bound"] == "mfma"
                 else "bytes per launch",
                 "duration_us_median_cold": dl["kernel_us_median"],
                 "timing": "hipEvents on the launch stream around each call, cold protocol"})

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu:
        rate, threads, note = cpu_baseline(layers, inputs, args.cpu_budget, chained)
        cpu = {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle", "sample": note,
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
                   "chained": chained,
                   "timing": f"cold: {FLUSH_MB} MB scratch write and a GPU spin (the host "
                             "enqueues the call meanwhile) before each call, outside the event "
                             "pair; ms_per_step = median over steps of the summed layer times",
                   "ms_per_step_min": round(min(step_us) / 1000.0, 5),
                   "warm_ms_per_step_eager": round(warm_eager, 5),
                   "warm_ms_per_step_graph": None if warm_graph is None else round(warm_graph, 5),
                   "graph": graph_note,
                   "wall_s_timed": round(wall_timed, 4)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layers": per_layer,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
