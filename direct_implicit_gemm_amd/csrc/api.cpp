// api.cpp -- the exported C ABI of libconv: argument validation, output
// extents, the shape-driven dispatcher and the launch.
//
// Error conventions follow the fault-tolerant backend bring-up of the page
// "OpenCL-101 issue 52" (githubissues.com/ysh329/OpenCL-101/52): nothing here
// aborts; every failure is a status the caller can inspect, and whether the
// device is usable is a query (libconv_device_supported).  Unsupported shapes
// are reported, never silently sent elsewhere (the page "SeedVR2 NCNN
// Vulkan", section 3.6, on a Convolution3D that fell back to the CPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "internal.h"
#include "libconv.h"

namespace libconv {
namespace {

// Byte offsets are 32-bit signed in the kernels, and an offset of 0x7ffffff0
// or more must lie past the end of every tensor (that is how they read zeros).
constexpr long long kMaxBytes = 0x7fff0000LL;

// a * b, saturated well below overflow (every factor here is a non-negative int)
long long mul_sat(long long a, long long b) {
  constexpr long long kCap = 1LL << 62;
  if (a == 0 || b == 0) return 0;
  if (a > kCap / b) return kCap;
  return a * b;
}

long long product(std::initializer_list<long long> v) {
  long long r = 1;
  for (long long f : v) r = mul_sat(r, f);
  return r;
}

// Output positions with pad_lo before and pad_hi after the input.
long long out_extent2(long long in, long long k, long long pad_lo, long long pad_hi,
                      long long stride) {
  if (in < 1 || k < 1 || pad_lo < 0 || pad_hi < 0 || stride < 1) return -1;
  const long long span = in + pad_lo + pad_hi - k;
  if (span < 0) return -1;
  return span / stride + 1;
}

long long out_extent(long long in, long long k, long long pad, long long stride) {
  return out_extent2(in, k, pad, pad, stride);
}

bool overlaps(const void* a, long long abytes, const void* b, long long bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Checks everything that can be checked without a GPU and fills the output
// extents.  Pointers are only checked when `with_pointers` is set.
libconv_status validate(Problem& p, int algo, bool with_pointers) {
  if (p.dtype != LIBCONV_F32 && p.dtype != LIBCONV_F16 && p.dtype != LIBCONV_BF16)
    return LIBCONV_ERR_BAD_DTYPE;
  if (p.act != LIBCONV_ACT_NONE && p.act != LIBCONV_ACT_RELU) return LIBCONV_ERR_BAD_ACTIVATION;
  if (algo != LIBCONV_ALGO_AUTO && algo != LIBCONV_ALGO_DIRECT && algo != LIBCONV_ALGO_IGEMM)
    return LIBCONV_ERR_BAD_ALGO;
  if (p.N < 0 || p.C < 1 || p.T < 1 || p.H < 1 || p.W < 1 || p.K < 1 || p.KT < 1 || p.KH < 1 ||
      p.KW < 1)
    return LIBCONV_ERR_BAD_SHAPE;
  const long long ot = out_extent2(p.T, p.KT, p.pt, p.ptb, p.st);
  const long long oh = out_extent(p.H, p.KH, p.ph, p.sh);
  const long long ow = out_extent(p.W, p.KW, p.pw, p.sw);
  if (ot < 1 || oh < 1 || ow < 1) return LIBCONV_ERR_BAD_SHAPE;
  if (ot > 0x7fffffff || oh > 0x7fffffff || ow > 0x7fffffff) return LIBCONV_ERR_TOO_LARGE;
  p.OT = (int)ot;
  p.OH = (int)oh;
  p.OW = (int)ow;
  if (p.pool && (p.T != 1 || p.KT != 1 || oh < 2 || ow < 2)) return LIBCONV_ERR_BAD_SHAPE;
  if (p.cpack && p.pool) return LIBCONV_ERR_UNSUPPORTED;
  const long long eb = dtype_bytes(p.dtype);
  // channel-packed tensors hold whole 16-byte groups of channels
  const long long se = 16 / eb;
  const long long cx = p.cpack ? (p.C + se - 1) / se * se : p.C;
  const long long cy = p.cpack ? (p.K + se - 1) / se * se : p.K;
  const long long xb = product({p.N, cx, p.T, p.H, p.W, eb});
  const long long wb = product({p.K, p.C, p.KT, p.KH, p.KW, eb});
  const long long yb = p.pool ? product({p.N, p.K, oh / 2, ow / 2, eb})
                              : product({p.N, cy, ot, oh, ow, eb});
  if (xb > kMaxBytes || wb > kMaxBytes || yb > kMaxBytes) return LIBCONV_ERR_TOO_LARGE;
  const long long pb = packed_weight_bytes(p.C, p.K, p.KT, p.KH, p.KW, p.dtype);
  if (pb > kMaxBytes) return LIBCONV_ERR_TOO_LARGE;
  if (p.ws_bytes < 0) return LIBCONV_ERR_BAD_SHAPE;
  if (with_pointers) {
    if (!p.x || !(p.w || p.wp) || !p.y) return LIBCONV_ERR_NULL_POINTER;
    const long long bb = (long long)p.K * eb;
    if (yb > 0 && (overlaps(p.y, yb, p.x, xb) || overlaps(p.y, yb, p.w, wb) ||
                   overlaps(p.y, yb, p.wp, pb) || overlaps(p.y, yb, p.b, bb)))
      return LIBCONV_ERR_ALIAS;
    if (p.ws) {
      if ((reinterpret_cast<uintptr_t>(p.ws) & 255) != 0) return LIBCONV_ERR_MISALIGNED;
      const long long wsb = p.ws_bytes;
      if (overlaps(p.ws, wsb, p.x, xb) || overlaps(p.ws, wsb, p.w, wb) ||
          overlaps(p.ws, wsb, p.wp, pb) || overlaps(p.ws, wsb, p.b, bb) ||
          overlaps(p.ws, wsb, p.y, yb))
        return LIBCONV_ERR_ALIAS;
    }
  }
  return LIBCONV_OK;
}

// Per-device "is this a gfx950" cache, filled once per process.
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once;
int g_dev_count = 0;
bool g_dev_ok[kMaxDevices];
int g_dev_cus[kMaxDevices];

void init_devices() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 0) n = 0;
  if (n > kMaxDevices) n = kMaxDevices;
  for (int d = 0; d < n; ++d) {
    hipDeviceProp_t prop;
    g_dev_ok[d] = hipGetDeviceProperties(&prop, d) == hipSuccess &&
                  std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_cus[d] = g_dev_ok[d] && prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  }
  g_dev_count = n;
  (void)hipGetLastError();  // a host without GPUs leaves an error behind: clear it
}

bool device_ok(int d) {
  std::call_once(g_dev_once, init_devices);
  return d >= 0 && d < g_dev_count && g_dev_ok[d];
}

// The library's own workspace for conv3d_forward_noalloc: a device array of a
// fixed size, one copy on every GPU the library runs on, held until the
// process ends.  Host code never uses the array's name as an address: its
// device address on each device is looked up once (hipGetSymbolAddress, with
// that device current) and only that pointer is passed to kernels.
constexpr long long kScratchBytes = 64LL << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

// The address of this device's scratch array, or null if the lookup failed.
void* device_scratch(int d) {
  std::call_once(g_scratch_once[d], [d] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      ptr = nullptr;
    }
    g_scratch_ptr[d] = ptr;
  });
  return g_scratch_ptr[d];
}

// The dispatcher.  The vector-ALU direct kernel takes layers whose
// reduction per output (C_in * taps) is too short to fill an MFMA k-step
// pipeline -- stems with 3 input channels, pointwise layers with fewer than
// 32 input channels -- and any geometry the MFMA family has no tile for;
// everything else is an implicit GEMM on the matrix cores.
constexpr long long kMinMfmaReduction = 32;

libconv_status plan_for(const Problem& p, int algo, Plan* plan, bool packed_only = false) {
  const long long red = (long long)p.C * p.KT * p.KH * p.KW;
  // Evidence hook: LIBCONV_FORCE_TILE=<id> runs that MFMA tile when it fits
  // the shape (tile ids: libconv_tile_name); ignored otherwise.
  if (const char* ft = std::getenv("LIBCONV_FORCE_TILE")) {
    Plan forced;
    if (igemm_plan_tile(p, std::atoi(ft), &forced) && algo != LIBCONV_ALGO_DIRECT &&
        (!packed_only || igemm_tile_packed(forced.tile))) {
      *plan = forced;
      return LIBCONV_OK;
    }
    if (!packed_only && algo != LIBCONV_ALGO_IGEMM && direct_plan_tile(p, std::atoi(ft), &forced)) {
      *plan = forced;
      return LIBCONV_OK;
    }
  }
  if (packed_only) {  // only packed weights exist: MFMA tiles that read them
    if (algo == LIBCONV_ALGO_DIRECT || !igemm_plan_packed(p, plan)) return LIBCONV_ERR_UNSUPPORTED;
    return LIBCONV_OK;
  }
  Plan ig, dr;
  const bool has_ig = igemm_plan(p, &ig);
  const bool has_dr = direct_plan(p, &dr);
  if (algo == LIBCONV_ALGO_IGEMM) {
    if (!has_ig) return LIBCONV_ERR_UNSUPPORTED;
    *plan = ig;
    return LIBCONV_OK;
  }
  if (algo == LIBCONV_ALGO_DIRECT) {
    if (!has_dr) return LIBCONV_ERR_UNSUPPORTED;
    *plan = dr;
    return LIBCONV_OK;
  }
  if (has_ig && red >= kMinMfmaReduction) {
    *plan = ig;
    return LIBCONV_OK;
  }
  if (has_dr) {
    *plan = dr;
    return LIBCONV_OK;
  }
  if (has_ig) {
    *plan = ig;
    return LIBCONV_OK;
  }
  return LIBCONV_ERR_UNSUPPORTED;
}

// Plans of recent calls, per host thread: a layer called again with the same
// shape reuses its plan instead of re-running the cost model.  The key holds
// everything the dispatcher reads (shape, dtype, activation, forced family,
// capture state, which weight forms exist, 16-byte alignment of x, compute
// units, fused pooling).  Not used while a LIBCONV_FORCE_* override is set.
struct PlanKey {
  int v[28];
  bool operator==(const PlanKey& o) const { return std::memcmp(v, o.v, sizeof(v)) == 0; }
};

PlanKey plan_key(const Problem& p, int algo) {
  PlanKey k;
  const int v[28] = {p.N, p.C, p.T, p.H, p.W, p.K, p.KT, p.KH, p.KW, p.pt, p.ph, p.pw, p.st, p.sh,
                     p.sw, p.dtype, p.act, algo, (int)(p.ws_bytes & 0x7fffffff),
                     (int)(p.ws_bytes >> 31), p.w == nullptr,
                     (int)(reinterpret_cast<uintptr_t>(p.x) & 15), p.cus, p.wp != nullptr, p.ptb,
                     (int)p.pool, (int)p.cpack, (int)(reinterpret_cast<uintptr_t>(p.y) & 15)};
  std::memcpy(k.v, v, sizeof(v));
  return k;
}

struct PlanCacheEntry {
  bool used = false;
  PlanKey key;
  Plan plan;
};
constexpr int kPlanCacheSlots = 64;
thread_local PlanCacheEntry t_plan_cache[kPlanCacheSlots];

libconv_status cached_plan(const Problem& p, int algo, Plan* plan) {
  if (std::getenv("LIBCONV_FORCE_TILE") || std::getenv("LIBCONV_FORCE_KSPLIT"))
    return plan_for(p, algo, plan, p.w == nullptr);
  const PlanKey k = plan_key(p, algo);
  uint32_t h = 2166136261u;  // FNV-1a over the key words
  for (int x : k.v) h = (h ^ (uint32_t)x) * 16777619u;
  PlanCacheEntry& e = t_plan_cache[h % kPlanCacheSlots];
  if (e.used && e.key == k) {
    *plan = e.plan;
    return LIBCONV_OK;
  }
  const libconv_status st = plan_for(p, algo, plan, p.w == nullptr);
  if (st == LIBCONV_OK) {
    e.used = true;
    e.key = k;
    e.plan = *plan;
  }
  return st;
}

libconv_status run(Problem& p, int algo) {
  libconv_status st = validate(p, algo, true);
  if (st != LIBCONV_OK) return st;
  if (p.N == 0) return LIBCONV_OK;  // empty batch: nothing to compute
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev)) {
    (void)hipGetLastError();
    return LIBCONV_ERR_NO_DEVICE;
  }
  p.cus = g_dev_cus[dev];
  // The plan is a function of the shape, the weight forms and the workspace
  // size only: a call recorded into a HIP graph runs the kernels the same
  // call runs eagerly (the fixed-shape rule of capture and replay).
  Plan plan;
  st = cached_plan(p, algo, &plan);
  if (st != LIBCONV_OK) return st;
  if (std::getenv("LIBCONV_LOG")) {
    const char* name = plan.algo == LIBCONV_ALGO_DIRECT ? direct_tile_name(plan.tile)
                                                        : igemm_tile_name(plan.tile);
    std::fprintf(stderr,
                 "libconv: %s grid=%lld ksplit=%d (N=%d C=%d T=%d H=%d W=%d K=%d k=%dx%dx%d)\n",
                 name ? name : "?", plan.grid, plan.ksplit, p.N, p.C, p.T, p.H, p.W, p.K, p.KT,
                 p.KH, p.KW);
  }
  if (plan.algo == LIBCONV_ALGO_DIRECT) return direct_launch(p, plan);
  return igemm_launch(p, plan);
}

Problem make_problem(const void* x, const void* w, const void* bias, void* y, int N, int C_in,
                     int T, int H, int W, int C_out, int KT, int KH, int KW, int pad_t, int pad_h,
                     int pad_w, int stride_t, int stride_h, int stride_w, int dtype, int act,
                     void* stream) {
  Problem p;
  std::memset(&p, 0, sizeof(p));
  p.N = N; p.C = C_in; p.T = T; p.H = H; p.W = W;
  p.K = C_out; p.KT = KT; p.KH = KH; p.KW = KW;
  p.pt = pad_t; p.ph = pad_h; p.pw = pad_w;
  p.ptb = pad_t;
  p.st = stride_t; p.sh = stride_h; p.sw = stride_w;
  p.dtype = dtype; p.act = act;
  p.x = x; p.w = w; p.b = bias; p.y = y;
  p.stream = reinterpret_cast<hipStream_t>(stream);
  p.cus = 256;  // MI355X; the device's own count replaces it before a launch
  p.ws = nullptr;
  p.ws_bytes = 0;
  return p;
}

// The call that computes output frames [o0, o0 + On) of a video convolution
// from a buffer holding exactly the input frames libconv_frame_window names:
// the same convolution on that window, with the time padding that makes its
// first and last taps land where they land in the whole video.
libconv_status window_problem(Problem* out, const void* x, const void* w, const void* packed_w,
                              const void* bias, void* y, int N, int C_in, int T, int H, int W,
                              int C_out, int KT, int KH, int KW, int pad_t_front, int pad_t_back,
                              int pad_h, int pad_w, int stride_t, int stride_h, int stride_w,
                              int o0, int On, int dtype, int act, void* stream) {
  int f0 = 0, tw = 0;
  const libconv_status st = libconv_frame_window(T, KT, pad_t_front, pad_t_back, stride_t, o0, On,
                                                 &f0, &tw);
  if (st != LIBCONV_OK) return st;
  const long long lo = (long long)o0 * stride_t - pad_t_front;
  const long long hi = (long long)(o0 + On - 1) * stride_t - pad_t_front + KT;
  Problem p = make_problem(x, w, bias, y, N, C_in, tw, H, W, C_out, KT, KH, KW,
                           (int)(f0 - lo), pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act,
                           stream);
  p.ptb = (int)(hi - (f0 + tw));
  p.wp = packed_w;
  *out = p;
  return LIBCONV_OK;
}

// Geometry of a chunked call: output frames in chunks of `chunk`, each
// computed from its own input window (consecutive windows overlap by the
// frames two chunks share).
struct ChunkPlan {
  int OT, OH, OW;
  int chunks;
  int max_window;        // frames of the largest input window
  long long x_buf;       // bytes of one input-window buffer (256-byte multiple)
  long long y_buf;       // bytes of one output-chunk buffer (256-byte multiple)
  long long w_buf;       // bytes for the weights packed once (0: no packed kernels)
};

libconv_status chunk_plan(int N, int C_in, int T, int H, int W, int C_out, int KT, int KH, int KW,
                          int pad_t_front, int pad_t_back, int pad_h, int pad_w, int stride_t,
                          int stride_h, int stride_w, int chunk, int dtype, ChunkPlan* cp) {
  if (dtype != LIBCONV_F32 && dtype != LIBCONV_F16 && dtype != LIBCONV_BF16)
    return LIBCONV_ERR_BAD_DTYPE;
  if (N < 0 || C_in < 1 || T < 1 || H < 1 || W < 1 || C_out < 1 || KT < 1 || KH < 1 || KW < 1 ||
      chunk < 1)
    return LIBCONV_ERR_BAD_SHAPE;
  // every output frame must read at least one input frame
  if (pad_t_front < 0 || pad_t_back < 0 || pad_t_front >= KT || pad_t_back >= KT)
    return LIBCONV_ERR_BAD_SHAPE;
  const long long ot = out_extent2(T, KT, pad_t_front, pad_t_back, stride_t);
  const long long oh = out_extent(H, KH, pad_h, stride_h);
  const long long ow = out_extent(W, KW, pad_w, stride_w);
  if (ot < 1 || oh < 1 || ow < 1) return LIBCONV_ERR_BAD_SHAPE;
  if (ot > 0x7fffffff || oh > 0x7fffffff || ow > 0x7fffffff) return LIBCONV_ERR_TOO_LARGE;
  cp->OT = (int)ot; cp->OH = (int)oh; cp->OW = (int)ow;
  chunk = (int)std::min<long long>(chunk, ot);
  cp->chunks = (int)((ot + chunk - 1) / chunk);
  cp->max_window = 0;
  for (int c = 0; c < cp->chunks; ++c) {
    int f0 = 0, tw = 0;
    const int o0 = c * chunk;
    const libconv_status st = libconv_frame_window(
        T, KT, pad_t_front, pad_t_back, stride_t, o0, std::min(chunk, cp->OT - o0), &f0, &tw);
    if (st != LIBCONV_OK) return st;
    cp->max_window = std::max(cp->max_window, tw);
  }
  const long long eb = dtype_bytes(dtype);
  const long long xb = product({N, C_in, cp->max_window, H, W, eb});
  const long long yb = product({N, C_out, chunk, oh, ow, eb});
  if (xb > kMaxBytes || yb > kMaxBytes) return LIBCONV_ERR_TOO_LARGE;
  cp->x_buf = (xb + 255) / 256 * 256;
  cp->y_buf = (yb + 255) / 256 * 256;
  cp->w_buf = pack_supported(KT, KH, KW, dtype)
                  ? (packed_weight_bytes(C_in, C_out, KT, KH, KW, dtype) + 255) / 256 * 256
                  : 0;
  if (cp->w_buf > kMaxBytes) cp->w_buf = 0;
  return LIBCONV_OK;
}

libconv_status layout_call(const void* src, void* dst, int N, int C, int T, int H, int W,
                           int dtype, bool to_packed, void* stream) {
  if (dtype != LIBCONV_F32 && dtype != LIBCONV_F16 && dtype != LIBCONV_BF16)
    return LIBCONV_ERR_BAD_DTYPE;
  if (N < 0 || C < 1 || T < 1 || H < 1 || W < 1) return LIBCONV_ERR_BAD_SHAPE;
  const long long spatial = (long long)T * H * W;
  const long long plain = product({N, C, spatial, dtype_bytes(dtype)});
  const long long packed = cpack_bytes(N, C, spatial, dtype);
  if (plain > kMaxBytes || packed > kMaxBytes) return LIBCONV_ERR_TOO_LARGE;
  if (!src || !dst) return LIBCONV_ERR_NULL_POINTER;
  if (overlaps(src, to_packed ? plain : packed, dst, to_packed ? packed : plain))
    return LIBCONV_ERR_ALIAS;
  if (N == 0) return LIBCONV_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev)) {
    (void)hipGetLastError();
    return LIBCONV_ERR_NO_DEVICE;
  }
  return layout_launch(src, dst, N, C, spatial, dtype, to_packed,
                       reinterpret_cast<hipStream_t>(stream));
}

// Everything a convolution call can ask for, in one place: OIHW / OIDHW
// weights (w) or packed ones (packed_w, exactly one of them), time padding
// before and after the frames, channel-packed activations or fused pooling
// (flags), a forced kernel family, and the caller's workspace.
libconv_status forward_ex(const void* x, const void* w, const void* packed_w, const void* bias,
                          void* y, int N, int C_in, int T, int H, int W, int C_out, int KT, int KH,
                          int KW, int pad_t_front, int pad_t_back, int pad_h, int pad_w,
                          int stride_t, int stride_h, int stride_w, int dtype, int act, int algo,
                          int flags, void* workspace, long long workspace_bytes, void* stream) {
  if ((w == nullptr) == (packed_w == nullptr)) return LIBCONV_ERR_NULL_POINTER;
  Problem p = make_problem(x, w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t_front,
                           pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, stream);
  p.ptb = pad_t_back;
  p.wp = packed_w;
  p.pool = (flags & LIBCONV_PLAN_POOL2) != 0;
  p.cpack = (flags & LIBCONV_PLAN_CPACK) != 0;
  p.ws = workspace;
  p.ws_bytes = workspace ? workspace_bytes : 0;
  if (workspace && workspace_bytes < 0) return LIBCONV_ERR_BAD_SHAPE;
  if (packed_w && algo == LIBCONV_ALGO_DIRECT) return LIBCONV_ERR_UNSUPPORTED;
  return run(p, packed_w ? LIBCONV_ALGO_IGEMM : algo);
}

// The plan a call with these arguments makes (no pointers are looked at);
// flags as libconv_query_plan.
libconv_status plan_query(Problem& p, int algo, int flags, Plan* plan) {
  p.pool = (flags & LIBCONV_PLAN_POOL2) != 0;
  p.cpack = (flags & LIBCONV_PLAN_CPACK) != 0;
  const bool packed_w = (flags & LIBCONV_PLAN_PACKED_W) != 0;
  static const char packed_marker = 0;  // planning only asks whether packed weights exist
  if (packed_w) p.wp = &packed_marker;
  libconv_status st = validate(p, algo, false);
  if (st != LIBCONV_OK) return st;
  if (packed_w && algo == LIBCONV_ALGO_DIRECT) return LIBCONV_ERR_UNSUPPORTED;
  return plan_for(p, packed_w ? LIBCONV_ALGO_IGEMM : algo, plan, packed_w);
}

}  // namespace

}  // namespace libconv

using namespace libconv;

extern "C" {

libconv_status conv2d_forward(const void* x, const void* w, const void* bias, void* y, int N,
                              int C_in, int H, int W, int C_out, int KH, int KW, int pad_h,
                              int pad_w, int stride_h, int stride_w, int dtype, int act,
                              void* stream) {
  return forward_ex(x, w, nullptr, bias, y, N, C_in, 1, H, W, C_out, 1, KH, KW, 0, 0, pad_h,
                    pad_w, 1, stride_h, stride_w, dtype, act, LIBCONV_ALGO_AUTO, 0, nullptr, 0,
                    stream);
}

libconv_status conv2d_forward_ws(const void* x, const void* w, const void* bias, void* y, int N,
                                 int C_in, int H, int W, int C_out, int KH, int KW, int pad_h,
                                 int pad_w, int stride_h, int stride_w, int dtype, int act,
                                 void* workspace, long long workspace_bytes, void* stream) {
  return forward_ex(x, w, nullptr, bias, y, N, C_in, 1, H, W, C_out, 1, KH, KW, 0, 0, pad_h,
                    pad_w, 1, stride_h, stride_w, dtype, act, LIBCONV_ALGO_AUTO, 0, workspace,
                    workspace_bytes, stream);
}

libconv_status conv3d_forward(const void* x, const void* w, const void* bias, void* y, int N,
                              int C_in, int T, int H, int W, int C_out, int KT, int KH, int KW,
                              int pad_t, int pad_h, int pad_w, int stride_t, int stride_h,
                              int stride_w, int dtype, int act, void* stream) {
  return forward_ex(x, w, nullptr, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_t,
                    pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, LIBCONV_ALGO_AUTO, 0,
                    nullptr, 0, stream);
}

libconv_status conv3d_forward_ws(const void* x, const void* w, const void* bias, void* y, int N,
                                 int C_in, int T, int H, int W, int C_out, int KT, int KH, int KW,
                                 int pad_t, int pad_h, int pad_w, int stride_t, int stride_h,
                                 int stride_w, int dtype, int act, void* workspace,
                                 long long workspace_bytes, void* stream) {
  return forward_ex(x, w, nullptr, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_t,
                    pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, LIBCONV_ALGO_AUTO, 0,
                    workspace, workspace_bytes, stream);
}

libconv_status libconv_forward_ex(const void* x, const void* w, const void* packed_w,
                                  const void* bias, void* y, int N, int C_in, int T, int H, int W,
                                  int C_out, int KT, int KH, int KW, int pad_t_front,
                                  int pad_t_back, int pad_h, int pad_w, int stride_t,
                                  int stride_h, int stride_w, int dtype, int act, int algo,
                                  int flags, void* workspace, long long workspace_bytes,
                                  void* stream) {
  return forward_ex(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t_front,
                    pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, algo,
                    flags, workspace, workspace_bytes, stream);
}

libconv_status conv3d_forward_noalloc(const void* x, const void* w, const void* bias, void* y,
                                     int N, int C_in, int T, int H, int W, int C_out, int KT,
                                     int KH, int KW, int pad_t, int pad_h, int pad_w,
                                     int stride_t, int stride_h, int stride_w, int dtype, int act,
                                     void* stream) {
  const long long need = libconv_workspace_size(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t,
                                                pad_t, pad_h, pad_w, stride_t, stride_h,
                                                stride_w, dtype, act, LIBCONV_ALGO_AUTO, 0);
  if (need > kScratchBytes) return LIBCONV_ERR_SCRATCH_TOO_SMALL;
  if (need < 0 || N == 0)  // argument errors and empty batches: as conv3d_forward_ws
    return forward_ex(x, w, nullptr, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_t,
                      pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, LIBCONV_ALGO_AUTO,
                      0, nullptr, 0, stream);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev)) {
    (void)hipGetLastError();
    return LIBCONV_ERR_NO_DEVICE;
  }
  void* ws = device_scratch(dev);
  if (!ws) return LIBCONV_ERR_LAUNCH;
  return forward_ex(x, w, nullptr, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_t,
                    pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, LIBCONV_ALGO_AUTO, 0,
                    ws, kScratchBytes, stream);
}

long long libconv_workspace_size(int N, int C_in, int T, int H, int W, int C_out, int KT, int KH,
                                 int KW, int pad_t_front, int pad_t_back, int pad_h, int pad_w,
                                 int stride_t, int stride_h, int stride_w, int dtype, int act,
                                 int algo, int flags) {
  Problem p = make_problem(nullptr, nullptr, nullptr, nullptr, N, C_in, T, H, W, C_out, KT, KH,
                           KW, pad_t_front, pad_h, pad_w, stride_t, stride_h, stride_w, dtype,
                           act, nullptr);
  p.ptb = pad_t_back;
  p.ws_bytes = 1LL << 40;  // as much as the best plan wants
  Plan plan;
  if (plan_query(p, algo, flags, &plan) != LIBCONV_OK) return -1;
  return plan_workspace(p, plan);
}

libconv_status libconv_forward_algo(const void* x, const void* w, const void* bias, void* y, int N,
                                    int C_in, int T, int H, int W, int C_out, int KT, int KH,
                                    int KW, int pad_t, int pad_h, int pad_w, int stride_t,
                                    int stride_h, int stride_w, int dtype, int act, int algo,
                                    void* stream) {
  return forward_ex(x, w, nullptr, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_t,
                    pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, algo, 0, nullptr, 0,
                    stream);
}

long long libconv_packed_weight_bytes(int C_in, int C_out, int KT, int KH, int KW, int dtype) {
  if (C_in < 1 || C_out < 1 || KT < 1 || KH < 1 || KW < 1) return -1;
  if (dtype != LIBCONV_F32 && dtype != LIBCONV_F16 && dtype != LIBCONV_BF16) return -1;
  if (!pack_supported(KT, KH, KW, dtype)) return -1;
  const long long b = packed_weight_bytes(C_in, C_out, KT, KH, KW, dtype);
  return b > 0x7fffffffLL ? -1 : b;
}

libconv_status libconv_pack_weights(const void* w, void* packed, long long packed_bytes, int C_in,
                                    int C_out, int KT, int KH, int KW, int dtype, void* stream) {
  if (dtype != LIBCONV_F32 && dtype != LIBCONV_F16 && dtype != LIBCONV_BF16)
    return LIBCONV_ERR_BAD_DTYPE;
  if (C_in < 1 || C_out < 1 || KT < 1 || KH < 1 || KW < 1) return LIBCONV_ERR_BAD_SHAPE;
  if (!w || !packed) return LIBCONV_ERR_NULL_POINTER;
  if (!pack_supported(KT, KH, KW, dtype)) return LIBCONV_ERR_UNSUPPORTED;
  const long long need = packed_weight_bytes(C_in, C_out, KT, KH, KW, dtype);
  const long long wb = (long long)C_out * C_in * KT * KH * KW * dtype_bytes(dtype);
  if (need > 0x7fffffffLL || wb > 0x7fffffffLL) return LIBCONV_ERR_TOO_LARGE;
  if (packed_bytes < need) return LIBCONV_ERR_BAD_SHAPE;
  if (overlaps(packed, need, w, wb)) return LIBCONV_ERR_ALIAS;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev)) {
    (void)hipGetLastError();
    return LIBCONV_ERR_NO_DEVICE;
  }
  return pack_launch(w, packed, C_in, C_out, KT, KH, KW, dtype,
                     reinterpret_cast<hipStream_t>(stream));
}

libconv_status conv2d_forward_pool(const void* x, const void* w, const void* bias, void* y, int N,
                                   int C_in, int H, int W, int C_out, int KH, int KW, int pad_h,
                                   int pad_w, int stride_h, int stride_w, int dtype, int act,
                                   void* stream) {
  return forward_ex(x, w, nullptr, bias, y, N, C_in, 1, H, W, C_out, 1, KH, KW, 0, 0, pad_h,
                    pad_w, 1, stride_h, stride_w, dtype, act, LIBCONV_ALGO_AUTO,
                    LIBCONV_PLAN_POOL2, nullptr, 0, stream);
}

libconv_status conv3d_forward_tpad(const void* x, const void* w, const void* packed_w,
                                   const void* bias, void* y, int N, int C_in, int T, int H, int W,
                                   int C_out, int KT, int KH, int KW, int pad_t_front,
                                   int pad_t_back, int pad_h, int pad_w, int stride_t,
                                   int stride_h, int stride_w, int dtype, int act, void* stream) {
  return forward_ex(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t_front,
                    pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act,
                    LIBCONV_ALGO_AUTO, 0, nullptr, 0, stream);
}

libconv_status conv3d_forward_cpack(const void* x, const void* w, const void* packed_w,
                                    const void* bias, void* y, int N, int C_in, int T, int H,
                                    int W, int C_out, int KT, int KH, int KW, int pad_t_front,
                                    int pad_t_back, int pad_h, int pad_w, int stride_t,
                                    int stride_h, int stride_w, int dtype, int act,
                                    void* stream) {
  return forward_ex(x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t_front,
                    pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act,
                    LIBCONV_ALGO_AUTO, LIBCONV_PLAN_CPACK, nullptr, 0, stream);
}

long long libconv_cpack_bytes(int N, int C, int T, int H, int W, int dtype) {
  if (dtype != LIBCONV_F32 && dtype != LIBCONV_F16 && dtype != LIBCONV_BF16) return -1;
  if (N < 0 || C < 1 || T < 1 || H < 1 || W < 1) return -1;
  const long long b = cpack_bytes(N, C, (long long)T * H * W, dtype);
  return b > kMaxBytes ? -1 : b;
}

libconv_status libconv_pack_activations(const void* x, void* x_packed, int N, int C, int T, int H,
                                        int W, int dtype, void* stream) {
  return layout_call(x, x_packed, N, C, T, H, W, dtype, true, stream);
}

libconv_status libconv_unpack_activations(const void* x_packed, void* x, int N, int C, int T,
                                          int H, int W, int dtype, void* stream) {
  return layout_call(x_packed, x, N, C, T, H, W, dtype, false, stream);
}

libconv_status libconv_frame_window(int T, int KT, int pad_t_front, int pad_t_back, int stride_t,
                                    int out_frame0, int out_frames, int* in_frame0,
                                    int* in_frames) {
  if (!in_frame0 || !in_frames) return LIBCONV_ERR_NULL_POINTER;
  const long long ot = out_extent2(T, KT, pad_t_front, pad_t_back, stride_t);
  if (ot < 1 || out_frame0 < 0 || out_frames < 1 || (long long)out_frame0 + out_frames > ot)
    return LIBCONV_ERR_BAD_SHAPE;
  // Output frame o reads frames o*stride_t - pad_t_front + kt, 0 <= kt < KT,
  // of which those in [0, T) exist: at least one exactly when
  // o*stride_t > pad_t_front - KT and o*stride_t < T + pad_t_front, which
  // holds for a contiguous run of output frames.
  auto floordiv = [](long long a, long long b) { return a >= 0 ? a / b : -((-a + b - 1) / b); };
  const long long s = stride_t;
  const long long o_lo = std::max<long long>(out_frame0, floordiv(pad_t_front - KT, s) + 1);
  const long long o_hi = std::min<long long>(out_frame0 + out_frames - 1,
                                             floordiv((long long)T + pad_t_front - 1, s));
  if (o_lo > o_hi) return LIBCONV_ERR_BAD_SHAPE;  // those output frames read padding only
  const long long f0 = std::max(0LL, o_lo * s - pad_t_front);
  const long long f1 = std::min<long long>(T, o_hi * s - pad_t_front + KT);
  *in_frame0 = (int)f0;
  *in_frames = (int)(f1 - f0);
  return LIBCONV_OK;
}

libconv_status conv3d_forward_frames(const void* x, const void* w, const void* packed_w,
                                     const void* bias, void* y, int N, int C_in, int T, int H,
                                     int W, int C_out, int KT, int KH, int KW, int pad_t_front,
                                     int pad_t_back, int pad_h, int pad_w, int stride_t,
                                     int stride_h, int stride_w, int out_frame0, int out_frames,
                                     int dtype, int act, void* stream) {
  if ((w == nullptr) == (packed_w == nullptr)) return LIBCONV_ERR_NULL_POINTER;
  Problem p;
  const libconv_status st =
      window_problem(&p, x, w, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW,
                     pad_t_front, pad_t_back, pad_h, pad_w, stride_t, stride_h, stride_w,
                     out_frame0, out_frames, dtype, act, stream);
  if (st != LIBCONV_OK) return st;
  return run(p, packed_w ? LIBCONV_ALGO_IGEMM : LIBCONV_ALGO_AUTO);
}

long long libconv_chunked_workspace_bytes(int N, int C_in, int T, int H, int W, int C_out, int KT,
                                          int KH, int KW, int pad_t_front, int pad_t_back,
                                          int pad_h, int pad_w, int stride_t, int stride_h,
                                          int stride_w, int chunk_frames, int dtype) {
  ChunkPlan cp;
  if (chunk_plan(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t_front, pad_t_back, pad_h, pad_w,
                 stride_t, stride_h, stride_w, chunk_frames, dtype, &cp) != LIBCONV_OK)
    return -1;
  return 2 * (cp.x_buf + cp.y_buf) + cp.w_buf;
}

libconv_status conv3d_forward_chunked(const void* x, const void* w, const void* packed_w,
                                      const void* bias, void* y, int N, int C_in, int T, int H,
                                      int W, int C_out, int KT, int KH, int KW, int pad_t_front,
                                      int pad_t_back, int pad_h, int pad_w, int stride_t,
                                      int stride_h, int stride_w, int chunk_frames,
                                      void* workspace, long long workspace_bytes, int dtype,
                                      int act, void* stream, void* copy_in_stream,
                                      void* copy_out_stream) {
  if ((w == nullptr) == (packed_w == nullptr)) return LIBCONV_ERR_NULL_POINTER;
  if (act != LIBCONV_ACT_NONE && act != LIBCONV_ACT_RELU) return LIBCONV_ERR_BAD_ACTIVATION;
  ChunkPlan cp;
  libconv_status st = chunk_plan(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t_front, pad_t_back,
                                 pad_h, pad_w, stride_t, stride_h, stride_w, chunk_frames, dtype,
                                 &cp);
  if (st != LIBCONV_OK) return st;
  if (!x || !y || !workspace) return LIBCONV_ERR_NULL_POINTER;
  if (workspace_bytes < 2 * (cp.x_buf + cp.y_buf) + cp.w_buf) return LIBCONV_ERR_BAD_SHAPE;
  const size_t eb = (size_t)dtype_bytes(dtype);
  const size_t x_frame = (size_t)H * W * eb, y_frame = (size_t)cp.OH * cp.OW * eb;
  const size_t x_all = (size_t)N * C_in * T * x_frame, y_all = (size_t)N * C_out * cp.OT * y_frame;
  if (overlaps(y, (long long)y_all, x, (long long)x_all) ||
      overlaps(workspace, workspace_bytes, x, (long long)x_all) ||
      overlaps(workspace, workspace_bytes, y, (long long)y_all))
    return LIBCONV_ERR_ALIAS;
  if (N == 0) return LIBCONV_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev)) {
    (void)hipGetLastError();
    return LIBCONV_ERR_NO_DEVICE;
  }
  const hipStream_t cs = reinterpret_cast<hipStream_t>(stream);
  const hipStream_t ki = copy_in_stream ? reinterpret_cast<hipStream_t>(copy_in_stream) : cs;
  const hipStream_t ko = copy_out_stream ? reinterpret_cast<hipStream_t>(copy_out_stream) : ki;
  for (hipStream_t s : {cs, ki, ko}) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) {
      (void)hipGetLastError();
      return LIBCONV_ERR_LAUNCH;
    }
    if (cap != hipStreamCaptureStatusNone) return LIBCONV_ERR_UNSUPPORTED;
  }
  const bool sync = ki != cs || ko != cs;  // more than one stream: order them with events
  const int chunk = std::min(chunk_frames, cp.OT);
  char* ws = static_cast<char*>(workspace);
  void* xb[2] = {ws, ws + cp.x_buf};
  void* yb[2] = {ws + 2 * cp.x_buf, ws + 2 * cp.x_buf + cp.y_buf};
  // OIDHW weights: packed once, into the workspace after the four buffers,
  // for every chunk (the chunks then run the packed kernels), when an MFMA
  // kernel that reads packed weights takes the chunk's shape
  bool pack_once = false;
  if (w && cp.w_buf > 0) {
    static const char packed_marker = 0;  // planning only asks whether packed weights exist
    Problem q;
    Plan pl;
    pack_once = window_problem(&q, xb[0], nullptr, &packed_marker, bias, yb[0], N, C_in, T, H,
                               W, C_out, KT, KH, KW, pad_t_front, pad_t_back, pad_h, pad_w,
                               stride_t, stride_h, stride_w, 0, chunk, dtype, act,
                               stream) == LIBCONV_OK &&
                validate(q, LIBCONV_ALGO_IGEMM, false) == LIBCONV_OK &&
                plan_for(q, LIBCONV_ALGO_IGEMM, &pl, true) == LIBCONV_OK;
  }
  if (pack_once) {
    void* wpk = ws + 2 * (cp.x_buf + cp.y_buf);
    const libconv_status ps = pack_launch(w, wpk, C_in, C_out, KT, KH, KW, dtype, cs);
    if (ps != LIBCONV_OK) return ps;
    packed_w = wpk;
    w = nullptr;
  }
  // ev_in[b] / ev_conv[b] / ev_out[b]: the latest copy into xb[b], convolution
  // into yb[b], copy out of yb[b]; ev_edge: the start and the end of the call.
  hipEvent_t ev[7] = {};
  hipEvent_t *ev_in = ev, *ev_conv = ev + 2, *ev_out = ev + 4, &ev_edge = ev[6];
  auto ok = [](hipError_t e) {
    if (e == hipSuccess) return true;
    (void)hipGetLastError();
    return false;
  };
  if (sync) {
    for (hipEvent_t& e : ev) {
      if (!ok(hipEventCreateWithFlags(&e, hipEventDisableTiming))) {
        for (hipEvent_t d : ev)
          if (d) (void)hipEventDestroy(d);
        return LIBCONV_ERR_LAUNCH;
      }
    }
  }
  auto record = [&](hipEvent_t e, hipStream_t s) { return !sync || ok(hipEventRecord(e, s)); };
  auto wait = [&](hipStream_t s, hipEvent_t e) {
    return !sync || ok(hipStreamWaitEvent(s, e, 0));
  };
  // Input window of chunk c into xb[c & 1]: N*C_in rows of tw frames, taken
  // at frame f0 of rows T frames apart.  Its buffer was last read by
  // conv(c - 2).  Frames the previous window also holds (the time halo) are
  // copied from xb[(c - 1) & 1] on the device, so that each frame of x is
  // read from its source once.
  int prev_f0 = 0, prev_tw = 0;
  auto copy_in = [&](int c) -> libconv_status {
    const int o0 = c * chunk, on = std::min(chunk, cp.OT - o0);
    int f0 = 0, tw = 0;
    const libconv_status s = libconv_frame_window(T, KT, pad_t_front, pad_t_back, stride_t, o0,
                                                  on, &f0, &tw);
    if (s != LIBCONV_OK) return s;
    if (c >= 2 && !wait(ki, ev_conv[c & 1])) return LIBCONV_ERR_LAUNCH;
    char* dst = static_cast<char*>(xb[c & 1]);
    const size_t rows = (size_t)N * C_in, pitch = tw * x_frame;
    // windows only move forward in time: the frames this window shares with
    // the previous one are that window's tail, held in xb[(c - 1) & 1]
    const int held = c > 0 && f0 >= prev_f0 ? std::clamp(prev_f0 + prev_tw - f0, 0, tw) : 0;
    if (held > 0) {
      const char* tail = static_cast<const char*>(xb[(c - 1) & 1]) + (f0 - prev_f0) * x_frame;
      if (!ok(hipMemcpy2DAsync(dst, pitch, tail, prev_tw * x_frame, held * x_frame, rows,
                               hipMemcpyDeviceToDevice, ki)))
        return LIBCONV_ERR_LAUNCH;
    }
    if (held < tw) {
      const char* src = static_cast<const char*>(x) + (size_t)(f0 + held) * x_frame;
      if (!ok(hipMemcpy2DAsync(dst + held * x_frame, pitch, src, (size_t)T * x_frame,
                               (tw - held) * x_frame, rows, hipMemcpyDefault, ki)))
        return LIBCONV_ERR_LAUNCH;
    }
    prev_f0 = f0;
    prev_tw = tw;
    return record(ev_in[c & 1], ki) ? LIBCONV_OK : LIBCONV_ERR_LAUNCH;
  };
  // Output chunk c from yb[c & 1] into frames [o0, o0 + on) of y, once
  // conv(c) is done.
  auto copy_out = [&](int c) -> libconv_status {
    const int o0 = c * chunk, on = std::min(chunk, cp.OT - o0);
    if (!wait(ko, ev_conv[c & 1])) return LIBCONV_ERR_LAUNCH;
    char* dst = static_cast<char*>(y) + (size_t)o0 * y_frame;
    if (!ok(hipMemcpy2DAsync(dst, (size_t)cp.OT * y_frame, yb[c & 1], on * y_frame, on * y_frame,
                             (size_t)N * C_out, hipMemcpyDefault, ko)))
      return LIBCONV_ERR_LAUNCH;
    return record(ev_out[c & 1], ko) ? LIBCONV_OK : LIBCONV_ERR_LAUNCH;
  };
  // The copies start after the work already on `stream` (which may produce
  // x or still use y).  The window of chunk c + 1 is copied in before chunk
  // c's output is copied out, so that with one copy stream the next input
  // does not queue behind an output that waits for the convolution.
  if (!record(ev_edge, cs) || !wait(ki, ev_edge) || !wait(ko, ev_edge)) st = LIBCONV_ERR_LAUNCH;
  if (st == LIBCONV_OK) st = copy_in(0);
  for (int c = 0; c < cp.chunks && st == LIBCONV_OK; ++c) {
    if (c + 1 < cp.chunks && (st = copy_in(c + 1)) != LIBCONV_OK) break;
    if (!wait(cs, ev_in[c & 1]) || (c >= 2 && !wait(cs, ev_out[c & 1]))) {
      st = LIBCONV_ERR_LAUNCH;
      break;
    }
    const int o0 = c * chunk, on = std::min(chunk, cp.OT - o0);
    Problem p;
    st = window_problem(&p, xb[c & 1], w, packed_w, bias, yb[c & 1], N, C_in, T, H, W, C_out, KT,
                        KH, KW, pad_t_front, pad_t_back, pad_h, pad_w, stride_t, stride_h,
                        stride_w, o0, on, dtype, act, stream);
    if (st == LIBCONV_OK) st = run(p, packed_w ? LIBCONV_ALGO_IGEMM : LIBCONV_ALGO_AUTO);
    if (st != LIBCONV_OK) break;
    if (!record(ev_conv[c & 1], cs)) {
      st = LIBCONV_ERR_LAUNCH;
      break;
    }
    st = copy_out(c);
  }
  if (sync) {
    // `stream` continues after every copy (also after a failure part-way,
    // so that nothing the caller frees next is still in use)
    for (hipStream_t s : {ki, ko})
      if (s != cs && ok(hipEventRecord(ev_edge, s))) (void)ok(hipStreamWaitEvent(cs, ev_edge, 0));
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
  return st;
}

libconv_status libconv_forward_packed(const void* x, const void* packed_w, const void* bias,
                                      void* y, int N, int C_in, int T, int H, int W, int C_out,
                                      int KT, int KH, int KW, int pad_t, int pad_h, int pad_w,
                                      int stride_t, int stride_h, int stride_w, int dtype,
                                      int act, void* stream) {
  if (!packed_w && x && y) return LIBCONV_ERR_NULL_POINTER;
  return forward_ex(x, nullptr, packed_w, bias, y, N, C_in, T, H, W, C_out, KT, KH, KW, pad_t,
                    pad_t, pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act,
                    LIBCONV_ALGO_IGEMM, 0, nullptr, 0, stream);
}

libconv_status libconv_query_algo(int N, int C_in, int T, int H, int W, int C_out, int KT, int KH,
                                  int KW, int pad_t, int pad_h, int pad_w, int stride_t,
                                  int stride_h, int stride_w, int dtype, int act, int algo,
                                  int* algo_out, int* tile_out, long long* grid_out) {
  int ksplit = 1;
  return libconv_query_plan(N, C_in, T, H, W, C_out, KT, KH, KW, pad_t, pad_h, pad_w, stride_t,
                            stride_h, stride_w, dtype, act, algo, 0, 0, algo_out, tile_out,
                            grid_out, &ksplit);
}

libconv_status libconv_query_plan(int N, int C_in, int T, int H, int W, int C_out, int KT, int KH,
                                  int KW, int pad_t, int pad_h, int pad_w, int stride_t,
                                  int stride_h, int stride_w, int dtype, int act, int algo,
                                  int flags, long long workspace_bytes, int* algo_out,
                                  int* tile_out, long long* grid_out, int* ksplit_out) {
  if (!algo_out || !tile_out || !grid_out || !ksplit_out) return LIBCONV_ERR_NULL_POINTER;
  if (workspace_bytes < 0) return LIBCONV_ERR_BAD_SHAPE;
  Problem p = make_problem(nullptr, nullptr, nullptr, nullptr, N, C_in, T, H, W, C_out, KT, KH, KW,
                           pad_t, pad_h, pad_w, stride_t, stride_h, stride_w, dtype, act, nullptr);
  p.ws_bytes = workspace_bytes;
  Plan plan;
  const libconv_status st = plan_query(p, algo, flags, &plan);
  if (st != LIBCONV_OK) return st;
  *algo_out = plan.algo;
  *tile_out = plan.tile;
  *grid_out = p.N == 0 ? 0 : plan.grid;
  *ksplit_out = plan.ksplit;
  return LIBCONV_OK;
}

libconv_status libconv_fold_batchnorm(const float* w, const float* b, const float* gamma,
                                      const float* beta, const float* mean, const float* var,
                                      float eps, int C_out, int k_per_out, float* w_out,
                                      float* b_out) {
  if (!w || !gamma || !beta || !mean || !var || !w_out || !b_out) return LIBCONV_ERR_NULL_POINTER;
  if (C_out < 1 || k_per_out < 1) return LIBCONV_ERR_BAD_SHAPE;
  for (int co = 0; co < C_out; ++co)
    if (!((double)var[co] + (double)eps > 0.0)) return LIBCONV_ERR_BAD_SHAPE;
  for (int co = 0; co < C_out; ++co) {
    const double s = (double)gamma[co] / std::sqrt((double)var[co] + (double)eps);
    const double bias = b ? (double)b[co] : 0.0;
    b_out[co] = (float)((bias - (double)mean[co]) * s + (double)beta[co]);
    const long long base = (long long)co * k_per_out;
    for (int k = 0; k < k_per_out; ++k) w_out[base + k] = (float)((double)w[base + k] * s);
  }
  return LIBCONV_OK;
}

const char* libconv_tile_name(int tile_id) {
  const char* n = direct_tile_name(tile_id);
  if (!n) n = igemm_tile_name(tile_id);
  return n ? n : "?";
}

int libconv_tile_occupancy(int tile_id, int dtype, int measured) {
  if (measured) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || !device_ok(dev)) {
      (void)hipGetLastError();
      return -1;
    }
  }
  return igemm_tile_occupancy(tile_id, dtype, measured != 0);
}

int libconv_out_size(int in, int k, int pad, int stride) {
  return libconv_out_size2(in, k, pad, pad, stride);
}

int libconv_out_size2(int in, int k, int pad_lo, int pad_hi, int stride) {
  const long long o = out_extent2(in, k, pad_lo, pad_hi, stride);
  return (o < 1 || o > 0x7fffffff) ? -1 : (int)o;
}

const char* libconv_status_string(int status) {
  switch (status) {
    case LIBCONV_OK: return "ok";
    case LIBCONV_ERR_NULL_POINTER: return "null pointer";
    case LIBCONV_ERR_BAD_SHAPE: return "bad shape";
    case LIBCONV_ERR_BAD_DTYPE: return "bad dtype";
    case LIBCONV_ERR_BAD_ACTIVATION: return "bad activation";
    case LIBCONV_ERR_ALIAS: return "output overlaps an input";
    case LIBCONV_ERR_UNSUPPORTED: return "unsupported shape for the requested algorithm";
    case LIBCONV_ERR_NO_DEVICE: return "no gfx950 device";
    case LIBCONV_ERR_LAUNCH: return "kernel launch failed";
    case LIBCONV_ERR_BAD_ALGO: return "bad algorithm";
    case LIBCONV_ERR_TOO_LARGE: return "tensor too large";
    case LIBCONV_ERR_OUT_OF_MEMORY: return "out of device memory";
    case LIBCONV_ERR_MISALIGNED: return "a pointer is not aligned as the call requires";
    case LIBCONV_ERR_SCRATCH_TOO_SMALL:
      return "the call needs more workspace than the library's 64 MiB scratch array";
    default: return "unknown status";
  }
}

libconv_status libconv_device_supported(int device) {
  return device_ok(device) ? LIBCONV_OK : LIBCONV_ERR_NO_DEVICE;
}

int libconv_version(void) { return 200; }

}  // extern "C"
