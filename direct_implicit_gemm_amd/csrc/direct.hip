// direct.hip -- LDS halo-tiled direct convolution on the vector ALUs.
//
// Meant for narrow layers whose reduction C_in * taps is short (C_in = 3
// stems, thin pointwise layers), where the work is bound by HBM traffic and
// an implicit GEMM would waste most of each matrix instruction.  It also runs
// every geometry, so it is the kernel of last resort for shapes the MFMA
// family has no tile for.
//
// Method: the gather rule of the page "PP-OCR on Vulkan compute shaders",
// section 2.2 -- each output element starts from its own coordinate, reads
// the input taps it covers (out-of-range taps contribute zero) and is written
// by exactly one lane, so there are no atomics and the result is
// deterministic.  ReLU is fused into the write-back (section 4.4 of that
// page).  What differs from the page's one-invocation-per-output shader:
//   * a workgroup owns a 4-row x (64*P)-column block of one output plane and
//     COT output channels; each lane keeps COT x P fp32 accumulators, so every
//     input value read from LDS feeds COT*P fused multiply-adds (the page's
//     Convolution3D work in "SeedVR2 NCNN Vulkan" computes 4 output channels
//     per invocation for the same reason);
//   * the input halo of the block (with the zero padding already applied) and
//     the block's weights are staged in LDS once per input-channel chunk
//     with coalesced row loads; weights are read back as wave-uniform
//     broadcasts;
//   * lanes walk consecutive output columns, so input rows are read and
//     output rows written as contiguous runs.
#include "device_common.h"
#include "internal.h"

namespace libconv {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 4;               // output rows per workgroup (one per wave)
constexpr int kLdsBudget = 60 * 1024;  // bytes of LDS a workgroup may use
constexpr int kBatch = 16;             // global loads in flight per lane while staging

struct DirectArgs {
  const void* x;
  const void* w;
  const void* b;
  void* y;
  int N, C, T, H, W, K, KT, KH, KW;
  int pt, ph, pw, st, sh, sw;
  int OT, OH, OW;
  int relu;
  int col_tiles, row_tiles;
  int cc;        // input channels per LDS stage
  int hr, hc;    // halo rows / columns
  int ws_off;    // float offset of the weight area (multiple of 4: 16-byte aligned)
  uint32_t x_bytes, w_bytes, b_bytes, y_bytes;
};

template <int DT, int COT, int P>
__global__ __launch_bounds__(kThreads) void direct_kernel(DirectArgs a) {
  extern __shared__ float smem[];
  using E = Elem<DT>;
  constexpr int eb = E::bytes;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  int t = blockIdx.x;
  const int ct = t % a.col_tiles;
  t /= a.col_tiles;
  const int rt = t % a.row_tiles;
  t /= a.row_tiles;
  const int ot = t % a.OT;
  const int n = t / a.OT;
  const int co0 = blockIdx.y * COT;
  const int oh0 = rt * kRows;
  const int ow0 = ct * (64 * P);
  const int ih0 = oh0 * a.sh - a.ph;
  const int iw0 = ow0 * a.sw - a.pw;
  const int taps2 = a.KH * a.KW;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);

  float* xs = smem;                          // [cc][hr][hc]
  float* ws = smem + a.ws_off;               // [cc][taps2][COT]

  float acc[COT][P];
#pragma unroll
  for (int j = 0; j < COT; ++j)
#pragma unroll
    for (int p = 0; p < P; ++p) acc[j][p] = 0.0f;

  for (int ci0 = 0; ci0 < a.C; ci0 += a.cc) {
    const int ccur = min(a.cc, a.C - ci0);
    for (int kt = 0; kt < a.KT; ++kt) {
      const int it = ot * a.st - a.pt + kt;
      if (it < 0 || it >= a.T) continue;  // whole frame is padding: contributes 0
      __syncthreads();                    // previous stage fully consumed
      // Input halo, zero outside the input (this is the padding).  Wave w
      // takes halo rows w, w+4, ...; a row is read as 64-column segments, one
      // element per lane.  Loads are issued in batches of kBatch before any
      // LDS store, so a wave waits for one round trip per batch, not per row.
      {
        const int nseg = (a.hc + 63) / 64;
        const int nrows = ccur * a.hr;
        const int items = wave < nrows ? ((nrows - 1 - wave) / 4 + 1) * nseg : 0;
        int m = 0, c = wave / a.hr, r = wave - (wave / a.hr) * a.hr;  // item (row, segment)
        for (int q0 = 0; q0 < items; q0 += kBatch) {
          float v[kBatch];
          int dst[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            const int col = m * 64 + lane;
            const int ih = ih0 + r, iw = iw0 + col;
            const bool live = q0 + u < items && col < a.hc;
            const bool ok = live && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
            const int off = ((((n * a.C + ci0 + c) * a.T + it) * a.H + ih) * a.W + iw) * eb;
            v[u] = E::load(xr, guard_offset(ok, off));
            dst[u] = live ? (c * a.hr + r) * a.hc + col : -1;
            if (++m == nseg) {  // next row of this wave: 4 halo rows further
              m = 0;
              r += 4;
              while (r >= a.hr) {
                r -= a.hr;
                ++c;
              }
            }
          }
#pragma unroll
          for (int u = 0; u < kBatch; ++u)
            if (dst[u] >= 0) xs[dst[u]] = v[u];
        }
      }
      // Weights of this channel chunk and frame tap, as [c][tap][co].
      const int nw = ccur * taps2 * COT;
      for (int e0 = 0; e0 < nw; e0 += kThreads * kBatch) {
        float v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int e = e0 + u * kThreads + threadIdx.x;
          const int j = e % COT;
          const int ctap = e / COT;
          const int c = ctap / taps2;
          const int tap = ctap - c * taps2;
          const int co = co0 + j;
          const bool ok = e < nw && co < a.K;
          v[u] = E::load(wr, guard_offset(ok, (((co * a.C + ci0 + c) * a.KT + kt) * taps2 + tap) * eb));
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int e = e0 + u * kThreads + threadIdx.x;
          if (e < nw) ws[e] = v[u];
        }
      }
      __syncthreads();

      for (int c = 0; c < ccur; ++c) {
        for (int kh = 0; kh < a.KH; ++kh) {
          const float* xrow = xs + (c * a.hr + wave * a.sh + kh) * a.hc;
          const float* wrow = ws + (c * taps2 + kh * a.KW) * COT;
          for (int kw = 0; kw < a.KW; ++kw) {
            float xv[P];
#pragma unroll
            for (int p = 0; p < P; ++p) xv[p] = xrow[(p * 64 + lane) * a.sw + kw];
            const float4* w4 = reinterpret_cast<const float4*>(wrow + kw * COT);
#pragma unroll
            for (int j4 = 0; j4 < COT / 4; ++j4) {
              const float4 wv = w4[j4];
#pragma unroll
              for (int p = 0; p < P; ++p) {
                acc[4 * j4 + 0][p] = fmaf(xv[p], wv.x, acc[4 * j4 + 0][p]);
                acc[4 * j4 + 1][p] = fmaf(xv[p], wv.y, acc[4 * j4 + 1][p]);
                acc[4 * j4 + 2][p] = fmaf(xv[p], wv.z, acc[4 * j4 + 2][p]);
                acc[4 * j4 + 3][p] = fmaf(xv[p], wv.w, acc[4 * j4 + 3][p]);
              }
            }
          }
        }
      }
    }
  }

  // Epilogue: bias, activation, one rounding, row-contiguous stores.
  const int oh = oh0 + wave;
  if (oh >= a.OH) return;
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, a.y_bytes);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.b, a.b_bytes);
  // All bias loads are issued before any store (one round trip, not one per
  // channel); channels beyond C_out read 0 and are not stored.
  float bias[COT];
#pragma unroll
  for (int j = 0; j < COT; ++j)
    bias[j] = E::load(br, guard_offset(a.b && co0 + j < a.K, (co0 + j) * eb));
#pragma unroll
  for (int j = 0; j < COT; ++j) {
    const int co = co0 + j;
    const int row = (((n * a.K + co) * a.OT + ot) * a.OH + oh) * a.OW;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int ow = ow0 + p * 64 + lane;
      if (co < a.K && ow < a.OW) E::store(epilogue(acc[j][p], bias[j], a.relu), yr, (row + ow) * eb);
    }
  }
}

// Tile ids: 100 + 10 * log2(COT / 4) + (P - 1).
struct DirectTile {
  int id, cot, p;
  const char* name;
};
constexpr DirectTile kDirectTiles[] = {
    {110, 8, 1, "direct_cot8_p1"},   {111, 8, 2, "direct_cot8_p2"},
    {120, 16, 1, "direct_cot16_p1"}, {121, 16, 2, "direct_cot16_p2"},
    {130, 32, 1, "direct_cot32_p1"}, {131, 32, 2, "direct_cot32_p2"},
    {140, 64, 1, "direct_cot64_p1"},
};

const DirectTile* find_tile(int id) {
  for (const auto& t : kDirectTiles)
    if (t.id == id) return &t;
  return nullptr;
}

struct Geometry {
  int hr, hc, cc, ws_off, lds;
};

// Halo size and the channel chunk that fits the LDS budget (>= 1 channel).
bool direct_geometry(const Problem& p, int cot, int P, Geometry* g) {
  g->hr = (kRows - 1) * p.sh + p.KH;
  g->hc = (64 * P - 1) * p.sw + p.KW;
  const long per_c = (long)g->hr * g->hc + (long)p.KH * p.KW * cot;  // floats per channel
  long cc = (kLdsBudget / 4 - 4) / per_c;
  if (cc < 1) return false;
  if (cc > p.C) cc = p.C;
  g->cc = (int)cc;
  g->ws_off = (int)((cc * g->hr * g->hc + 3) / 4 * 4);
  g->lds = (int)(g->ws_off + cc * p.KH * p.KW * cot) * 4;
  return true;
}

template <int DT, int COT, int P>
hipError_t launch_one(const DirectArgs& a, dim3 grid, int lds, hipStream_t s) {
  hipLaunchKernelGGL((direct_kernel<DT, COT, P>), grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const DirectArgs& a, int cot, int P, dim3 grid, int lds, hipStream_t s) {
  switch (cot * 10 + P) {
    case 81: return launch_one<DT, 8, 1>(a, grid, lds, s);
    case 82: return launch_one<DT, 8, 2>(a, grid, lds, s);
    case 161: return launch_one<DT, 16, 1>(a, grid, lds, s);
    case 162: return launch_one<DT, 16, 2>(a, grid, lds, s);
    case 321: return launch_one<DT, 32, 1>(a, grid, lds, s);
    case 322: return launch_one<DT, 32, 2>(a, grid, lds, s);
    case 641: return launch_one<DT, 64, 1>(a, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

const char* direct_tile_name(int id) {
  const DirectTile* t = find_tile(id);
  return t ? t->name : nullptr;
}

bool direct_plan(const Problem& p, Plan* plan) {
  // Output channels per workgroup: the smallest tile covering C_out, capped
  // at 64 (register budget); columns per lane: 2 when the row is long enough
  // that the wider tile wastes less than the narrower one.
  int cot = p.K <= 8 ? 8 : p.K <= 16 ? 16 : p.K <= 32 ? 32 : 64;
  int P = (cot < 64 && p.OW >= 128 && (p.OW % 128 == 0 || p.OW % 64 != 0)) ? 2 : 1;
  Geometry g;
  if (!direct_geometry(p, cot, P, &g)) {
    P = 1;
    if (!direct_geometry(p, cot, P, &g)) return false;
  }
  const long long col_tiles = (p.OW + 64 * P - 1) / (64 * P);
  const long long row_tiles = (p.OH + kRows - 1) / kRows;
  const long long co_tiles = (p.K + cot - 1) / cot;
  plan->algo = LIBCONV_ALGO_DIRECT;
  plan->tile = 100 + 10 * (cot == 8 ? 1 : cot == 16 ? 2 : cot == 32 ? 3 : 4) + (P - 1);
  plan->grid = (long long)p.N * p.OT * row_tiles * col_tiles * co_tiles;
  return true;
}

libconv_status direct_launch(const Problem& p, const Plan& plan) {
  const DirectTile* t = find_tile(plan.tile);
  if (!t) return LIBCONV_ERR_UNSUPPORTED;
  Geometry g;
  if (!direct_geometry(p, t->cot, t->p, &g)) return LIBCONV_ERR_UNSUPPORTED;
  DirectArgs a;
  a.x = p.x; a.w = p.w; a.b = p.b; a.y = p.y;
  a.N = p.N; a.C = p.C; a.T = p.T; a.H = p.H; a.W = p.W;
  a.K = p.K; a.KT = p.KT; a.KH = p.KH; a.KW = p.KW;
  a.pt = p.pt; a.ph = p.ph; a.pw = p.pw; a.st = p.st; a.sh = p.sh; a.sw = p.sw;
  a.OT = p.OT; a.OH = p.OH; a.OW = p.OW;
  a.relu = p.act == LIBCONV_ACT_RELU;
  a.col_tiles = (p.OW + 64 * t->p - 1) / (64 * t->p);
  a.row_tiles = (p.OH + kRows - 1) / kRows;
  a.cc = g.cc; a.hr = g.hr; a.hc = g.hc; a.ws_off = g.ws_off;
  const int eb = dtype_bytes(p.dtype);
  a.x_bytes = (uint32_t)((long long)p.N * p.C * p.T * p.H * p.W * eb);
  a.w_bytes = (uint32_t)((long long)p.K * p.C * p.KT * p.KH * p.KW * eb);
  a.b_bytes = p.b ? (uint32_t)(p.K * eb) : 0u;
  a.y_bytes = (uint32_t)((long long)p.N * p.K * p.OT * p.OH * p.OW * eb);
  const long long spatial_tiles = (long long)p.N * p.OT * a.row_tiles * a.col_tiles;
  const int co_tiles = (p.K + t->cot - 1) / t->cot;
  if (spatial_tiles > 0x7fffffffLL || co_tiles > 65535) return LIBCONV_ERR_UNSUPPORTED;
  dim3 grid((unsigned)spatial_tiles, (unsigned)co_tiles);
  hipError_t e;
  switch (p.dtype) {
    case LIBCONV_F32: e = launch_dt<DT_F32>(a, t->cot, t->p, grid, g.lds, p.stream); break;
    case LIBCONV_F16: e = launch_dt<DT_F16>(a, t->cot, t->p, grid, g.lds, p.stream); break;
    case LIBCONV_BF16: e = launch_dt<DT_BF16>(a, t->cot, t->p, grid, g.lds, p.stream); break;
    default: return LIBCONV_ERR_BAD_DTYPE;
  }
  return e == hipSuccess ? LIBCONV_OK : LIBCONV_ERR_LAUNCH;
}

}  // namespace libconv
