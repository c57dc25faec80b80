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
#include <algorithm>
#include <cmath>
#include <type_traits>

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
  int cpack;     // 1: x and y channel-packed ([N][C/g][T][H][W][g], g = 16 bytes of channels)
  int cc;        // input channels per LDS stage
  int hr, hc;    // halo rows / columns
  int ws_off;    // float offset of the weight area (multiple of 4: 16-byte aligned)
  uint32_t x_bytes, w_bytes, b_bytes, y_bytes;
};

// Byte offset of element (n, c, t, h, w) of an activation tensor with C
// channels: plain [N][C][T][H][W], or channel-packed
// [N][ceil(C/g)][T][H][W][g] with g = 16 / EB.
template <int EB>
__device__ __forceinline__ int act_offset(int cpack, int n, int C, int c, int T, int t, int H,
                                          int h, int W, int w) {
  if (cpack) {
    constexpr int g = 16 / EB;
    const int cg = (C + g - 1) / g;
    return (((((n * cg + c / g) * T + t) * H + h) * W + w) * g + c % g) * EB;
  }
  return ((((n * C + c) * T + t) * H + h) * W + w) * EB;
}

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
            const int off = act_offset<eb>(a.cpack, n, a.C, ci0 + c, a.T, it, a.H, ih, a.W, iw);
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
  // channel-packed output: the channels past C_out in the last group are
  // written too (as 0: their weights and bias read 0)
  const int k_store = a.cpack ? (a.K + 16 / eb - 1) / (16 / eb) * (16 / eb) : a.K;
#pragma unroll
  for (int j = 0; j < COT; ++j) {
    const int co = co0 + j;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int ow = ow0 + p * 64 + lane;
      if (co < k_store && ow < a.OW)
        E::store_out(epilogue(acc[j][p], bias[j], a.relu), yr,
                 act_offset<eb>(a.cpack, n, a.K, co, a.OT, ot, a.OH, oh, a.OW, ow));
    }
  }
}

// ------------------------------------------------------------- tap kernels
// Small fixed geometries (KH x KW taps, strides SH x SW, one frame tap):
// the tap loops are unrolled at compile time; the weights of the
// workgroup's COT output channels are wave-uniform, so they are read with
// scalar loads and used straight from scalar registers (no LDS traffic for
// them); each lane keeps R output rows x COT channels of one output column,
// so every input value it reads from LDS feeds up to R*COT fused
// multiply-adds.  A workgroup is 4 waves stacked in rows: 4R output rows x
// 64 columns.  The input halo of a channel chunk is staged in LDS as fp32,
// read as aligned 16-byte runs when the row length allows (VX), else element
// by element; positions outside the input are zero (the padding).
struct TapArgs {
  const void* x;
  const void* w;
  const void* b;
  void* y;
  int N, C, T, H, W, K;
  int ph, pw;
  int OH, OW;
  int relu;
  int col_tiles, row_tiles, co_tiles;
  int cc;  // input channels per LDS stage
  uint32_t x_bytes, y_bytes;
};

// Wait until at most N of this wave's vector-memory reads are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; the other counters
// left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-over: this wave's LDS writes complete, then
// s_barrier.  Unlike __syncthreads() it does not wait for outstanding global
// reads, so the next channel's reads stay in flight; the "memory" clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wave-uniform reads of a read-only tensor through the scalar cache: a
// pointer into the constant address space, so that reads at constant
// offsets from one pointer become wide scalar loads.  Every caller keeps its
// reads inside the tensor.
template <int DT>
struct Uniform {
  using raw = typename std::conditional<DT == DT_F32, float, uint16_t>::type;
  using ptr = const __attribute__((address_space(4))) raw*;
  __device__ static __forceinline__ ptr at(const void* base, unsigned elem) {
    return (ptr)(const __attribute__((address_space(1))) raw*)base + elem;
  }
  __device__ static __forceinline__ float get(ptr p, int i) {
    if constexpr (DT == DT_F32)
      return p[i];
    else if constexpr (DT == DT_F16)
      return (float)__builtin_bit_cast(_Float16, p[i]);
    else
      return __builtin_bit_cast(float, (uint32_t)p[i] << 16);
  }
};

template <int DT, int KH, int KW, int SH, int SW, int COT, int R, int VX>
struct TapCfg {
  static constexpr int EB = Elem<DT>::bytes;
  static constexpr int ROWS = 4 * R;               // output rows per workgroup
  static constexpr int HR = (ROWS - 1) * SH + KH;  // halo rows
  static constexpr int HC = 63 * SW + KW;          // halo columns
  static constexpr int RUN = 16 / EB;              // elements per 16-byte read
  // LDS row length in floats: VX rows start at an aligned run up to RUN-1
  // columns left of the first halo column
  static constexpr int XC = VX ? (HC + 2 * (RUN - 1)) / RUN * RUN : HC;
  static constexpr int NRUN = XC / RUN;
  static constexpr int UNITS_PER_C = VX ? HR * NRUN : HR * HC;
  static constexpr int BATCH = VX ? 8 : 16;        // reads in flight per lane while staging
  static constexpr int SPAN = (R - 1) * SH + KH;   // halo rows one wave reads
};

template <int DT, int KH, int KW, int SH, int SW, int COT, int R, int VX>
__global__ __launch_bounds__(kThreads) void tap_kernel(TapArgs a) {
  using G = TapCfg<DT, KH, KW, SH, SW, COT, R, VX>;
  using E = Elem<DT>;
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // tile: output-channel tile fastest, then column, row, frame, image; the
  // workgroups of consecutive tiles (which share input rows) are gathered on
  // one XCD (the hardware deals workgroups to the 8 XCDs round-robin)
  const int G_ = gridDim.x;
  int t = blockIdx.x;
  if ((G_ & 7) == 0) t = (t & 7) * (G_ >> 3) + (t >> 3);
  const int cot = t % a.co_tiles;
  t /= a.co_tiles;
  const int ct = t % a.col_tiles;
  t /= a.col_tiles;
  const int rt = t % a.row_tiles;
  t /= a.row_tiles;
  const int fr = t % a.T;
  const int n = t / a.T;
  const int co0 = cot * COT;
  const int oh0 = rt * G::ROWS;
  const int ow0 = ct * 64;
  const int ih0 = oh0 * SH - a.ph;
  const int iw0 = ow0 * SW - a.pw;
  const int shift = VX ? (iw0 & (G::RUN - 1)) : 0;
  const int hw = a.H * a.W;
  const int plane = a.T * hw;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_bytes);

  // weight row of each output channel (clamped: channels past C_out read a
  // real row and are not stored)
  constexpr int TAPS = KH * KW;
  using U = Uniform<DT>;
  unsigned wrow[COT];
#pragma unroll
  for (int j = 0; j < COT; ++j) wrow[j] = (unsigned)(min(co0 + j, a.K - 1) * a.C * TAPS);

  float acc[R][COT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < COT; ++j) acc[r][j] = 0.0f;

  // Staging, one input channel at a time: each lane reads SLOTS units of a
  // channel's halo (offsets computed once; the channel moves the scalar
  // offset), the reads of channel c+1 are in flight while channel c is
  // written to LDS and multiplied.
  constexpr int SLOTS = (G::UNITS_PER_C + kThreads - 1) / kThreads;
  int voff[SLOTS], loff[SLOTS];  // global byte offset (or out of range), LDS float offset (or -1)
#pragma unroll
  for (int k = 0; k < SLOTS; ++k) {
    const int u = k * kThreads + tid;
    int hr, col;
    if constexpr (VX) {
      hr = u / G::NRUN;
      col = (u % G::NRUN) * G::RUN;
    } else {
      hr = u / G::HC;
      col = u % G::HC;
    }
    const int ih = ih0 + hr, iw = iw0 - shift + col;
    const bool live = u < G::UNITS_PER_C;
    const bool ok = live && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
    voff[k] = guard_offset(true, ok ? (((n * a.C) * a.T + fr) * hw + ih * a.W + iw) * G::EB
                                    : kFarOffset);
    loff[k] = live ? hr * G::XC + col : -1;
  }
  using XR = typename std::conditional<VX, u32x4_t, float>::type;
  const int cstride = plane * G::EB;  // bytes between input channels
  auto load_c = [&](XR (&v)[SLOTS], int ci) {
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
      if constexpr (VX)
        v[k] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(xr, voff[k], ci * cstride, 0));
      else
        v[k] = E::bits_to_f32(E::load_raw(xr, voff[k] + ci * cstride));
    }
  };
  auto store_c = [&](const XR (&v)[SLOTS], float* region) {
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) {
      if (loff[k] < 0) continue;
      float* dst = region + loff[k];
      if constexpr (!VX) {
        *dst = v[k];
      } else if constexpr (G::EB == 4) {
        *reinterpret_cast<u32x4_t*>(dst) = v[k];
      } else {
        float4_t lo, hi;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          lo[2 * m] = E::bits_to_f32(v[k][m] & 0xffffu);
          lo[2 * m + 1] = E::bits_to_f32(v[k][m] >> 16);
          hi[2 * m] = E::bits_to_f32(v[k][m + 2] & 0xffffu);
          hi[2 * m + 1] = E::bits_to_f32(v[k][m + 2] >> 16);
        }
        *reinterpret_cast<float4_t*>(dst) = lo;
        *reinterpret_cast<float4_t*>(dst + 4) = hi;
      }
    }
  };
  // the multiply-adds of input channel ci, whose halo is in `region`
  auto compute_c = [&](const float* region, int ci) {
    const float* xc = region + wave * R * SH * G::XC + shift + lane * SW;
    typename U::ptr wp[COT];  // the TAPS weights of channel ci, per output channel
#pragma unroll
    for (int j = 0; j < COT; ++j) wp[j] = U::at(a.w, wrow[j] + (unsigned)(ci * TAPS));
#pragma unroll
    for (int ihr = 0; ihr < G::SPAN; ++ihr) {
      float xv[KW];
#pragma unroll
      for (int kw = 0; kw < KW; ++kw) xv[kw] = xc[ihr * G::XC + kw];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int kh = ihr - r * SH;
        if (kh < 0 || kh >= KH) continue;  // resolved at compile time
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
#pragma unroll
          for (int j = 0; j < COT; ++j)
            acc[r][j] = fmaf(xv[kw], U::get(wp[j], kh * KW + kw), acc[r][j]);
      }
    }
  };

  XR v[SLOTS];
  constexpr int CF = G::HR * G::XC;  // LDS floats per channel
  for (int ci0 = 0; ci0 < a.C; ci0 += a.cc) {
    const int cc = min(a.cc, a.C - ci0);
    if (ci0 > 0) __syncthreads();  // the previous chunk's LDS is consumed
    load_c(v, ci0);
    for (int c = 0; c < cc; ++c) {
      // channel c to LDS, then channel c+1's reads go out (into the same
      // registers, which the LDS writes have consumed) and stay in flight
      // while channel c is multiplied
      wait_vmcnt<0>();
      store_c(v, smem + c * CF);
      if (c + 1 < cc) load_c(v, ci0 + c + 1);
      lds_barrier();
      compute_c(smem + c * CF, ci0 + c);
    }
  }

  // epilogue: bias (uniform), activation, one rounding, row-contiguous stores
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, a.y_bytes);
  const int ow = ow0 + lane;
#pragma unroll
  for (int j = 0; j < COT; ++j) {
    const int co = co0 + j;
    const float bias = a.b ? U::get(U::at(a.b, (unsigned)min(co, a.K - 1)), 0) : 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int oh = oh0 + wave * R + r;
      if (co < a.K && oh < a.OH && ow < a.OW)
        E::store_out(epilogue(acc[r][j], bias, a.relu), yr,
                 ((((n * a.K + co) * a.T + fr) * a.OH + oh) * a.OW + ow) * G::EB);
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

// ---- tap kernels: table, geometry, launch
using TapLaunch = hipError_t (*)(const TapArgs&, unsigned, int, hipStream_t);

template <int DT, int KH, int KW, int SH, int SW, int COT, int R, int VX>
hipError_t launch_tap(const TapArgs& a, unsigned grid, int lds, hipStream_t s) {
  hipLaunchKernelGGL((tap_kernel<DT, KH, KW, SH, SW, COT, R, VX>), dim3(grid), dim3(kThreads),
                     lds, s, a);
  return hipGetLastError();
}

struct TapTile {
  int id, KH, KW, SH, SW, cot, R, vx;
  const char* name;
  TapLaunch fn[3];  // by libconv_dtype
};

#define LIBCONV_TAP(ID, KH, KW, SH, SW, COT, R, VX, NAME)                            \
  {ID, KH, KW, SH, SW, COT, R, VX, NAME,                                             \
   {&launch_tap<DT_F32, KH, KW, SH, SW, COT, R, VX>,                                 \
    &launch_tap<DT_F16, KH, KW, SH, SW, COT, R, VX>,                                 \
    &launch_tap<DT_BF16, KH, KW, SH, SW, COT, R, VX>}}

const TapTile kTapTiles[] = {
    LIBCONV_TAP(150, 3, 3, 1, 1, 8, 2, 1, "tap_k3s1_cot8_r2"),
    LIBCONV_TAP(151, 3, 3, 1, 1, 8, 2, 0, "tap_k3s1_cot8_r2_e"),
    LIBCONV_TAP(152, 3, 3, 2, 2, 8, 2, 1, "tap_k3s2_cot8_r2"),
    LIBCONV_TAP(153, 3, 3, 2, 2, 8, 2, 0, "tap_k3s2_cot8_r2_e"),
    LIBCONV_TAP(154, 1, 1, 1, 1, 8, 2, 1, "tap_k1_cot8_r2"),
    LIBCONV_TAP(155, 1, 1, 1, 1, 8, 2, 0, "tap_k1_cot8_r2_e"),
    LIBCONV_TAP(160, 3, 3, 1, 1, 16, 1, 1, "tap_k3s1_cot16_r1"),
    LIBCONV_TAP(162, 3, 3, 2, 2, 16, 1, 1, "tap_k3s2_cot16_r1"),
    LIBCONV_TAP(164, 1, 1, 1, 1, 16, 1, 1, "tap_k1_cot16_r1"),
    LIBCONV_TAP(166, 3, 3, 1, 1, 4, 4, 1, "tap_k3s1_cot4_r4"),
    LIBCONV_TAP(168, 3, 3, 2, 2, 4, 4, 1, "tap_k3s2_cot4_r4"),
};

#undef LIBCONV_TAP

constexpr int kTapLdsBudget = 32 * 1024;  // bytes of LDS per workgroup (several per CU)

const TapTile* find_tap(int id) {
  for (const auto& t : kTapTiles)
    if (t.id == id) return &t;
  return nullptr;
}

// LDS floats per input channel of a tap tile (mirrors TapCfg).
long tap_floats_per_channel(const TapTile& t, int dtype) {
  const int run = 16 / dtype_bytes(dtype);
  const int hr = (4 * t.R - 1) * t.SH + t.KH;
  const int hc = 63 * t.SW + t.KW;
  const int xc = t.vx ? (hc + 2 * (run - 1)) / run * run : hc;
  return (long)hr * xc;
}

bool tap_fits(const TapTile& t, const Problem& p) {
  if (p.cpack) return false;  // plain layout only
  if (p.KT != 1 || p.st != 1 || p.pt != 0 || p.ptb != 0) return false;
  if (p.KH != t.KH || p.KW != t.KW || p.sh != t.SH || p.sw != t.SW) return false;
  if (t.vx) {
    const int run = 16 / dtype_bytes(p.dtype);
    if (p.W % run != 0 || (reinterpret_cast<uintptr_t>(p.x) & 15) != 0) return false;
  }
  return tap_floats_per_channel(t, p.dtype) * 4 <= kTapLdsBudget;
}

long long tap_grid(const TapTile& t, const Problem& p) {
  const long long cols = (p.OW + 63) / 64;
  const long long rows = (p.OH + 4 * t.R - 1) / (4 * t.R);
  const long long cot = (p.K + t.cot - 1) / t.cot;
  return (long long)p.N * p.T * rows * cols * cot;
}

// Among the tap tiles that fit, the one with the least padded work per
// compute unit: rounds of workgroups on 256 CUs (4 resident per CU) times the
// outputs of one workgroup.  Ties go to the earlier tile of the table.
const TapTile* tap_choose(const Problem& p) {
  const TapTile* best = nullptr;
  double best_cost = 0.0;
  for (const auto& t : kTapTiles) {
    if (!tap_fits(t, p)) continue;
    const double g = (double)tap_grid(t, p);
    const double rounds = std::ceil(g / (256.0 * 4.0));
    const double cost = rounds * 4.0 * t.R * 64.0 * t.cot;
    if (!best || cost < best_cost) {
      best = &t;
      best_cost = cost;
    }
  }
  return best;
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
  if (t) return t->name;
  const TapTile* tt = find_tap(id);
  return tt ? tt->name : nullptr;
}

bool direct_plan_tile(const Problem& p, int tile_id, Plan* plan) {
  if (p.pool) return false;
  const TapTile* t = find_tap(tile_id);
  if (!t || !tap_fits(*t, p)) return false;
  plan->algo = LIBCONV_ALGO_DIRECT;
  plan->tile = t->id;
  plan->grid = tap_grid(*t, p);
  return true;
}

bool direct_plan(const Problem& p, Plan* plan) {
  if (p.pool) return false;  // the fused max pooling lives in the MFMA epilogue only
  if (const TapTile* t = tap_choose(p)) {
    plan->algo = LIBCONV_ALGO_DIRECT;
    plan->tile = t->id;
    plan->grid = tap_grid(*t, p);
    return true;
  }
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

static libconv_status tap_launch(const Problem& p, const TapTile& t) {
  if (!tap_fits(t, p)) return LIBCONV_ERR_UNSUPPORTED;
  TapArgs a;
  a.x = p.x; a.w = p.w; a.b = p.b; a.y = p.y;
  a.N = p.N; a.C = p.C; a.T = p.T; a.H = p.H; a.W = p.W; a.K = p.K;
  a.ph = p.ph; a.pw = p.pw; a.OH = p.OH; a.OW = p.OW;
  a.relu = p.act == LIBCONV_ACT_RELU;
  a.col_tiles = (p.OW + 63) / 64;
  a.row_tiles = (p.OH + 4 * t.R - 1) / (4 * t.R);
  a.co_tiles = (p.K + t.cot - 1) / t.cot;
  const long per_c = tap_floats_per_channel(t, p.dtype);
  a.cc = (int)std::min<long>(p.C, std::max<long>(1, kTapLdsBudget / (per_c * 4)));
  const int eb = dtype_bytes(p.dtype);
  a.x_bytes = (uint32_t)((long long)p.N * p.C * p.T * p.H * p.W * eb);
  a.y_bytes = (uint32_t)((long long)p.N * p.K * p.OT * p.OH * p.OW * eb);
  const long long grid = tap_grid(t, p);
  if (grid > 0x7fffffffLL) return LIBCONV_ERR_UNSUPPORTED;
  const hipError_t e = t.fn[p.dtype](a, (unsigned)grid, (int)(a.cc * per_c * 4), p.stream);
  return e == hipSuccess ? LIBCONV_OK : LIBCONV_ERR_LAUNCH;
}

libconv_status direct_launch(const Problem& p, const Plan& plan) {
  if (const TapTile* tt = find_tap(plan.tile)) return tap_launch(p, *tt);
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
  a.cpack = p.cpack ? 1 : 0;
  const int eb = dtype_bytes(p.dtype);
  a.x_bytes = (uint32_t)(p.cpack ? cpack_bytes(p.N, p.C, (long long)p.T * p.H * p.W, p.dtype)
                                 : (long long)p.N * p.C * p.T * p.H * p.W * eb);
  a.w_bytes = (uint32_t)((long long)p.K * p.C * p.KT * p.KH * p.KW * eb);
  a.b_bytes = p.b ? (uint32_t)(p.K * eb) : 0u;
  a.y_bytes = (uint32_t)(p.cpack ? cpack_bytes(p.N, p.K, (long long)p.OT * p.OH * p.OW, p.dtype)
                                 : (long long)p.N * p.K * p.OT * p.OH * p.OW * eb);
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
