// igemm.hip -- implicit-GEMM convolution on the gfx950 matrix cores (MFMA).
//
// The convolution of the page "PP-OCR on Vulkan compute shaders" (section
// 2.2; the frame axis as in the Convolution3D layer of "SeedVR2 NCNN Vulkan",
// section 3.2) is, for wide layers, a dense contraction:
//     Y[co][px] = sum_k Wm[co][k] * Xcol[k][px],   k = (ci, kt, kh, kw)
// with Xcol the zero-padded input window of each output pixel (im2col).  The
// im2col matrix is never materialised in memory: each workgroup stages the
// input halo of its pixel tile in LDS and the MFMA operands are read from it
// at per-tap offsets.
//
// Workgroup tile: BM output channels x (TH x TW) output pixels of one output
// plane (n, ot); four waves in a WM x WN grid, each owning (BM/WM) x (BN/WN)
// outputs as 32x32 MFMA blocks held in fp32 accumulators.
//
// K loop: one stage = CK = CG * SE input channels (SE = 8 for 16-bit types,
// 4 for fp32: one 16-byte "slot") at one frame tap kt, with all KH x KW
// spatial taps.  Stages whose input frame lies wholly in the time padding are
// skipped (they contribute zero).  Per stage:
//   * weights land in LDS as Wl[slot][co][SE], slot = tap*CG + g (the SE
//     channels of group g at one spatial tap, for each output channel):
//       - from OIHW weights (2-D tiles): each thread reads one channel's
//         KH*KW contiguous 16-byte vectors and transposes them in registers
//         (16-byte LDS stores, lanes on consecutive channels);
//       - from packed weights ([C/SE][taps][C_out padded][SE], made by the
//         pack kernel below -- the per-layer weight packing of the
//         Convolution3D work in "SeedVR2 NCNN Vulkan", section 3.2): a stage
//         is NSLOT contiguous runs copied straight into LDS by direct-to-LDS
//         loads (no registers, no arithmetic);
//   * the input halo (HR rows x HC cols of one frame) is read
//     row-contiguously and written channel-innermost as Xl[g][hr][hc][SE];
//     taps outside the input are zero (this is the padding);
//   * the stage's slots are consumed in pairs by one MFMA k-step (32x32x16
//     f16/bf16: lanes 0-31 carry slot 2p, lanes 32-63 slot 2p+1) or by four
//     (32x32x2 f32, one element of each slot per step).  Both operands of a
//     slot are single 16-byte LDS reads.
// LDS holds two stages; the global loads of stage s+1 are in flight while
// stage s is multiplied.  Each lane's load offsets are computed once; the
// per-stage part of every address is wave-uniform and moves the base of the
// buffer descriptor (scalar arithmetic), so staging costs almost no vector
// arithmetic and every access stays range-checked.
//
// Epilogue (shared with the direct kernel): fp32 accumulator + bias ->
// optional ReLU -> one round-to-nearest-even conversion -> store, with the
// 32 lanes of a half-wave writing 32 consecutive output pixels of one
// channel.  Every output element has exactly one writer.
#include "device_common.h"
#include "internal.h"

namespace libconv {
namespace {

constexpr int kThreads = 256;
constexpr int kPackAlign = 128;   // output channels of packed weights are padded to this
constexpr int kFar = 0x7ffffff0;  // offset past the end of every tensor (all are < 0x7fff0000 bytes)

// One MFMA k-step over a pair of 16-byte slots.  KSUB is the number of
// instructions a slot pair takes; step(.., k) issues sub-step k.
template <int DT> struct Mma;

template <> struct Mma<DT_F16> {
  static constexpr int SE = 8;  // elements per 16-byte slot
  static constexpr int KSUB = 1;
  __device__ static __forceinline__ void step(const u32x4_t& a, const u32x4_t& b, float16_t& c,
                                              int) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                               __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
};

template <> struct Mma<DT_BF16> {
  static constexpr int SE = 8;
  static constexpr int KSUB = 1;
  __device__ static __forceinline__ void step(const u32x4_t& a, const u32x4_t& b, float16_t& c,
                                              int) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};

// fp32: 32x32x2, lanes 0-31 give K index 0 (slot 2p), lanes 32-63 K index 1
// (slot 2p+1); sub-step k multiplies element k of both slots.  The fragment
// is reinterpreted as a whole float4 before indexing: bit-casting a single
// vector element has been seen to compile to element 0 for every k.
template <> struct Mma<DT_F32> {
  static constexpr int SE = 4;
  static constexpr int KSUB = 4;
  __device__ static __forceinline__ void step(const u32x4_t& a, const u32x4_t& b, float16_t& c,
                                              int k) {
    const float4_t af = __builtin_bit_cast(float4_t, a);
    const float4_t bf = __builtin_bit_cast(float4_t, b);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[k], bf[k], c, 0, 0, 0);
  }
};

struct IgemmArgs {
  const void* x;
  const void* w;      // OIHW weights, or packed weights when the tile is packed
  const void* b;
  void* y;
  int N, C, T, H, W, K;
  int OT, OH, OW;
  int pt, ph, pw;
  int st;             // time stride (the spatial strides are template parameters)
  int relu;
  int chunks;         // ceil(C / CK)
  int kp;             // packed weights: output-channel stride (C_out rounded up)
  int co_tiles, row_tiles, col_tiles;
  uint32_t x_bytes, w_bytes, b_bytes, y_bytes;
};

template <int DT_, int KT_, int KH_, int KW_, int SH_, int SW_, int BM_, int TH_, int TW_,
          int WM_, int WN_, int CG_, int PK_>
struct Cfg {
  static constexpr int DT = DT_, KT = KT_, KH = KH_, KW = KW_, SH = SH_, SW = SW_;
  static constexpr int BM = BM_, TH = TH_, TW = TW_, WM = WM_, WN = WN_, CG = CG_;
  static constexpr bool PK = PK_ != 0;
  static constexpr int EB = Elem<DT>::bytes;
  static constexpr int SE = Mma<DT>::SE;
  static constexpr int CK = CG * SE;
  static constexpr int TS = KT * KH * KW;          // all taps (weight layout)
  static constexpr int TS2 = KH * KW;              // spatial taps of one stage
  static constexpr int NSLOT = TS2 * CG;
  static constexpr int NPAIR = (NSLOT + 1) / 2;
  static constexpr int BN = TH * TW;
  static constexpr int HR = (TH - 1) * SH + KH;
  static constexpr int HC = (TW - 1) * SW + KW;
  static constexpr int XPLANE = HR * HC;           // halo pixels per channel group
  static constexpr int WBYTES = NSLOT * BM * 16;
  static constexpr int XBYTES = CG * XPLANE * 16;
  static constexpr int BUF = WBYTES + XBYTES;
  static constexpr int LDS = 2 * BUF;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FA = WTM / 32, FB = WTN / 32;
  static constexpr int BPR = TW / 32;              // 32-pixel blocks per tile row
  // weight staging from OIHW: one unit = one output channel x one group of
  // SE input channels = TS contiguous 16-byte vectors; unit u = g * BM + channel
  static constexpr int WUNITS = PK ? 0 : BM * CG;
  static constexpr int WPASS = PK ? 0 : (WUNITS + kThreads - 1) / kThreads;
  // weight staging from packed weights: NSLOT runs of BM 16-byte vectors,
  // moved as 1 KB chunks (one wave, one instruction each)
  static constexpr int WCHUNKS = NSLOT * BM / 64;
  // input staging: one unit = one halo pixel of one channel group
  static constexpr int XUNITS = CG * XPLANE;
  static constexpr int XPASS = (XUNITS + kThreads - 1) / kThreads;

  static_assert(WM * WN == 4, "four waves");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(TW % 32 == 0, "tile rows are whole 32-pixel blocks");
  static_assert(BM % 64 == 0 || !PK, "packed tiles move whole 64-channel chunks");
  static_assert(BM <= kPackAlign, "packed channel padding covers one tile");
  static_assert(PK || KT == 1, "weights from OIHW: 2-D tiles only");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Global -> registers for one stage (weights only when they are transposed
// here; packed weights go straight to LDS).  Input elements are kept exactly
// as loaded and only packed into 16-byte words when they are written to LDS,
// after the current stage's MFMAs: any arithmetic on them right after the
// loads would make the wave wait for the loads before computing.
template <class G>
struct StageRegs {
  u32x4_t wv[G::WPASS > 0 ? G::WPASS : 1][G::TS];
  uint32_t xe[G::XPASS][G::SE];
};

// Slot vector of tap t from a unit's TS vectors: the unit holds
// w[co][c0 .. c0+SE)[0 .. TS) with the tap index fastest; the slot wants the
// SE channels of one tap.  All indices are compile-time, so this is register
// selection (fp32) or one byte permute per output word (16-bit).
template <int SE, int TS, int t>
__device__ __forceinline__ u32x4_t transpose_slot(const u32x4_t (&v)[TS]) {
  u32x4_t o;
  if constexpr (SE == 4) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = m * TS + t;
      o[m] = v[e / 4][e % 4];
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e0 = (2 * m) * TS + t, e1 = (2 * m + 1) * TS + t;
      const uint32_t d0 = v[e0 / 8][(e0 % 8) / 2];
      const uint32_t d1 = v[e1 / 8][(e1 % 8) / 2];
      const uint32_t lo = (e0 & 1) ? (d0 >> 16) : (d0 & 0xffffu);
      const uint32_t hi = (e1 & 1) ? (d1 & 0xffff0000u) : (d1 << 16);
      o[m] = lo | hi;
    }
  }
  return o;
}

// LDS stores of the TS slot vectors of one unit (t = 0 .. TS-1).
template <int SE, int TS, int t>
__device__ __forceinline__ void store_slots(unsigned char* base, int slot_stride,
                                            const u32x4_t (&v)[TS]) {
  if constexpr (t < TS) {
    *reinterpret_cast<u32x4_t*>(base + t * slot_stride) = transpose_slot<SE, TS, t>(v);
    store_slots<SE, TS, t + 1>(base, slot_stride, v);
  }
}

template <class G>
__global__ __launch_bounds__(kThreads) void igemm_kernel(IgemmArgs a) {
  using E = Elem<G::DT>;
  constexpr int EB = G::EB;
  constexpr int SE = G::SE;
  __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int il = lane & 31;   // row (A) / column (B) inside a 32x32 block
  const int hf = lane >> 5;   // which slot of the pair this lane carries

  // ---- tile coordinates; XCD-aware order: the hardware deals workgroups to
  // the 8 XCDs round-robin, so consecutive logical tiles (same output-channel
  // tile, neighbouring pixel tiles) are gathered onto one XCD and its L2.
  const int G_ = gridDim.x;
  int bid = blockIdx.x;
  if ((G_ & 7) == 0) bid = (bid & 7) * (G_ >> 3) + (bid >> 3);
  const int ctile = bid % a.col_tiles;
  bid /= a.col_tiles;
  const int rtile = bid % a.row_tiles;
  bid /= a.row_tiles;
  const int ot = bid % a.OT;
  bid /= a.OT;
  const int n = bid % a.N;
  const int cot = bid / a.N;
  const int co0 = cot * G::BM;
  const int oh0 = rtile * G::TH;
  const int ow0 = ctile * G::TW;
  const int ih0 = oh0 * G::SH - a.ph;
  const int iw0 = ow0 * G::SW - a.pw;
  const int it0 = ot * a.st - a.pt;
  // frame taps whose input frame exists; the others are time padding
  const int kt_lo = it0 < 0 ? -it0 : 0;
  const int kt_hi = min(G::KT, a.T - it0);
  const int nkt = kt_hi > kt_lo ? kt_hi - kt_lo : 0;
  const int nstages = a.chunks * nkt;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);

  const int hw = a.H * a.W;
  const int plane = a.T * hw;            // elements between input channels in x

  // ---- per-lane, stage-invariant load offsets (bytes).  The per-stage part
  // of every address is wave-uniform: it moves the base of the buffer
  // descriptor (scalar arithmetic), while the range check keeps covering
  // every access up to the end of the tensor.
  // input halo unit u = (g * HR + hr) * HC + hc, channel j of its group
  int xoff[G::XPASS][SE];                // kFar when the position is padding
  int xgrp[G::XPASS];
#pragma unroll
  for (int i = 0; i < G::XPASS; ++i) {
    const int u = tid + i * kThreads;
    const int hc = u % G::HC;
    const int hr = (u / G::HC) % G::HR;
    const int g = u / (G::HC * G::HR);
    const int ih = ih0 + hr, iw = iw0 + hc;
    const bool ok = u < G::XUNITS && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
#pragma unroll
    for (int j = 0; j < SE; ++j)
      xoff[i][j] = guard_offset(true, ok ? ((g * SE + j) * plane + ih * a.W + iw) * EB : kFar);
    xgrp[i] = g;
  }
  // OIHW weight unit u = g * BM + col
  int woff[G::WPASS > 0 ? G::WPASS : 1];
  int wgrp[G::WPASS > 0 ? G::WPASS : 1];
#pragma unroll
  for (int i = 0; i < G::WPASS; ++i) {
    const int u = tid + i * kThreads;
    const int g = u / G::BM, col = u % G::BM;
    const int co = co0 + col;
    const bool ok = u < G::WUNITS && co < a.K;
    woff[i] = guard_offset(true, ok ? (co * a.C * G::TS + g * SE * G::TS) * EB : kFar);
    wgrp[i] = g;
  }
  const int n_base = n * a.C * plane * EB;

  // Issue the global reads of stage (chunk, kt): packed weights straight into
  // LDS buffer `buf`, everything else into registers.
  auto load_stage = [&](int chunk, int kt, StageRegs<G>& r, unsigned char* buf) {
    const int ci0 = chunk * G::CK;
    const bool full = ci0 + G::CK <= a.C;  // uniform: no channel of the stage is past C
    if constexpr (G::PK) {
      // chunk c = 64 channels of one slot; lane l lands at chunk base + 16 l
      for (int c = wave; c < G::WCHUNKS; c += kThreads / 64) {
        const int slot = c / (G::BM / 64), part = c % (G::BM / 64);
        const int t2 = slot / G::CG, g = slot % G::CG;
        const int run = ((chunk * G::CG + g) * G::TS + kt * G::TS2 + t2) * a.kp + co0 + part * 64;
        unsigned char* dst = buf + (slot * G::BM + part * 64) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (__attribute__((address_space(3))) void*)dst,
                                                 16, (run + lane) * 16, 0, 0, 0);
      }
    } else {
      const int sb = ci0 * G::TS * EB;
      const __amdgpu_buffer_rsrc_t ws = make_rsrc((const char*)a.w + sb, a.w_bytes - sb);
#pragma unroll
      for (int i = 0; i < G::WPASS; ++i) {
        int v = woff[i];
        if (!full && ci0 + wgrp[i] * SE >= a.C) v = guard_offset(true, kFar);
#pragma unroll
        for (int k = 0; k < G::TS; ++k)
          r.wv[i][k] = __builtin_bit_cast(
              u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ws, v + k * 16, 0, 0));
      }
    }
    const int sb = n_base + (ci0 * plane + (it0 + kt) * hw) * EB;
    const __amdgpu_buffer_rsrc_t xs = make_rsrc((const char*)a.x + sb, a.x_bytes - sb);
#pragma unroll
    for (int i = 0; i < G::XPASS; ++i) {
#pragma unroll
      for (int j = 0; j < SE; ++j) {
        int v = xoff[i][j];
        if (!full && ci0 + xgrp[i] * SE + j >= a.C) v = guard_offset(true, kFar);
        r.xe[i][j] = E::load_bits(xs, v);
      }
    }
  };

  auto store_stage = [&](const StageRegs<G>& r, unsigned char* buf) {
    // weights from OIHW: [ci][tap] per unit -> Wl[slot = tap * CG + g][co][SE];
    // lanes of a wave hold consecutive channels, so each 16-byte store is
    // conflict-free
#pragma unroll
    for (int i = 0; i < G::WPASS; ++i) {
      const int u = tid + i * kThreads;
      if (u < G::WUNITS)
        store_slots<SE, G::TS, 0>(buf + ((u / G::BM) * G::BM + u % G::BM) * 16,
                                  G::CG * G::BM * 16, r.wv[i]);
    }
    // input halo: pack the SE channels of each unit into one 16-byte word
    unsigned char* xbuf = buf + G::WBYTES;
#pragma unroll
    for (int i = 0; i < G::XPASS; ++i) {
      const int u = tid + i * kThreads;
      const uint32_t* e = r.xe[i];
      u32x4_t v;
      if constexpr (SE == 8)
        v = u32x4_t{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                    e[6] | (e[7] << 16)};
      else
        v = u32x4_t{e[0], e[1], e[2], e[3]};
      if (u < G::XUNITS) *reinterpret_cast<u32x4_t*>(xbuf + u * 16) = v;
    }
  };

  // ---- MFMA operand addressing
  const int wm = wave % G::WM;
  const int wn = wave / G::WM;
  const int co_w0 = wm * G::WTM;
  const int blk0 = wn * G::FB;                       // first 32-pixel block of this wave
  const int prow0 = blk0 / G::BPR, pcol0 = (blk0 % G::BPR) * 32;
  // A: Wl[slot][co][16 B]; lanes of half hf read slot 2p + hf.
  const int a_lane = ((hf * G::BM) + co_w0 + il) * 16;
  // B: Xl[g][hr][hc][16 B] at the lane's pixel.
  const int b_lane = ((prow0 * G::SH) * G::HC + (pcol0 + il) * G::SW) * 16;

  float16_t acc[G::FA][G::FB];
#pragma unroll
  for (int i = 0; i < G::FA; ++i)
#pragma unroll
    for (int j = 0; j < G::FB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // byte offset of slot s inside the halo area (pixel (0,0) of the tile)
  auto xslot = [](int s) constexpr -> int {
    const int tap = s / G::CG, g = s % G::CG;
    const int kh = tap / G::KW;
    const int kw = tap % G::KW;
    return ((g * G::HR + kh) * G::HC + kw) * 16;
  };
  // byte offset of block j of this wave relative to its first block
  auto xblock = [&](int j) -> int {
    const int b = blk0 + j;
    const int r = b / G::BPR, c = (b % G::BPR) * 32;
    return ((r - prow0) * G::SH * G::HC + (c - pcol0) * G::SW) * 16;
  };

  auto compute = [&](const unsigned char* buf) {
    const unsigned char* wl = buf;
    const unsigned char* xl = buf + G::WBYTES;
    u32x4_t fa[2][G::FA], fb[2][G::FB];
    auto load_frags = [&](int p, int k) {
      const int s0 = 2 * p;
      const int s1 = (2 * p + 1 < G::NSLOT) ? 2 * p + 1 : 2 * p;
      const int xo = hf ? xslot(s1) : xslot(s0);
#pragma unroll
      for (int i = 0; i < G::FA; ++i)
        fa[k][i] = *reinterpret_cast<const u32x4_t*>(wl + a_lane + (s0 * G::BM + i * 32) * 16);
#pragma unroll
      for (int j = 0; j < G::FB; ++j)
        fb[k][j] = *reinterpret_cast<const u32x4_t*>(xl + b_lane + xo + xblock(j));
      if (2 * p + 1 >= G::NSLOT && hf) {
        // odd slot count: the second half of the last pair carries nothing
#pragma unroll
        for (int i = 0; i < G::FA; ++i) fa[k][i] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < G::FB; ++j) fb[k][j] = u32x4_t{0u, 0u, 0u, 0u};
      }
    };
    load_frags(0, 0);
#pragma unroll
    for (int p = 0; p < G::NPAIR; ++p) {
      if (p + 1 < G::NPAIR) load_frags(p + 1, (p + 1) & 1);
#pragma unroll
      for (int k = 0; k < Mma<G::DT>::KSUB; ++k)
#pragma unroll
        for (int i = 0; i < G::FA; ++i)
#pragma unroll
          for (int j = 0; j < G::FB; ++j)
            Mma<G::DT>::step(fa[p & 1][i], fb[p & 1][j], acc[i][j], k);
    }
  };

  // ---- main loop over stages (chunk, kt), chunk-major: two LDS buffers,
  // the next stage's global reads in flight during the current MFMAs
  if (nstages > 0) {
    StageRegs<G> regs;
    int chunk = 0, kt = kt_lo;
    load_stage(chunk, kt, regs, lds);
    store_stage(regs, lds);
    __builtin_amdgcn_s_waitcnt(0);  // direct-to-LDS copies are counted as loads
    __syncthreads();
    for (int s = 0; s < nstages; ++s) {
      unsigned char* cur = lds + (s & 1) * G::BUF;
      unsigned char* nxt = lds + ((s + 1) & 1) * G::BUF;
      const bool more = s + 1 < nstages;
      if (more) {
        if (++kt == kt_hi) {
          kt = kt_lo;
          ++chunk;
        }
        load_stage(chunk, kt, regs, nxt);
      }
      compute(cur);
      if (more) store_stage(regs, nxt);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- epilogue
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, a.y_bytes);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.b, a.b_bytes);
  const int ohw = a.OH * a.OW;
  // All bias loads first (one round trip); channels beyond C_out read 0 and
  // are not stored.
  float bias[G::FA][16];
#pragma unroll
  for (int i = 0; i < G::FA; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int co = co0 + co_w0 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
      bias[i][r] = E::load(br, guard_offset(a.b && co < a.K, co * EB));
    }
#pragma unroll
  for (int i = 0; i < G::FA; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int co = co0 + co_w0 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
      const int cbase = ((n * a.K + co) * a.OT + ot) * ohw;
#pragma unroll
      for (int j = 0; j < G::FB; ++j) {
        const int b = blk0 + j;
        const int oh = oh0 + b / G::BPR;
        const int ow = ow0 + (b % G::BPR) * 32 + il;
        if (co < a.K && oh < a.OH && ow < a.OW)
          E::store(epilogue(acc[i][j][r], bias[i][r], a.relu), yr,
                   (cbase + oh * a.OW + ow) * EB);
      }
    }
  }
}

// ------------------------------------------------------------ weight packing
// w [K][C][TS] -> wp [G = ceil(C/SE)][TS][Kp][SE] (16 bytes per entry), zero
// for channels >= C and output channels >= K.  One thread per (output
// channel, channel group): the group's SE*TS elements are contiguous in w;
// when C is a multiple of SE they are TS aligned 16-byte vectors, otherwise
// they are read element by element.  The thread transposes them in registers
// and writes its TS slot vectors; lanes hold consecutive output channels, so
// each store instruction of a wave writes 1 KB contiguous.
struct PackArgs {
  const void* w;
  void* wp;
  int K, C, Kp, G;
  uint32_t w_bytes, wp_bytes;
};

template <int SE, int TS, int t>
__device__ __forceinline__ void store_packed(__amdgpu_buffer_rsrc_t pr, int off, int tstride,
                                             const u32x4_t (&v)[TS]) {
  if constexpr (t < TS) {
    __builtin_amdgcn_raw_buffer_store_b128(transpose_slot<SE, TS, t>(v), pr, off + t * tstride, 0,
                                           0);
    store_packed<SE, TS, t + 1>(pr, off, tstride, v);
  }
}

template <int DT, int TS>
__global__ __launch_bounds__(kThreads) void pack_kernel(PackArgs a) {
  using E = Elem<DT>;
  constexpr int SE = Mma<DT>::SE;
  constexpr int EB = E::bytes;
  const int u = blockIdx.x * kThreads + threadIdx.x;
  if (u >= a.G * a.Kp) return;
  const int g = u / a.Kp, co = u % a.Kp;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.wp, a.wp_bytes);
  const bool co_ok = co < a.K;
  const int base = (co * a.C + g * SE) * TS;  // first element of the group block
  u32x4_t v[TS];
  if (a.C % SE == 0) {
#pragma unroll
    for (int k = 0; k < TS; ++k)
      v[k] = __builtin_bit_cast(
          u32x4_t,
          __builtin_amdgcn_raw_buffer_load_b128(wr, guard_offset(co_ok, base * EB + k * 16), 0, 0));
  } else {
#pragma unroll
    for (int k = 0; k < TS; ++k) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t word = 0;
#pragma unroll
        for (int h = 0; h < 4 / EB; ++h) {
          const int e = k * SE + m * (4 / EB) + h;  // element of the [SE][TS] block
          const bool ok = co_ok && g * SE + e / TS < a.C;
          const uint32_t bits = E::load_bits(wr, guard_offset(ok, (base + e) * EB));
          word |= (EB == 2) ? ((bits & 0xffffu) << (16 * h)) : bits;
        }
        v[k][m] = word;
      }
    }
  }
  store_packed<SE, TS, 0>(pr, (g * TS * a.Kp + co) * 16, a.Kp * 16, v);
}

// ------------------------------------------------------------------ tiles
using LaunchFn = hipError_t (*)(const IgemmArgs&, unsigned, hipStream_t);

template <class G>
hipError_t launch_cfg(const IgemmArgs& a, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL(igemm_kernel<G>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

struct TileDesc {
  int id;
  int wide;       // 0: fp32 operands, 1: 16-bit operands
  int KT, KH, KW, SH, SW;
  int flat;       // 1: 1x1 stride-1 pad-0 layer viewed as one long row per plane
  int BM, TH, TW, CG;
  int packed;     // 1: reads packed weights
  int eff;        // fraction of MFMA peak one CU reaches on this tile, in percent
                  // (measured on MI355X on large grids; used to rank tiles)
  int lds;
  const char* name;
  LaunchFn fn[3];  // by libconv_dtype
};

// Launcher of a tile for one storage dtype, or null when the tile's operand
// width does not match the dtype.
template <int DT, int WIDE, int KT, int KH, int KW, int SH, int SW, int BM, int TH, int TW,
          int WM, int WN, int CG, int PK>
constexpr LaunchFn launcher() {
  if constexpr ((DT == DT_F32) == (WIDE == 0))
    return &launch_cfg<Cfg<DT, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK>>;
  else
    return nullptr;
}

#define LIBCONV_TILE(ID, WIDE, KT, KH, KW, SH, SW, FLAT, BM, TH, TW, WM, WN, CG, PK, EFF, NAME) \
  {ID, WIDE, KT, KH, KW, SH, SW, FLAT, BM, TH, TW, CG, PK, EFF,                                  \
   Cfg<WIDE ? DT_F16 : DT_F32, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK>::LDS, NAME,  \
   {launcher<DT_F32, WIDE, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK>(),               \
    launcher<DT_F16, WIDE, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK>(),               \
    launcher<DT_BF16, WIDE, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK>()}}

const TileDesc kTiles[] = {
    // 16-bit operands, 3x3 stride 1, weights transposed in the kernel
    LIBCONV_TILE(200, 1, 1, 3, 3, 1, 1, 0, 128, 8, 32, 2, 2, 2, 0, 20, "igemm16_k3s1_m128_n8x32"),
    LIBCONV_TILE(201, 1, 1, 3, 3, 1, 1, 0, 128, 4, 32, 2, 2, 2, 0, 17, "igemm16_k3s1_m128_n4x32"),
    LIBCONV_TILE(202, 1, 1, 3, 3, 1, 1, 0, 128, 2, 64, 2, 2, 2, 0, 14, "igemm16_k3s1_m128_n2x64"),
    LIBCONV_TILE(203, 1, 1, 3, 3, 1, 1, 0, 64, 8, 32, 1, 4, 2, 0, 28, "igemm16_k3s1_m64_n8x32"),
    // 16-bit operands, 3x3 stride 2
    LIBCONV_TILE(210, 1, 1, 3, 3, 2, 2, 0, 64, 4, 32, 2, 2, 2, 0, 20, "igemm16_k3s2_m64_n4x32"),
    // 16-bit operands, 1x1 stride 1 pad 0 (flattened planes)
    LIBCONV_TILE(220, 1, 1, 1, 1, 1, 1, 1, 128, 1, 256, 2, 2, 8, 0, 20, "igemm16_k1_m128_n256"),
    LIBCONV_TILE(221, 1, 1, 1, 1, 1, 1, 1, 128, 1, 128, 2, 2, 8, 0, 20, "igemm16_k1_m128_n128"),
    // fp32 operands
    LIBCONV_TILE(240, 0, 1, 3, 3, 1, 1, 0, 32, 8, 32, 1, 4, 4, 0, 50, "igemm32_k3s1_m32_n8x32"),
    LIBCONV_TILE(241, 0, 1, 3, 3, 1, 1, 0, 64, 4, 32, 2, 2, 4, 0, 40, "igemm32_k3s1_m64_n4x32"),
    LIBCONV_TILE(242, 0, 1, 3, 3, 2, 2, 0, 64, 2, 32, 2, 2, 4, 0, 35, "igemm32_k3s2_m64_n2x32"),
    LIBCONV_TILE(243, 0, 1, 1, 1, 1, 1, 1, 64, 1, 128, 2, 2, 8, 0, 15, "igemm32_k1_m64_n128"),
    // fp32, 8 channels per stage: small LDS stages, several workgroups per CU
    LIBCONV_TILE(244, 0, 1, 3, 3, 1, 1, 0, 32, 8, 32, 1, 4, 2, 0, 48, "igemm32_k3s1_m32_n8x32_c8"),
    LIBCONV_TILE(245, 0, 1, 3, 3, 2, 2, 0, 64, 2, 32, 2, 2, 2, 0, 44, "igemm32_k3s2_m64_n2x32_c8"),
    LIBCONV_TILE(246, 0, 1, 3, 3, 2, 2, 0, 64, 4, 32, 2, 2, 2, 0, 44, "igemm32_k3s2_m64_n4x32_c8"),
    LIBCONV_TILE(247, 0, 1, 3, 3, 1, 1, 0, 32, 4, 32, 1, 4, 2, 0, 48, "igemm32_k3s1_m32_n4x32_c8"),
    // packed weights: 16-bit, 3x3x3 stride 1 (one frame tap per stage)
    LIBCONV_TILE(260, 1, 3, 3, 3, 1, 1, 0, 128, 8, 32, 2, 2, 2, 1, 30, "igemm16p_k333s1_m128_n8x32"),
    LIBCONV_TILE(261, 1, 3, 3, 3, 1, 1, 0, 128, 4, 32, 2, 2, 2, 1, 23, "igemm16p_k333s1_m128_n4x32"),
    LIBCONV_TILE(262, 1, 3, 3, 3, 1, 1, 0, 64, 8, 32, 1, 4, 2, 1, 33, "igemm16p_k333s1_m64_n8x32"),
    LIBCONV_TILE(263, 1, 3, 3, 3, 1, 1, 0, 64, 4, 32, 1, 4, 2, 1, 30, "igemm16p_k333s1_m64_n4x32"),
    LIBCONV_TILE(264, 1, 3, 3, 3, 1, 1, 0, 128, 8, 32, 2, 2, 1, 1, 24, "igemm16p_k333s1_m128_n8x32_c8"),
    // packed weights: 16-bit, 3x3 stride 1
    LIBCONV_TILE(270, 1, 1, 3, 3, 1, 1, 0, 128, 8, 32, 2, 2, 2, 1, 30, "igemm16p_k3s1_m128_n8x32"),
    LIBCONV_TILE(271, 1, 1, 3, 3, 1, 1, 0, 64, 8, 32, 1, 4, 2, 1, 36, "igemm16p_k3s1_m64_n8x32"),
    LIBCONV_TILE(272, 1, 1, 3, 3, 1, 1, 0, 128, 4, 32, 2, 2, 2, 1, 23, "igemm16p_k3s1_m128_n4x32"),
};

#undef LIBCONV_TILE

const TileDesc* find_tile(int id) {
  for (const auto& t : kTiles)
    if (t.id == id) return &t;
  return nullptr;
}

bool is_flat(const Problem& p) {
  return p.KT == 1 && p.KH == 1 && p.KW == 1 && p.st == 1 && p.sh == 1 && p.sw == 1 &&
         p.pt == 0 && p.ph == 0 && p.pw == 0;
}

bool tile_fits(const TileDesc& t, const Problem& p) {
  const int wide = p.dtype == LIBCONV_F32 ? 0 : 1;
  if (t.wide != wide) return false;
  const int se = wide ? 8 : 4;
  // 16-byte weight vectors read from OIHW must not straddle channels; packed
  // weights are zero-padded to whole groups instead.
  if (!t.packed && p.C % se != 0) return false;
  if (t.flat) return is_flat(p);
  return p.KT == t.KT && p.KH == t.KH && p.KW == t.KW && p.sh == t.SH && p.sw == t.SW &&
         (t.KT > 1 || (p.st == 1 && p.pt == 0));
}

struct TileCounts {
  long long co, rows, cols, total;
};

TileCounts counts(const TileDesc& t, const Problem& p) {
  TileCounts c;
  c.co = (p.K + t.BM - 1) / t.BM;
  if (t.flat) {
    c.rows = 1;
    c.cols = ((long long)p.OH * p.OW + t.TW - 1) / t.TW;
  } else {
    c.rows = (p.OH + t.TH - 1) / t.TH;
    c.cols = (p.OW + t.TW - 1) / t.TW;
  }
  c.total = c.co * p.N * p.OT * c.rows * c.cols;
  return c;
}

using PackFn = hipError_t (*)(const PackArgs&, unsigned, hipStream_t);

template <int DT, int TS>
hipError_t launch_pack(const PackArgs& a, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((pack_kernel<DT, TS>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

PackFn pack_fn(int dtype, int ts) {
  switch (dtype * 100 + ts) {
    case LIBCONV_F32 * 100 + 1: return &launch_pack<DT_F32, 1>;
    case LIBCONV_F32 * 100 + 9: return &launch_pack<DT_F32, 9>;
    case LIBCONV_F32 * 100 + 27: return &launch_pack<DT_F32, 27>;
    case LIBCONV_F16 * 100 + 1: return &launch_pack<DT_F16, 1>;
    case LIBCONV_F16 * 100 + 9: return &launch_pack<DT_F16, 9>;
    case LIBCONV_F16 * 100 + 27: return &launch_pack<DT_F16, 27>;
    case LIBCONV_BF16 * 100 + 1: return &launch_pack<DT_BF16, 1>;
    case LIBCONV_BF16 * 100 + 9: return &launch_pack<DT_BF16, 9>;
    case LIBCONV_BF16 * 100 + 27: return &launch_pack<DT_BF16, 27>;
    default: return nullptr;
  }
}

}  // namespace

const char* igemm_tile_name(int id) {
  const TileDesc* t = find_tile(id);
  return t ? t->name : nullptr;
}

bool igemm_tile_packed(int id) {
  const TileDesc* t = find_tile(id);
  return t && t->packed;
}

long long packed_weight_bytes(int C, int K, int KT, int KH, int KW, int dtype) {
  const long long se = dtype == LIBCONV_F32 ? 4 : 8;
  const long long groups = (C + se - 1) / se;
  const long long kp = (K + kPackAlign - 1) / kPackAlign * kPackAlign;
  return groups * KT * KH * KW * kp * 16;
}

bool pack_supported(int KT, int KH, int KW, int dtype) {
  return pack_fn(dtype, KT * KH * KW) != nullptr;
}

libconv_status pack_launch(const void* w, void* wp, int C, int K, int KT, int KH, int KW,
                           int dtype, hipStream_t stream) {
  const int ts = KT * KH * KW;
  const PackFn fn = pack_fn(dtype, ts);
  if (!fn) return LIBCONV_ERR_UNSUPPORTED;
  PackArgs a;
  a.w = w;
  a.wp = wp;
  a.K = K;
  a.C = C;
  const int se = dtype == LIBCONV_F32 ? 4 : 8;
  a.G = (C + se - 1) / se;
  a.Kp = (K + kPackAlign - 1) / kPackAlign * kPackAlign;
  a.w_bytes = (uint32_t)((long long)K * C * ts * dtype_bytes(dtype));
  a.wp_bytes = (uint32_t)packed_weight_bytes(C, K, KT, KH, KW, dtype);
  const long long units = (long long)a.G * a.Kp;
  const hipError_t e = fn(a, (unsigned)((units + kThreads - 1) / kThreads), stream);
  return e == hipSuccess ? LIBCONV_OK : LIBCONV_ERR_LAUNCH;
}

// Estimated time of a tile on this shape, in microseconds: rounds of
// workgroups on 256 compute units times the (padded) MFMA work of one tile at
// the tile's measured efficiency, plus -- for packed tiles when the caller
// gave OIHW weights -- the pack kernel (a launch plus reading and writing the
// weights once).
static double estimate_us(const TileDesc& t, const Problem& p, const TileCounts& c) {
  const double ck = t.CG * (t.wide ? 8 : 4);
  const double chunks = std::ceil(p.C / ck);
  const double kred = chunks * ck * p.KT * p.KH * p.KW;
  const double tile_flop = 2.0 * t.BM * t.TH * t.TW * kred;
  const double cu_flop_per_us = (t.wide ? 4096.0 : 256.0) * 2400.0 * (t.eff / 100.0);
  const double rounds = std::ceil(c.total / 256.0);
  double us = rounds * tile_flop / cu_flop_per_us;
  if (t.packed && !p.wp) {
    const double wbytes = (double)packed_weight_bytes(p.C, p.K, p.KT, p.KH, p.KW, p.dtype);
    us += 6.0 + 2.0 * wbytes / 3.0e6;
  }
  return us;
}

// Among the tiles that fit (packed or not, as asked), the one with the
// smallest estimated time.
static bool plan_among(const Problem& p, int want_packed, Plan* plan) {
  const TileDesc* best = nullptr;
  double best_cost = 0.0;
  long long best_total = 0;
  for (const auto& t : kTiles) {
    if (want_packed >= 0 && t.packed != want_packed) continue;
    if (!tile_fits(t, p) || !t.fn[p.dtype]) continue;
    const TileCounts c = counts(t, p);
    const double cost = estimate_us(t, p, c);
    if (!best || cost < best_cost) {
      best = &t;
      best_cost = cost;
      best_total = c.total;
    }
  }
  if (!best) return false;
  plan->algo = LIBCONV_ALGO_IGEMM;
  plan->tile = best->id;
  plan->grid = best_total;
  return true;
}

bool igemm_plan(const Problem& p, Plan* plan) { return plan_among(p, -1, plan); }

bool igemm_plan_packed(const Problem& p, Plan* plan) { return plan_among(p, 1, plan); }

bool igemm_plan_tile(const Problem& p, int tile_id, Plan* plan) {
  const TileDesc* t = find_tile(tile_id);
  if (!t || !tile_fits(*t, p) || !t->fn[p.dtype]) return false;
  plan->algo = LIBCONV_ALGO_IGEMM;
  plan->tile = t->id;
  plan->grid = counts(*t, p).total;
  return true;
}

libconv_status igemm_launch(const Problem& p, const Plan& plan) {
  const TileDesc* t = find_tile(plan.tile);
  if (!t || !tile_fits(*t, p)) return LIBCONV_ERR_UNSUPPORTED;
  const LaunchFn fn = t->fn[p.dtype];
  if (!fn) return LIBCONV_ERR_UNSUPPORTED;
  if (t->packed && !p.wp) return LIBCONV_ERR_UNSUPPORTED;
  const TileCounts c = counts(*t, p);
  if (c.total > 0x7fffffffLL) return LIBCONV_ERR_UNSUPPORTED;
  IgemmArgs a;
  a.x = p.x; a.w = t->packed ? p.wp : p.w; a.b = p.b; a.y = p.y;
  a.N = p.N; a.C = p.C; a.T = p.T; a.K = p.K; a.OT = p.OT;
  if (t->flat) {  // a 1x1 layer: each plane is one row of H*W pixels
    a.H = 1; a.W = p.H * p.W; a.OH = 1; a.OW = p.OH * p.OW;
  } else {
    a.H = p.H; a.W = p.W; a.OH = p.OH; a.OW = p.OW;
  }
  a.pt = p.pt; a.ph = p.ph; a.pw = p.pw; a.st = p.st;
  a.relu = p.act == LIBCONV_ACT_RELU;
  const int ck = t->CG * (t->wide ? 8 : 4);
  a.chunks = (p.C + ck - 1) / ck;
  a.kp = (p.K + kPackAlign - 1) / kPackAlign * kPackAlign;
  a.co_tiles = (int)c.co; a.row_tiles = (int)c.rows; a.col_tiles = (int)c.cols;
  const int eb = dtype_bytes(p.dtype);
  a.x_bytes = (uint32_t)((long long)p.N * p.C * p.T * p.H * p.W * eb);
  a.w_bytes = t->packed ? (uint32_t)packed_weight_bytes(p.C, p.K, p.KT, p.KH, p.KW, p.dtype)
                        : (uint32_t)((long long)p.K * p.C * p.KT * p.KH * p.KW * eb);
  a.b_bytes = p.b ? (uint32_t)(p.K * eb) : 0u;
  a.y_bytes = (uint32_t)((long long)p.N * p.K * p.OT * p.OH * p.OW * eb);
  const hipError_t e = fn(a, (unsigned)c.total, p.stream);
  return e == hipSuccess ? LIBCONV_OK : LIBCONV_ERR_LAUNCH;
}

}  // namespace libconv
