// igemm_kernel.h -- the implicit-GEMM convolution kernel on the gfx950 matrix
// cores (MFMA), as a template over its tile configuration.  Instantiated in
// the igemm_inst_*.hip units (one per group of tiles, so that they compile in
// parallel); planned and launched by igemm.hip.
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
//       - from packed weights ([C_out padded / 64][C/SE][taps][64][SE], made
//         by the pack kernel below -- the per-layer weight packing of the
//         Convolution3D work in "SeedVR2 NCNN Vulkan", section 3.2): a stage
//         is NSLOT 1 KB runs copied straight into LDS by direct-to-LDS loads
//         (no registers, no arithmetic), and all the weights one 64-channel
//         block of a tile reads are one contiguous range of memory;
//   * the input halo (HR rows x HC cols of one frame) is read
//     row-contiguously -- as aligned 16-byte runs of one channel where the
//     row length allows, else element by element -- and written
//     channel-innermost as Xl[g][hr][col][SE]; taps outside the input are
//     zero (this is the padding);
//   * the stage's slots are consumed in pairs by one MFMA k-step (32x32x16
//     f16/bf16: lanes 0-31 carry slot 2p, lanes 32-63 slot 2p+1) or by four
//     (32x32x2 f32, one element of each slot per step).  Both operands of a
//     slot are single 16-byte LDS reads.
// While stage s is multiplied, the reads of stage s+2 into registers and the
// direct-to-LDS copy of stage s+1's packed weights (which come from L2) are
// in flight; LDS holds two stages.  Each lane's load offsets are computed
// once; the per-stage part of every address is wave-uniform and moves the
// base of the buffer descriptor (scalar arithmetic), so staging costs almost
// no vector arithmetic and every access stays range-checked.
//
// Epilogue (shared with the direct kernel): fp32 accumulator + bias ->
// optional ReLU -> one round-to-nearest-even conversion -> store, with the
// 32 lanes of a half-wave writing 32 consecutive output pixels of one
// channel.  Every output element has exactly one writer.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace libconv {
namespace igk {

constexpr int kThreads = 256;
constexpr int kPackAlign = 128;   // output channels of packed weights are padded to this
// Offset past the end of every tensor (all are below 0x7fff0000 bytes), with
// room to add the offsets of a unit's 16-byte vectors without overflow.
constexpr int kFar = 0x7ffff000;

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
  int wblk;           // packed weights: entries per 64-output-channel block
  int co_tiles, row_tiles, col_tiles;
  int co_group;       // output-channel tiles per group of the launch order
  // split-K: `ksplit` workgroups share a tile, each summing a contiguous range
  // of `cps` channel chunks and writing its fp32 partial sums (no bias, no
  // activation) to part[split][n][co][ot][oh][ow]; 1 = no split
  int ksplit, cps;
  float* part;
  int vec_out;        // 1: output rows are whole 16-byte vectors and y is 16-byte aligned
  // 1: y is the 2x2 stride-2 max pool of act(conv + bias), [N][K][OH/2][OW/2]
  // (floor), computed in the epilogue; vec_out then refers to the pooled rows
  int pool;
  // 1: the output frame is the fastest-varying part of the pixel tile index
  int frame_fast;
  uint32_t x_bytes, w_bytes, b_bytes, y_bytes, part_bytes;
};

// Slot pairs of a stage over which a one-weight-set tile (Cfg::W1) reads the
// next stage's weights: the rest of the stage, up to SPAIR, covers their
// latency.
constexpr int kW1Pairs = 2;

template <int DT_, int KT_, int KH_, int KW_, int SH_, int SW_, int BM_, int TH_, int TW_,
          int WM_, int WN_, int CG_, int PK_, int VX_>
struct Cfg {
  static constexpr int DT = DT_, KT = KT_, KH = KH_, KW = KW_, SH = SH_, SW = SW_;
  static constexpr int BM = BM_, TH = TH_, TW = TW_, WM = WM_, WN = WN_, CG = CG_;
  // waves of a workgroup (a WM x WN grid) and its threads
  static constexpr int NWV = WM * WN;
  static constexpr int NT = 64 * NWV;
  // PK_ bit 0: packed weights; bit 1: single-stage tile (all input channels
  // of the layer in one stage; one LDS buffer, no overlap machinery)
  static constexpr bool PK = (PK_ & 1) != 0;
  static constexpr bool ONE = (PK_ & 2) != 0;
  // PK_ bit 2 (OIHW / OIDHW weights): the weights go through one register
  // set, read at the start of a stage for the next one and transposed into
  // LDS before slot pair SPAIR (the input keeps two sets, two stages ahead),
  // which frees a set of weight registers for a second workgroup per CU
  static constexpr bool W1 = (PK_ & 4) != 0;
  static constexpr bool VX = VX_ == 1;
  // VX_ == 2: channel-packed activations, x [N][C/SE][T][H][W][SE] and y
  // likewise over C_out.  A halo row of one channel group is then a run of
  // 16-byte words in memory, copied straight into LDS (no registers, no
  // repacking), and the accumulators leave as 16-byte channel groups.
  static constexpr bool XP = VX_ == 2;
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
  // Input staging.  VX tiles read the halo as aligned runs of RUN pixels of
  // one channel (one 16-byte read per channel and run); the halo rows are
  // widened to whole runs, starting up to MAXSHIFT columns left of the first
  // tap column.  Other tiles read one element per channel and pixel.
  static constexpr int RUN = 16 / EB;
  static constexpr int MAXSHIFT = (VX && KW > 1) ? RUN - 1 : 0;
  static constexpr int XCOLS = VX ? (HC + MAXSHIFT + RUN - 1) / RUN * RUN : HC;
  static constexpr int NRUN = XCOLS / RUN;
  // LDS row pitch in 16-byte words.  A VX unit writes RUN consecutive words
  // of one row; eight lanes side by side hold eight consecutive rows, and an
  // odd pitch puts their words in eight different bank groups.
  static constexpr int PITCH = VX ? XCOLS + 1 : XCOLS;
  static constexpr int NROWS = CG * HR;            // halo rows of a stage (all groups)
  static constexpr int XPLANE = HR * PITCH;        // LDS words per channel group
  static constexpr int WBYTES = NSLOT * BM * 16;
  // channel-packed input: CG x HR x HC words per stage, 64 per wave-wide
  // direct-to-LDS copy (the buffer is rounded up to whole copies)
  static constexpr int XDMA = XP ? (CG * HR * HC + 63) / 64 : 0;
  static constexpr int NXDMA = (XDMA + NWV - 1) / NWV;  // copies per wave
  static constexpr int XBYTES = XP ? XDMA * 1024 : CG * XPLANE * 16;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FA = WTM / 32, FB = WTN / 32;
  static constexpr int BPR = TW / 32;              // 32-pixel blocks per tile row
  // one set of B fragments (the next pair's B reads wait for this pair's
  // MFMAs, the other wave of the SIMD covers them): eight-wave tiles of four
  // 32-pixel blocks per wave that stage through registers, whose fragments
  // do not fit twice beside the accumulators and the staged stages
  static constexpr bool SB = NWV == 8 && FB >= 4 && !(XP && PK);
  // weight staging from OIHW: one unit = one output channel x one group of
  // SE input channels = TS contiguous 16-byte vectors; unit u = g * BM + channel.
  // From OIDHW (W3: 3-D tiles that read unpacked weights) a stage is one
  // frame tap, so a unit is SE runs of the TS2 spatial taps, one per input
  // channel, TS elements apart: each run is read as one (unaligned) 16-byte
  // load of its first 8 taps and one 2-byte load of the ninth.
  static constexpr bool W3 = !PK && KT > 1;
  static constexpr int WUNITS = PK ? 0 : BM * CG;
  static constexpr int WPASS = PK ? 0 : (WUNITS + NT - 1) / NT;
  static constexpr int NWREG = PK ? 0 : W3 ? WPASS * SE * 2 : WPASS * TS;
  // weight staging from packed weights: NSLOT runs of BM 16-byte vectors,
  // moved as 1 KB chunks (one wave, one instruction each), NDMA per weight
  // wave (below); when the chunks do not divide evenly, the spare copies read
  // nothing (zeros) into a 1 KB scratch area at the end of LDS
  static constexpr int WCHUNKS = NSLOT * BM / 64;
  // input staging: one unit = one run (VX) or one halo pixel of one channel
  // group.  VX units come in blocks of 8 rows x NRUN runs (8 lanes side by
  // side on 8 rows), or, when the halo's rows are not a multiple of 8 and
  // that saves a wave-wide read per channel, densely as NRUN runs of all the
  // rows (lanes side by side on consecutive rows, then the next run).  Every
  // wave-wide read costs the address unit alike, however many of its lanes
  // fall outside the halo.
  static constexpr int XUNITS_BLK = (NROWS + 7) / 8 * 8 * NRUN;
  static constexpr bool XDENSE = VX && (NROWS * NRUN + 63) / 64 < (XUNITS_BLK + 63) / 64;
  static constexpr int XUNITS = VX ? (XDENSE ? NROWS * NRUN : XUNITS_BLK) : CG * HR * HC;
  static constexpr int XPASS = XP ? 0 : (XUNITS + NT - 1) / NT;
  static constexpr int XPASS1 = XPASS > 0 ? XPASS : 1;  // array extent
  // Which waves stage what.  When a stage's input units fit in fewer waves
  // than the workgroup has, only those (the first XW) read the input, so that
  // no wave issues reads that would all fall outside the tensor (such reads
  // still cost the address unit a full wave instruction).  Packed weights are
  // copied by all the waves: a wave that copied them alone (as many
  // one-instruction copies as the input waves' reads, repacking and LDS
  // writes together) finished each stage last and held the others at the
  // barrier (measured per wave on the 3x3x3 video-VAE layers), and leaving
  // them to the waves without input units measured no faster.  OIHW weight
  // units go to the last WW waves.  A wave may have both roles.
  static constexpr int XW = (VX && XPASS == 1) ? (XUNITS + 63) / 64 : NWV;
  static constexpr int WW = PK ? NWV : (WPASS == 1 ? (WUNITS + 63) / 64 : NWV);
  static constexpr int W0 = NWV - WW;              // first weight wave
  static constexpr int NDMA = PK ? (WCHUNKS + WW - 1) / WW : 0;
  static constexpr int DMA_PAD =
      ((PK && WCHUNKS % WW != 0) || (XP && XDMA % NWV != 0)) ? 1024 : 0;
  // LDS: two weight and two input buffers (one of each for single-stage tiles)
  static constexpr int NBUF = ONE ? 1 : 2;
  // the vectorised epilogue reuses LDS as wave-private 32x32 tiles
  static constexpr int EPI_LDS = NWV * 32 * (32 + 16 / EB) * EB;
  // 2x2 max pooling in the epilogue: a wave's consecutive blocks are
  // consecutive output rows (one 32-pixel block per tile row) in even-odd
  // pairs; two fp32 32x36 LDS tiles per wave
  static constexpr bool POOLABLE = NWV == 4 && BPR == 1 && FB % 2 == 0 && TH % 2 == 0 && KT == 1;
  static constexpr int EPI_POOL_LDS = POOLABLE ? NWV * 2 * 32 * 36 * 4 : 0;
  static constexpr int STAGES_LDS = NBUF * (WBYTES + XBYTES) + DMA_PAD;
  static constexpr int LDS0 = STAGES_LDS > EPI_LDS ? STAGES_LDS : EPI_LDS;
  static constexpr int LDS = LDS0 > EPI_POOL_LDS ? LDS0 : EPI_POOL_LDS;
  // global reads into registers each wave issues per stage
  static constexpr int REG_LOADS = XPASS * SE + NWREG;
  // slot pair before whose MFMAs the next stage's registers are written to
  // LDS (the free buffer), so that two pairs of MFMAs still cover the write
  // latency before the end-of-stage barrier; -1: after the last pair
  static constexpr int SPAIR = NPAIR >= 3 ? NPAIR - 2 : -1;

  static_assert(NWV == 4 || (NWV == 8 && !ONE), "four waves, or eight");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  static_assert(TW % 32 == 0, "tile rows are whole 32-pixel blocks");
  static_assert(BM % 64 == 0 || !PK, "packed tiles move whole 64-channel chunks");
  static_assert(BM <= kPackAlign, "packed channel padding covers one tile");
  static_assert(!W3 || (TS2 == 9 && EB == 2), "OIDHW weights: 3x3 spatial taps, 16-bit types");
  static_assert(!XP || !ONE, "channel-packed tiles run two stages");
  static_assert(!W1 || (!PK && !XP && !ONE && NPAIR >= 5), "one weight set: OIHW tiles of 5+ pairs");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// Global -> registers for one stage (weights only when they are transposed
// here; packed weights go straight to LDS).  Input elements are kept exactly
// as loaded and only packed into 16-byte words when they are written to LDS,
// after the current stage's MFMAs: any arithmetic on them right after the
// loads would make the wave wait for the loads before computing.
template <class G>
struct StageRegs {
  using XE = typename Elem<G::DT>::raw_t;
  // OIHW units (TS vectors); OIDHW units: wv[i][j] = taps 0-7 of channel j's
  // run, wt[i][j] = its ninth tap
  u32x4_t wv[G::WPASS > 0 ? G::WPASS : 1][G::W3 ? G::SE : G::TS];
  uint32_t wt[G::W3 ? G::WPASS : 1][G::W3 ? G::SE : 1];
  XE xe[G::VX ? 1 : G::XPASS1][G::VX ? 1 : G::SE];       // one element per read
  u32x4_t xr[G::VX ? G::XPASS1 : 1][G::VX ? G::SE : 1];  // one run per read
};

// Make a register's value opaque to the optimiser at this point.  Applied to
// staged values right before they are repacked, it keeps the repacking (and
// the wait for the loads) from being moved up next to the loads.
template <class T>
__device__ __forceinline__ void pin(T& v) {
  asm volatile("" : "+v"(v));
}

// f(std::integral_constant<int, i>) for i = B .. E-1, unrolled at compile time.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Wait until at most N of this wave's global reads are outstanding (gfx9
// s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left
// at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS hand-over: this wave's LDS writes complete, then
// s_barrier.  Unlike __syncthreads() it does not wait for outstanding global
// reads (those of later stages stay in flight); the "memory" clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One 16-byte global read per lane written straight into LDS: lane l's
// vector lands at dst + 16 l (dst is wave-uniform).  Kept out of the generic
// lambdas of the kernel: inside them the host pass drops the kernel's launch
// stub.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, unsigned char* dst,
                                              int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           off, 0, 0, 0);
}

// This wave's LDS accesses so far are complete and none of the later ones
// is moved above this point (a wave-private LDS region changes hands between
// lanes of the same wave).
__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

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

// Four-wave one-weight-set tiles are built for two workgroups per CU (the
// second launch bound holds the register allocation to half the file; an
// eight-wave workgroup already holds two waves per SIMD).
template <class G>
__global__ __launch_bounds__(G::NT, (G::W1 && G::NWV == 4) ? 2 : 1) void igemm_kernel(IgemmArgs a) {
  using E = Elem<G::DT>;
  constexpr int EB = G::EB;
  constexpr int SE = G::SE;
  __shared__ __attribute__((aligned(16))) unsigned char lds[G::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int il = lane & 31;   // row (A) / column (B) inside a 32x32 block
  const int hf = lane >> 5;   // which slot of the pair this lane carries
  const bool xwave = wave < G::XW;     // stages input (wave-uniform)
  const bool wwave = wave >= G::W0;    // stages weights (wave-uniform)

  // ---- tile coordinates; XCD-aware order: the hardware deals workgroups to
  // the 8 XCDs round-robin, so consecutive logical tiles are gathered onto one
  // XCD and its L2.  Logical order: groups of co_group output-channel tiles
  // (whose weights fit in L2 together); inside a group the output-channel
  // tile varies fastest, so the tiles that read the same input pixels run
  // side by side, then the pixel tile.
  // With split-K the split index is the slowest part of the logical order,
  // so an XCD mostly works on one split's channels.
  const int G_ = gridDim.x;
  int bid = blockIdx.x;
  if ((G_ & 7) == 0) bid = (bid & 7) * (G_ >> 3) + (bid >> 3);
  const int pix_tiles = a.col_tiles * a.row_tiles * a.OT * a.N;
  const int tiles = a.co_tiles * pix_tiles;
  const int split = bid / tiles;
  bid -= split * tiles;
  const int full_groups = a.co_tiles / a.co_group;
  int cot;
  if (bid < full_groups * a.co_group * pix_tiles) {
    const int gt = a.co_group * pix_tiles;
    const int grp = bid / gt, rem = bid % gt;
    cot = grp * a.co_group + rem % a.co_group;
    bid = rem / a.co_group;
  } else {
    const int rem = bid - full_groups * a.co_group * pix_tiles;
    const int last = a.co_tiles - full_groups * a.co_group;
    cot = full_groups * a.co_group + rem % last;
    bid = rem / last;
  }
  // A frame kernel (KT > 1) reads each input frame for KT output frames:
  // with the output frame varying fastest (frame_fast) those tiles run
  // together and the frame is fetched into L2 once instead of once per
  // output frame.
  int ctile, rtile, ot;
  if (G::KT > 1 && a.frame_fast) {
    ot = bid % a.OT;
    bid /= a.OT;
    ctile = bid % a.col_tiles;
    bid /= a.col_tiles;
    rtile = bid % a.row_tiles;
    bid /= a.row_tiles;
  } else {
    ctile = bid % a.col_tiles;
    bid /= a.col_tiles;
    rtile = bid % a.row_tiles;
    bid /= a.row_tiles;
    ot = bid % a.OT;
    bid /= a.OT;
  }
  const int n = bid;
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
  const int chunk0 = split * a.cps;  // this workgroup's channel chunks
  const int nstages = max(0, min(a.chunks - chunk0, a.cps)) * nkt;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);

  const int hw = a.H * a.W;
  const int plane = a.T * hw;            // elements between input channels in x

  // ---- per-lane, stage-invariant load offsets (bytes).  The per-stage part
  // of every address is wave-uniform: it moves the base of the buffer
  // descriptor (scalar arithmetic), while the range check keeps covering
  // every access up to the end of the tensor.
  // VX: halo unit u holds run (u / 8) % NRUN of row 8 * (u / (8 * NRUN)) +
  // u % 8 (dense: run u / NROWS of row u % NROWS), row = g * HR + hr; one
  // offset per unit (the channel j of its group
  // is added as the scalar offset j * plane).  The runs start at a multiple
  // of RUN columns, `shift` columns left of the first tap column; with W a
  // multiple of RUN a run lies wholly inside or wholly outside the row.
  // Otherwise: unit u = (g * HR + hr) * HC + hc, one offset per channel.
  const int shift = G::VX ? (iw0 & (G::RUN - 1)) : 0;
  int xoff[G::VX ? 1 : G::XPASS1][G::VX ? 1 : SE];  // kFar when the position is padding
  int xv[G::VX ? G::XPASS1 : 1];
  int xgrp[G::XPASS1];
#pragma unroll
  for (int i = 0; i < G::XPASS; ++i) {
    const int u = tid + i * G::NT;
    if constexpr (G::VX) {
      const int run = G::XDENSE ? u / G::NROWS : (u >> 3) % G::NRUN;
      const int row = G::XDENSE ? u % G::NROWS : (u >> 3) / G::NRUN * 8 + (u & 7);
      const int hr = row % G::HR;
      const int g = row / G::HR;
      const int ih = ih0 + hr, iw = iw0 - shift + run * G::RUN;
      const bool ok = u < G::XUNITS && row < G::NROWS && (unsigned)ih < (unsigned)a.H &&
                      (unsigned)iw < (unsigned)a.W;
      xv[i] = guard_offset(true, ok ? (g * SE * plane + ih * a.W + iw) * EB : kFar);
      xgrp[i] = g;
    } else {
      const int hc = u % G::HC;
      const int hr = (u / G::HC) % G::HR;
      const int g = u / (G::HC * G::HR);
      const int ih = ih0 + hr, iw = iw0 + hc;
      const bool ok =
          u < G::XUNITS && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
#pragma unroll
      for (int j = 0; j < SE; ++j)
        xoff[i][j] = guard_offset(true, ok ? ((g * SE + j) * plane + ih * a.W + iw) * EB : kFar);
      xgrp[i] = g;
    }
  }
  const int ch_bytes = plane * EB;       // scalar offset between channels
  // Channel-packed input: copy k of this wave is words (wave + NWV k) * 64 +
  // lane of the stage's halo, word f = (g * HR + hr) * HC + hc, i.e. the
  // 16-byte channel group g of halo pixel (hr, hc); one offset per copy,
  // relative to the stage's first channel group at the stage's frame.
  const int cgs = (a.C + SE - 1) / SE;    // channel groups of x
  int xdo[G::XP ? G::NXDMA : 1];
  int xdg[G::XP ? G::NXDMA : 1];
  if constexpr (G::XP) {
#pragma unroll
    for (int k = 0; k < G::NXDMA; ++k) {
      const int f = (wave + G::NWV * k) * 64 + lane;
      const int g = f / (G::HR * G::HC);
      const int hr = (f / G::HC) % G::HR, hc = f % G::HC;
      const int ih = ih0 + hr, iw = iw0 + hc;
      const bool ok = f < G::XUNITS && (unsigned)ih < (unsigned)a.H && (unsigned)iw < (unsigned)a.W;
      xdo[k] = guard_offset(true, ok ? (g * a.T * hw + ih * a.W + iw) * 16 : kFar);
      xdg[k] = g;
    }
  }
  // OIHW weight unit u = g * BM + col
  int woff[G::WPASS > 0 ? G::WPASS : 1];
  int wgrp[G::WPASS > 0 ? G::WPASS : 1];
#pragma unroll
  for (int i = 0; i < G::WPASS; ++i) {
    const int u = tid - 64 * G::W0 + i * G::NT;  // weight units start at the first weight wave
    const int g = u / G::BM, col = u % G::BM;
    const int co = co0 + col;
    const bool ok = u >= 0 && u < G::WUNITS && co < a.K;
    woff[i] = guard_offset(true, ok ? (co * a.C * G::TS + g * SE * G::TS) * EB : kFar);
    wgrp[i] = g;
  }
  const int n_base = n * a.C * plane * EB;

  // The global reads of a stage, as pieces of one instruction each that are
  // spread over the MFMA work of an earlier stage: pieces [0, NWP) read the
  // weights (packed ones straight into the LDS weight buffer `wdst`, OIHW ones
  // into registers), pieces [NWP, NWP + NXP) the input into registers.  When
  // C is a multiple of the stage's channel count (`ragged` false) every
  // channel exists and the reads are unguarded; otherwise every read is
  // guarded per channel.
  constexpr int NWP = G::PK ? G::NDMA : G::NWREG;
  constexpr int NXP = G::XPASS * SE;
  struct Src {  // wave-uniform addressing of one stage
    __amdgpu_buffer_rsrc_t rs;  // input or OIHW weights, based at the stage's first channel
    int ci0;
    int wrun;                   // packed weights: first 16-byte entry of the stage's slots
  };
  auto w_src = [&](int chunk, int kt) -> Src {
    Src q;
    q.ci0 = chunk * G::CK;
    if constexpr (G::PK) {
      q.rs = wr;
      q.wrun = (chunk * G::CG * G::TS + kt * G::TS2) * 64 + (co0 >> 6) * a.wblk;
    } else {  // OIHW / OIDHW: the stage's first channel at the stage's frame tap
      const int sb = (q.ci0 * G::TS + kt * G::TS2) * EB;
      q.rs = make_rsrc((const char*)a.w + sb, a.w_bytes - sb);
      q.wrun = 0;
    }
    return q;
  };
  auto x_src = [&](int chunk, int kt) -> Src {
    Src q;
    q.ci0 = chunk * G::CK;
    const int sb = G::XP ? (((n * cgs + chunk * G::CG) * a.T + it0 + kt) * hw) * 16
                         : n_base + (q.ci0 * plane + (it0 + kt) * hw) * EB;
    q.rs = make_rsrc((const char*)a.x + sb, a.x_bytes - sb);
    q.wrun = 0;
    return q;
  };
  // `role` (compile time): bit 0 the wave stages input, bit 1 weights; a
  // read of the other kind is not issued at all.
  auto read_w = [&](auto role, auto ragged, auto kc, const Src& q, StageRegs<G>& r,
                    unsigned char* wdst) __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    if constexpr ((decltype(role)::value & 2) == 0) {
      return;
    } else if constexpr (G::PK) {
      // chunk c = 64 channels of one slot; lane l lands at chunk base + 16 l
      const int c = (wave - G::W0) + k * G::WW;
      const int slot = c / (G::BM / 64), part = c % (G::BM / 64);
      const int t2 = slot / G::CG, g = slot % G::CG;
      const int run = q.wrun + (g * G::TS + t2) * 64 + part * a.wblk;
      const bool real = c < G::WCHUNKS;  // wave-uniform
      unsigned char* dst = real ? wdst + (slot * G::BM + part * 64) * 16 : lds + G::LDS - 1024;
      copy16_to_lds(q.rs, dst, guard_offset(true, real ? (run + lane) * 16 : kFar));
    } else if constexpr (G::W3) {
      // piece k: channel j of unit i, first 8 taps (even k) or the ninth
      constexpr int i = k / (2 * SE), j = (k / 2) % SE, part = k % 2;
      int v = woff[i];
      if constexpr (decltype(ragged)::value)
        v = guard_offset(true, q.ci0 + wgrp[i] * SE < a.C ? v : kFar);
      const int off = j * G::TS * EB + part * 8 * EB;
      if constexpr (part == 0)
        r.wv[i][j] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(q.rs, v + off, 0, 0));
      else
        r.wt[i][j] = E::load_raw(q.rs, v + off);
    } else {
      constexpr int i = k / G::TS, t = k % G::TS;
      int v = woff[i];
      if constexpr (decltype(ragged)::value)
        v = guard_offset(true, q.ci0 + wgrp[i] * SE < a.C ? v : kFar);
      r.wv[i][t] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(q.rs, v + t * 16, 0, 0));
    }
  };
  auto read_x = [&](auto role, auto ragged, auto kc, const Src& q, StageRegs<G>& r)
      __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    constexpr int i = k / SE, j = k % SE;
    constexpr bool rg = decltype(ragged)::value;
    if constexpr ((decltype(role)::value & 1) == 0) {
      return;
    } else if constexpr (G::VX) {
      int v = xv[i];
      if constexpr (rg) v = guard_offset(true, q.ci0 + xgrp[i] * SE + j < a.C ? v : kFar);
      r.xr[i][j] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(q.rs, v, j * ch_bytes, 0));
    } else {
      int v = xoff[i][j];
      if constexpr (rg) v = guard_offset(q.ci0 + xgrp[i] * SE + j < a.C, v);
      r.xe[i][j] = E::load_raw(q.rs, v);
    }
  };

  // Channel-packed input: copy k of this wave straight into the halo buffer
  // `xdst` (copies past the halo land in the scratch area and read nothing);
  // in a ragged last chunk the groups past the input's read zero.
  auto read_xd = [&](auto ragged, auto kc, const Src& q, unsigned char* xdst)
      __attribute__((always_inline)) {
    constexpr int k = decltype(kc)::value;
    const int ins = wave + G::NWV * k;
    int off = xdo[k];
    if constexpr (decltype(ragged)::value)
      off = guard_offset(true, q.ci0 / SE + xdg[k] < cgs ? off : kFar);
    unsigned char* dst = ins < G::XDMA ? xdst + ins * 1024 : lds + G::LDS - 1024;
    copy16_to_lds(q.rs, dst, off);
  };

  // Registers of a stage -> LDS (weights into `wdst` unless they were copied
  // there directly, the input halo into `xdst`).
  // `part` (compile time): bit 0 the input, bit 1 the weights
  auto store_part = [&](auto partc, StageRegs<G>& r, unsigned char* wdst, unsigned char* xdst)
      __attribute__((always_inline)) {
    constexpr bool SW_ = (decltype(partc)::value & 2) != 0;  // weights
    constexpr bool SX_ = (decltype(partc)::value & 1) != 0;  // input
    constexpr int WP = SW_ ? G::WPASS : 0, XPS = SX_ ? G::XPASS : 0;
#pragma unroll
    for (int i = 0; i < WP; ++i) {
#pragma unroll
      for (int k = 0; k < (G::W3 ? SE : G::TS); ++k) pin(r.wv[i][k]);
      if constexpr (G::W3) {
#pragma unroll
        for (int k = 0; k < SE; ++k) pin(r.wt[i][k]);
      }
    }
#pragma unroll
    for (int i = 0; i < XPS; ++i)
#pragma unroll
      for (int j = 0; j < SE; ++j) {
        if constexpr (G::VX) {
          pin(r.xr[i][j]);
        } else {
          pin(r.xe[i][j]);
        }
      }
    // weights from OIHW: [ci][tap] per unit -> Wl[slot = tap * CG + g][co][SE];
    // lanes of a wave hold consecutive channels, so each 16-byte store is
    // conflict-free
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int u = tid - 64 * G::W0 + i * G::NT;
      unsigned char* base = wdst + ((u / G::BM) * G::BM + u % G::BM) * 16;
      if constexpr (G::W3) {
        // slot of spatial tap t: word m = channels 2m, 2m+1 at tap t
#pragma unroll
        for (int t = 0; t < G::TS2; ++t) {
          u32x4_t v;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            if (t < 8) {
              const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
              v[m] = __builtin_amdgcn_perm(r.wv[i][2 * m + 1][t >> 1], r.wv[i][2 * m][t >> 1],
                                           sel);
            } else {
              v[m] = (r.wt[i][2 * m] & 0xffffu) | (r.wt[i][2 * m + 1] << 16);
            }
          }
          if (u >= 0 && u < G::WUNITS)
            *reinterpret_cast<u32x4_t*>(base + t * G::CG * G::BM * 16) = v;
        }
      } else {
        if (u >= 0 && u < G::WUNITS)
          store_slots<SE, G::TS, 0>(base, G::CG * G::BM * 16, r.wv[i]);
      }
    }
    // input halo: gather the SE channels of each pixel into one 16-byte word
#pragma unroll
    for (int i = 0; i < XPS; ++i) {
      const int u = tid + i * G::NT;
      if constexpr (G::VX) {
        // unit u covers the RUN words of its run in its row
        const int run = G::XDENSE ? u / G::NROWS : (u >> 3) % G::NRUN;
        const int row = G::XDENSE ? u % G::NROWS : (u >> 3) / G::NRUN * 8 + (u & 7);
        unsigned char* dst = xdst + (row * G::PITCH + run * G::RUN) * 16;
#pragma unroll
        for (int q = 0; q < G::RUN; ++q) {
          u32x4_t v;
          if constexpr (SE == 8) {
            const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
#pragma unroll
            for (int m = 0; m < 4; ++m)
              v[m] = __builtin_amdgcn_perm(r.xr[i][2 * m + 1][q >> 1], r.xr[i][2 * m][q >> 1], sel);
          } else {
#pragma unroll
            for (int m = 0; m < 4; ++m) v[m] = r.xr[i][m][q];
          }
          if (u < G::XUNITS && row < G::NROWS) *reinterpret_cast<u32x4_t*>(dst + q * 16) = v;
        }
      } else {
        const auto* e = r.xe[i];
        u32x4_t v;
        if constexpr (SE == 8)
          v = u32x4_t{e[0] | ((uint32_t)e[1] << 16), e[2] | ((uint32_t)e[3] << 16),
                      e[4] | ((uint32_t)e[5] << 16), e[6] | ((uint32_t)e[7] << 16)};
        else
          v = u32x4_t{e[0], e[1], e[2], e[3]};
        if (u < G::XUNITS) *reinterpret_cast<u32x4_t*>(xdst + u * 16) = v;
      }
    }
  };

  auto store_stage = [&](StageRegs<G>& r, unsigned char* wdst, unsigned char* xdst)
      __attribute__((always_inline)) {
    store_part(std::integral_constant<int, 3>{}, r, wdst, xdst);
  };

  // ---- MFMA operand addressing
  const int wm = wave % G::WM;
  const int wn = wave / G::WM;
  const int co_w0 = wm * G::WTM;
  const int blk0 = wn * G::FB;                       // first 32-pixel block of this wave
  const int prow0 = blk0 / G::BPR, pcol0 = (blk0 % G::BPR) * 32;
  // A: Wl[slot][co][16 B]; lanes of half hf read slot 2p + hf.
  const int a_lane = ((hf * G::BM) + co_w0 + il) * 16;
  // B: Xl[g][hr][col][16 B] (rows PITCH words apart) at the lane's pixel
  // (col = hc + shift).
  const int b_lane = ((prow0 * G::SH) * G::PITCH + (pcol0 + il) * G::SW + shift) * 16;

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
    return ((g * G::HR + kh) * G::PITCH + kw) * 16;
  };
  // byte offset of block j of this wave relative to its first block
  auto xblock = [&](int j) -> int {
    const int b = blk0 + j;
    const int r = b / G::BPR, c = (b % G::BPR) * 32;
    return ((r - prow0) * G::SH * G::PITCH + (c - pcol0) * G::SW) * 16;
  };

  // The MFMA work of one stage; hook(p) runs before the MFMAs of slot pair p
  // (it issues pieces of later stages' reads).
  auto compute = [&](const unsigned char* wl, const unsigned char* xl, auto&& hook)
      __attribute__((always_inline)) {
    constexpr int NBB = G::SB ? 1 : 2;  // B fragment sets
    u32x4_t fa[2][G::FA], fb[NBB][G::FB];
    auto load_a = [&](auto pc, int k) {
      constexpr int p = decltype(pc)::value;
      const int s0 = 2 * p;
#pragma unroll
      for (int i = 0; i < G::FA; ++i)
        fa[k][i] = *reinterpret_cast<const u32x4_t*>(wl + a_lane + (s0 * G::BM + i * 32) * 16);
      if (2 * p + 1 >= G::NSLOT && hf) {
        // odd slot count: the second half of the last pair carries nothing
#pragma unroll
        for (int i = 0; i < G::FA; ++i) fa[k][i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    };
    auto load_b = [&](auto pc, int k) {
      constexpr int p = decltype(pc)::value;
      const int s0 = 2 * p;
      const int s1 = (2 * p + 1 < G::NSLOT) ? 2 * p + 1 : 2 * p;
      const int xo = hf ? xslot(s1) : xslot(s0);
#pragma unroll
      for (int j = 0; j < G::FB; ++j)
        fb[k][j] = *reinterpret_cast<const u32x4_t*>(xl + b_lane + xo + xblock(j));
      if (2 * p + 1 >= G::NSLOT && hf) {
#pragma unroll
        for (int j = 0; j < G::FB; ++j) fb[k][j] = u32x4_t{0u, 0u, 0u, 0u};
      }
    };
    load_a(std::integral_constant<int, 0>{}, 0);
    load_b(std::integral_constant<int, 0>{}, 0);
    static_for<0, G::NPAIR>([&](auto pc) {
      constexpr int p = decltype(pc)::value;
      if constexpr (p + 1 < G::NPAIR) {
        load_a(std::integral_constant<int, p + 1>{}, (p + 1) & 1);
        if constexpr (!G::SB) load_b(std::integral_constant<int, p + 1>{}, (p + 1) & 1);
      }
      hook(pc);
      // keep the next pair's LDS reads (and the hook's global reads) ahead of
      // this pair's MFMAs: left alone, the scheduler sinks them below the
      // MFMAs and every pair waits out the LDS latency
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < Mma<G::DT>::KSUB; ++k)
#pragma unroll
        for (int i = 0; i < G::FA; ++i)
#pragma unroll
          for (int j = 0; j < G::FB; ++j)
            Mma<G::DT>::step(fa[p & 1][i], fb[G::SB ? 0 : p & 1][j], acc[i][j], k);
      if constexpr (G::SB && p + 1 < G::NPAIR) {
        // one B set: the next pair's B reads follow this pair's MFMAs (the
        // other wave of the SIMD covers their latency)
        __builtin_amdgcn_sched_barrier(0);
        load_b(std::integral_constant<int, p + 1>{}, 0);
      }
    });
  };

  // ---- main loop over stages (chunk, kt), chunk-major.  Stage s+1 is written
  // to LDS after stage s's MFMAs, then one barrier hands it over.
  auto wbuf = [&](int i) -> unsigned char* { return lds + i * G::WBYTES; };
  auto xbuf = [&](int i) -> unsigned char* {
    return lds + G::NBUF * G::WBYTES + i * G::XBYTES;
  };
  // Stage s: packed weights are copied into LDS one stage ahead (they are
  // read from L2), everything else goes through registers two stages ahead.
  // Every step issues the same instructions, so that the compiler can track
  // the outstanding reads exactly: past the last stage the reads repeat the
  // last stage into buffers nobody reads again.
  struct Cursor {
    int chunk, kt, idx;
  };
  auto advance = [&](Cursor& c) {
    if (c.idx + 1 < nstages) {
      ++c.idx;
      if (++c.kt == kt_hi) {
        c.kt = kt_lo;
        ++c.chunk;
      }
    }
  };
  // Reads a wave of role `role` has issued among a step's first lo pieces
  // (weight pieces come first), and the register reads it issues per stage.
  auto issued = [](int role, int lo) constexpr -> int {
    return ((role & 2) ? (lo < NWP ? lo : NWP) : 0) + ((role & 1) ? (lo > NWP ? lo - NWP : 0) : 0);
  };
  auto reg_loads = [](int role) constexpr -> int {
    return ((role & 1) ? G::XPASS * SE : 0) + ((role & 2) ? G::NWREG : 0);
  };
  auto main_loop = [&](auto ragged, auto rolec) __attribute__((always_inline)) {
    constexpr int role = decltype(rolec)::value;
    if constexpr (G::ONE) {  // the one stage: read, write to LDS, multiply
      StageRegs<G> r1;
      const Src qw = w_src(chunk0, kt_lo), qx = x_src(chunk0, kt_lo);
      static_for<0, NWP>([&](auto kc) { read_w(rolec, ragged, kc, qw, r1, wbuf(0)); });
      static_for<0, NXP>([&](auto kc) { read_x(rolec, ragged, kc, qx, r1); });
      wait_vmcnt<0>();
      store_stage(r1, wbuf(0), xbuf(0));
      lds_barrier();
      compute(wbuf(0), xbuf(0), [](auto) {});
      return;
    }
    if constexpr (G::W1) {
      // One weight register set: stage s+1's weights are read in the first
      // kW1Pairs slot pairs of stage s and go to LDS at SPAIR with the input
      // of stage s+1 (read during stage s-1); the input of stage s+2 is read
      // over the remaining pairs.  Weight reads precede the step's input
      // reads, so waiting for all but the input reads issued so far waits
      // for the weights.
      constexpr int PW = kW1Pairs;
      constexpr int NXR = (role & 1) ? NXP : 0;  // this wave's input reads per stage
      StageRegs<G> ra, rb, wr;
      Cursor cw{chunk0, kt_lo, 0}, cx{chunk0, kt_lo, 0};
      {
        const Src qw = w_src(cw.chunk, cw.kt);
        static_for<0, NWP>([&](auto kc) { read_w(rolec, ragged, kc, qw, wr, nullptr); });
        advance(cw);
        const Src qx0 = x_src(cx.chunk, cx.kt);
        static_for<0, NXP>([&](auto kc) { read_x(rolec, ragged, kc, qx0, ra); });
        advance(cx);
        const Src qx1 = x_src(cx.chunk, cx.kt);
        static_for<0, NXP>([&](auto kc) { read_x(rolec, ragged, kc, qx1, rb); });
        advance(cx);
      }
      wait_vmcnt<NXR>();  // stage 0 is in; stage 1's input may be in flight
      store_part(std::integral_constant<int, 2>{}, wr, wbuf(0), nullptr);
      store_part(std::integral_constant<int, 1>{}, ra, nullptr, xbuf(0));
      lds_barrier();
      auto step1 = [&](int s, StageRegs<G>& mine, StageRegs<G>& other)
          __attribute__((always_inline)) {
        const Src qw = w_src(cw.chunk, cw.kt);  // stage s+1
        const Src qx = x_src(cx.chunk, cx.kt);  // stage s+2
        compute(wbuf(s & 1), xbuf(s & 1), [&](auto pc) {
          constexpr int p = decltype(pc)::value;
          if constexpr (p == G::SPAIR) {
            // the input reads issued so far in this step: pairs PW .. SPAIR-1
            constexpr int xin = (role & 1) ? (G::SPAIR - PW) * NXP / (G::NPAIR - PW) : 0;
            wait_vmcnt<xin>();
            store_part(std::integral_constant<int, 2>{}, wr, wbuf((s + 1) & 1), nullptr);
            store_part(std::integral_constant<int, 1>{}, other, nullptr, xbuf((s + 1) & 1));
          }
          if constexpr (p < PW) {
            static_for<p * NWP / PW, (p + 1) * NWP / PW>(
                [&](auto kc) { read_w(rolec, ragged, kc, qw, wr, nullptr); });
          } else {
            static_for<(p - PW) * NXP / (G::NPAIR - PW), (p - PW + 1) * NXP / (G::NPAIR - PW)>(
                [&](auto kc) { read_x(rolec, ragged, kc, qx, mine); });
          }
        });
        advance(cw);
        advance(cx);
        lds_barrier();
      };
      int s = 0;
      for (; s + 1 < nstages; s += 2) {
        step1(s, ra, rb);
        step1(s + 1, rb, ra);
      }
      if (s < nstages) step1(s, ra, rb);
      wait_vmcnt<0>();
      return;
    }
    StageRegs<G> ra, rb;
    Cursor cw{chunk0, kt_lo, 0}, cx{chunk0, kt_lo, 0};  // next stage to read: weights, input
    // all reads of the stage at cursor cx (and, for packed weights, of the
    // stage at cw) at once
    auto read_all = [&](StageRegs<G>& r, unsigned char* wdst) __attribute__((always_inline)) {
      const Src qw = G::PK ? w_src(cw.chunk, cw.kt) : w_src(cx.chunk, cx.kt);
      const Src qx = x_src(cx.chunk, cx.kt);
      static_for<0, NWP>([&](auto kc) { read_w(rolec, ragged, kc, qw, r, wdst); });
      static_for<0, NXP>([&](auto kc) { read_x(rolec, ragged, kc, qx, r); });
      if constexpr (G::PK) advance(cw);
      advance(cx);
    };
    if constexpr (G::PK) {
      read_all(ra, wbuf(0));              // weights of stage 0, input of stage 0
      const Src qx = x_src(cx.chunk, cx.kt);
      static_for<0, NXP>([&](auto kc) { read_x(rolec, ragged, kc, qx, rb); });  // input of stage 1
      advance(cx);
    } else {
      read_all(ra, nullptr);
      read_all(rb, nullptr);
    }
    wait_vmcnt<reg_loads(role)>();
    store_stage(ra, wbuf(0), xbuf(0));
    lds_barrier();
    // Stage s: `mine` is free and receives the input (and OIHW weights) of
    // stage s+2, packed weights of stage s+1 go to the free LDS weight
    // buffer; `other` holds stage s+1.  The reads are spread over the slot
    // pairs, weights first.  Stage s+1 is written from `other` to the free
    // buffer before slot pair SPAIR: by then every read of `other` has had
    // most of a stage to arrive, and the last pairs' MFMAs cover the LDS
    // write latency, so the barrier that ends the stage finds the writes
    // done.  The free buffer held stage s-1, whose reads all finished before
    // the barrier that ended stage s-1.
    auto step = [&](int s, StageRegs<G>& mine, StageRegs<G>& other)
        __attribute__((always_inline)) {
      const Src qw = G::PK ? w_src(cw.chunk, cw.kt) : w_src(cx.chunk, cx.kt);
      const Src qx = x_src(cx.chunk, cx.kt);
      unsigned char* wdst = wbuf((s + 1) & 1);
      compute(wbuf(s & 1), xbuf(s & 1), [&](auto pc) {
        constexpr int p = decltype(pc)::value;
        constexpr int lo = p * (NWP + NXP) / G::NPAIR, hi = (p + 1) * (NWP + NXP) / G::NPAIR;
        if constexpr (p == G::SPAIR) {
          // `other`'s reads precede the reads this step has issued so far
          wait_vmcnt<issued(role, lo)>();
          store_stage(other, wbuf((s + 1) & 1), xbuf((s + 1) & 1));
        }
        static_for<lo, hi>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          if constexpr (k < NWP)
            read_w(rolec, ragged, kc, qw, mine, wdst);
          else
            read_x(rolec, ragged, std::integral_constant<int, k - NWP>{}, qx, mine);
        });
      });
      if constexpr (G::PK) advance(cw);
      advance(cx);
      // packed weights of stage s+1 (copied straight to LDS, the first reads
      // of this step) have landed; the register reads of stage s+2 issued
      // after them may still be in flight
      wait_vmcnt<reg_loads(role)>();
      if constexpr (G::SPAIR < 0) store_stage(other, wbuf((s + 1) & 1), xbuf((s + 1) & 1));
      lds_barrier();
    };
    int s = 0;
    for (; s + 1 < nstages; s += 2) {
      step(s, ra, rb);
      step(s + 1, rb, ra);
    }
    if (s < nstages) step(s, ra, rb);
    wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  };
  // Each wave runs the loop of its role (a wave-uniform branch), in which
  // every step issues a fixed sequence of reads, so that the waits on the
  // reads in flight are exact; every role runs the same barriers.
  auto run_roles = [&](auto ragged, auto&& loop) __attribute__((always_inline)) {
    using R1 = std::integral_constant<int, 1>;
    using R2 = std::integral_constant<int, 2>;
    using R3 = std::integral_constant<int, 3>;
    if constexpr (G::XW == G::NWV && G::W0 == 0) {
      loop(ragged, R3{});
    } else {
      if (xwave && wwave) {
        if constexpr (G::XW > G::W0) loop(ragged, R3{});
      } else if (xwave) {
        if constexpr (G::W0 > 0) loop(ragged, R1{});
      } else {
        if constexpr (G::XW < G::NWV) loop(ragged, R2{});
      }
    }
  };
  // Channel-packed input: weights and input of stage s+1 are both copied
  // straight into the free LDS buffers while stage s is multiplied (spread
  // over its slot pairs); a step ends when the copies have landed and every
  // wave is done with stage s.  The free buffers held stage s-1, whose reads
  // finished before the barrier that ended stage s-1.
  auto main_loop_dma = [&](auto ragged) __attribute__((always_inline)) {
    StageRegs<G> unused;  // packed weights go straight to LDS
    Cursor c{chunk0, kt_lo, 0};
    {
      const Src qw = w_src(c.chunk, c.kt), qx = x_src(c.chunk, c.kt);
      static_for<0, NWP>([&](auto kc) {
        read_w(std::integral_constant<int, 3>{}, ragged, kc, qw, unused, wbuf(0));
      });
      static_for<0, G::NXDMA>([&](auto kc) { read_xd(ragged, kc, qx, xbuf(0)); });
      advance(c);
    }
    wait_vmcnt<0>();
    lds_barrier();
    constexpr int NP = NWP + G::NXDMA;
    for (int s = 0; s < nstages; ++s) {
      const bool more = s + 1 < nstages;
      const Src qw = w_src(c.chunk, c.kt), qx = x_src(c.chunk, c.kt);
      unsigned char* wdst = wbuf((s + 1) & 1);
      unsigned char* xdst = xbuf((s + 1) & 1);
      compute(wbuf(s & 1), xbuf(s & 1), [&](auto pc) {
        constexpr int p = decltype(pc)::value;
        constexpr int lo = p * NP / G::NPAIR, hi = (p + 1) * NP / G::NPAIR;
        if (more) {
          static_for<lo, hi>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            if constexpr (k < NWP)
              read_w(std::integral_constant<int, 3>{}, ragged, kc, qw, unused, wdst);
            else
              read_xd(ragged, std::integral_constant<int, k - NWP>{}, qx, xdst);
          });
        }
      });
      advance(c);
      wait_vmcnt<0>();
      lds_barrier();
    }
  };
  // Channel-packed input with OI(D)HW weights: the input of stage s+1 is
  // copied straight into the free LDS buffer while stage s is multiplied (as
  // packed weights are in the loop above), and the weights go through
  // registers two stages ahead, transposed into LDS before slot pair SPAIR
  // (as the input is there).  A step's copies come before its register
  // reads, so that waiting for all but the register reads waits for the
  // copies.
  auto main_loop_xo = [&](auto ragged, auto rolec) __attribute__((always_inline)) {
    constexpr int role = decltype(rolec)::value;
    constexpr int NXD = G::NXDMA;                 // copy pieces of a step
    constexpr int NWR = (role & 2) ? G::NWREG : 0;  // this wave's register reads per stage
    StageRegs<G> ra, rb;
    Cursor cd{chunk0, kt_lo, 0}, cr{chunk0, kt_lo, 0};  // next stage to copy / to read weights of
    auto copy_x = [&](auto kc, const Src& q, unsigned char* xdst) __attribute__((always_inline)) {
      if constexpr ((role & 1) != 0) read_xd(ragged, kc, q, xdst);
    };
    auto read_ws = [&](StageRegs<G>& r) __attribute__((always_inline)) {
      const Src qw = w_src(cr.chunk, cr.kt);
      static_for<0, G::NWREG>([&](auto kc) { read_w(rolec, ragged, kc, qw, r, nullptr); });
      advance(cr);
    };
    {
      const Src qx = x_src(cd.chunk, cd.kt);
      static_for<0, NXD>([&](auto kc) { copy_x(kc, qx, xbuf(0)); });
      advance(cd);
    }
    read_ws(ra);
    read_ws(rb);
    wait_vmcnt<NWR>();  // stage 0's copies and weights are in; stage 1's weights may be in flight
    store_stage(ra, wbuf(0), xbuf(0));
    lds_barrier();
    // reads of role `role` among a step's first lo pieces (copies first)
    auto issued_xo = [](int lo) constexpr -> int {
      return ((role & 1) ? (lo < NXD ? lo : NXD) : 0) + ((role & 2) ? (lo > NXD ? lo - NXD : 0) : 0);
    };
    auto step = [&](int s, StageRegs<G>& mine, StageRegs<G>& other)
        __attribute__((always_inline)) {
      const Src qx = x_src(cd.chunk, cd.kt);  // stage s+1
      const Src qw = w_src(cr.chunk, cr.kt);  // stage s+2
      unsigned char* xdst = xbuf((s + 1) & 1);
      compute(wbuf(s & 1), xbuf(s & 1), [&](auto pc) {
        constexpr int p = decltype(pc)::value;
        constexpr int NP = NXD + G::NWREG;
        constexpr int lo = p * NP / G::NPAIR, hi = (p + 1) * NP / G::NPAIR;
        if constexpr (p == G::SPAIR) {
          // `other`'s weight reads precede every read this step has issued
          wait_vmcnt<issued_xo(lo)>();
          store_stage(other, wbuf((s + 1) & 1), xbuf((s + 1) & 1));
        }
        static_for<lo, hi>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          if constexpr (k < NXD)
            copy_x(kc, qx, xdst);
          else
            read_w(rolec, ragged, std::integral_constant<int, k - NXD>{}, qw, mine, nullptr);
        });
      });
      advance(cd);
      advance(cr);
      wait_vmcnt<NWR>();  // this step's copies have landed
      if constexpr (G::SPAIR < 0) store_stage(other, wbuf((s + 1) & 1), xbuf((s + 1) & 1));
      lds_barrier();
    };
    int s = 0;
    for (; s + 1 < nstages; s += 2) {
      step(s, ra, rb);
      step(s + 1, rb, ra);
    }
    if (s < nstages) step(s, ra, rb);
    wait_vmcnt<0>();  // no copy into LDS may outlive the workgroup
  };
  if (nstages > 0) {
    if constexpr (G::XP && G::PK) {
      if (cgs % G::CG == 0)
        main_loop_dma(std::false_type{});
      else
        main_loop_dma(std::true_type{});
    } else if constexpr (G::XP) {
      // OI(D)HW weights need C a multiple of the group (the planner's rule),
      // so a ragged last chunk is the same test on channels or groups
      if (a.C % G::CK == 0)
        run_roles(std::false_type{}, main_loop_xo);
      else
        run_roles(std::true_type{}, main_loop_xo);
    } else {
      if (a.C % G::CK == 0)
        run_roles(std::false_type{}, main_loop);
      else
        run_roles(std::true_type{}, main_loop);
    }
  }

  // ---- epilogue
  const int ohw = a.OH * a.OW;
  if (a.ksplit > 1) {  // fp32 partial sums of this split, one writer per element
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.part, a.part_bytes);
#pragma unroll
    for (int i = 0; i < G::FA; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int co = co0 + co_w0 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        const int cbase = (((split * a.N + n) * a.K + co) * a.OT + ot) * ohw;
#pragma unroll
        for (int j = 0; j < G::FB; ++j) {
          const int b = blk0 + j;
          const int oh = oh0 + b / G::BPR;
          const int ow = ow0 + (b % G::BPR) * 32 + il;
          if (co < a.K && oh < a.OH && ow < a.OW)
            Elem<DT_F32>::store(acc[i][j][r], pr, (cbase + oh * a.OW + ow) * 4);
        }
      }
    return;
  }
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, a.y_bytes);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.b, a.b_bytes);
  if constexpr (G::XP) {
    // Channel-packed output: accumulator elements 4q .. 4q+3 of a lane are
    // 4 consecutive output channels of one pixel (rows 8q + 4hf .. +3 of the
    // 32x32 block), i.e. half a 16-byte group (16-bit) or a whole one (fp32):
    // one store each, the 32 pixels of a half-wave side by side.  Channels
    // past C_out in the last group are written as 0 (their packed weights
    // and bias read 0).
    const int kgs = (a.K + SE - 1) / SE;
#pragma unroll
    for (int i = 0; i < G::FA; ++i) {
      float bias[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int co = co0 + co_w0 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        bias[r] = E::load(br, guard_offset(a.b && co < a.K, co * EB));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cob = co0 + co_w0 + i * 32 + 8 * q + 4 * hf;
        const int grp = cob / SE, sub = cob % SE;
#pragma unroll
        for (int j = 0; j < G::FB; ++j) {
          const int b = blk0 + j;
          const int oh = oh0 + b / G::BPR;
          const int ow = ow0 + (b % G::BPR) * 32 + il;
          const bool ok = grp < kgs && oh < a.OH && ow < a.OW;
          const int off = ((((n * kgs + grp) * a.OT + ot) * a.OH + oh) * a.OW + ow) * 16 + sub * EB;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = epilogue(acc[i][j][4 * q + e], bias[4 * q + e], a.relu);
          if constexpr (EB == 4) {
            const u32x4_t word{__builtin_bit_cast(uint32_t, v[0]), __builtin_bit_cast(uint32_t, v[1]),
                               __builtin_bit_cast(uint32_t, v[2]), __builtin_bit_cast(uint32_t, v[3])};
            __builtin_amdgcn_raw_buffer_store_b128(word, yr, guard_offset(ok, off), 0, kOutPolicy);
          } else {
            const u32x2_t word{(uint32_t)E::from_f32(v[0]) | ((uint32_t)E::from_f32(v[1]) << 16),
                               (uint32_t)E::from_f32(v[2]) | ((uint32_t)E::from_f32(v[3]) << 16)};
            __builtin_amdgcn_raw_buffer_store_b64(word, yr, guard_offset(ok, off), 0, kOutPolicy);
          }
        }
      }
    }
    return;
  }
  if constexpr (G::POOLABLE) {
    if (a.pool) {
      // Fused 2x2 stride-2 max pooling: blocks j and j+1 of the wave are output
      // rows oh (even) and oh+1; both go, after bias and activation, into two
      // wave-private fp32 LDS tiles, and lane (row = channel, half h) takes the
      // max over each 2x2 window of 8 pooled columns.  max commutes with the
      // monotonic rounding to the storage dtype, so pooling the fp32 values
      // and rounding once equals rounding every conv output, then pooling.
      lds_barrier();  // the stage buffers are free (as for the vectorised epilogue)
      constexpr int PE = 36;                         // LDS row pitch in floats
      float* ta = reinterpret_cast<float*>(lds) + wave * 2 * 32 * PE;
      float* tb = ta + 32 * PE;
      const int ohp_n = a.OH / 2, owp_n = a.OW / 2;  // pooled extents
      const int prow = lane & 31, ph = lane >> 5;
      constexpr int VP = 16 / EB;                    // pooled outputs per 16-byte store
#pragma unroll
      for (int i = 0; i < G::FA; ++i) {
        float bias[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int co = co0 + co_w0 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          bias[r] = E::load(br, guard_offset(a.b && co < a.K, co * EB));
        }
#pragma unroll
        for (int jp = 0; jp < G::FB / 2; ++jp) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * hf + (r & 3);
            ta[row * PE + il] = epilogue(acc[i][2 * jp][r], bias[r], a.relu);
            tb[row * PE + il] = epilogue(acc[i][2 * jp + 1][r], bias[r], a.relu);
          }
          lds_fence();
          float m[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int c = 16 * ph + 2 * q;
            m[q] = fmaxf(fmaxf(ta[prow * PE + c], ta[prow * PE + c + 1]),
                         fmaxf(tb[prow * PE + c], tb[prow * PE + c + 1]));
          }
          lds_fence();
          const int co = co0 + co_w0 + i * 32 + prow;
          const int ohp = (oh0 + blk0 + 2 * jp) / 2;
          const int owp = ow0 / 2 + 8 * ph;
          const bool ok = co < a.K && ohp < ohp_n;
          const int off = ((n * a.K + co) * ohp_n + ohp) * owp_n + owp;
          if (a.vec_out) {  // pooled rows of whole 16-byte vectors: owp .. owp+7 in or out together
#pragma unroll
            for (int v = 0; v < 8 / VP; ++v) {
              u32x4_t word;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if constexpr (EB == 4)
                  word[e] = __builtin_bit_cast(uint32_t, m[v * VP + e]);
                else
                  word[e] = (uint32_t)E::from_f32(m[v * VP + 2 * e]) |
                            ((uint32_t)E::from_f32(m[v * VP + 2 * e + 1]) << 16);
              }
              __builtin_amdgcn_raw_buffer_store_b128(
                  word, yr, guard_offset(ok && owp + v * VP < owp_n, (off + v * VP) * EB), 0, kOutPolicy);
            }
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (ok && owp + q < owp_n) E::store_out(m[q], yr, (off + q) * EB);
          }
        }
      }
      return;
    }
  }
  if (a.vec_out) {
    // Rows of whole 16-byte vectors: each 32x32 block goes through a
    // wave-private LDS tile and leaves as 16-byte row segments, VEC outputs
    // per store instead of one.  The stage buffers are free once every wave
    // has finished its last reads of them and its last copies into them (each
    // wave waits for its own copies at the end of the main loop): one barrier.
    lds_barrier();
    constexpr int VEC = 16 / EB;                   // outputs per 16-byte store
    constexpr int PITCH_E = 32 + VEC;              // LDS row pitch in elements (16 B aligned)
    constexpr int SEGS = 32 / VEC;                 // 16-byte segments per row
    constexpr int ROWS_PER_READ = 64 / SEGS;       // rows one wave-wide read covers
    unsigned char* tile = lds + wave * (32 * PITCH_E * EB);
#pragma unroll
    for (int i = 0; i < G::FA; ++i) {
      float bias[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int co = co0 + co_w0 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        bias[r] = E::load(br, guard_offset(a.b && co < a.K, co * EB));
      }
#pragma unroll
      for (int j = 0; j < G::FB; ++j) {
        // accumulator element r of this lane: row 8 (r / 4) + 4 hf + r % 4, column il
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * hf + (r & 3);
          const float v = epilogue(acc[i][j][r], bias[r], a.relu);
          if constexpr (EB == 4)
            *reinterpret_cast<float*>(tile + (row * PITCH_E + il) * 4) = v;
          else
            *reinterpret_cast<uint16_t*>(tile + (row * PITCH_E + il) * 2) = E::from_f32(v);
        }
        lds_fence();
        const int b = blk0 + j;
        const int oh = oh0 + b / G::BPR;
        const int owb = ow0 + (b % G::BPR) * 32;
#pragma unroll
        for (int k = 0; k < 32 / ROWS_PER_READ; ++k) {
          const int row = lane / SEGS + k * ROWS_PER_READ;
          const int seg = lane % SEGS;
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(tile + (row * PITCH_E + seg * VEC) * EB);
          const int co = co0 + co_w0 + i * 32 + row;
          const int ow = owb + seg * VEC;
          const int off = (((n * a.K + co) * a.OT + ot) * ohw + oh * a.OW + ow) * EB;
          // a.OW is a multiple of VEC, so a segment is wholly inside or
          // wholly outside the row; outside the output the store is dropped
          __builtin_amdgcn_raw_buffer_store_b128(
              v, yr, guard_offset(co < a.K && oh < a.OH && ow < a.OW, off), 0, kOutPolicy);
        }
        lds_fence();
      }
    }
    return;
  }
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
          E::store_out(epilogue(acc[i][j][r], bias[i][r], a.relu), yr,
                   (cbase + oh * a.OW + ow) * EB);
      }
    }
  }
}


// Launch of a tile kernel, and its occupancy from the runtime; defined in
// igemm_launch.h and instantiated per tile in the igemm_inst_*.hip units.
using LaunchFn = hipError_t (*)(const IgemmArgs&, unsigned, hipStream_t);
using OccFn = int (*)();
template <class G>
hipError_t launch_cfg(const IgemmArgs& a, unsigned grid, hipStream_t s);
template <class G>
int occupancy_cfg();

}  // namespace igk
}  // namespace libconv
