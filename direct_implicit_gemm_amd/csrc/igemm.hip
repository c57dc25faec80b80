// igemm.hip -- implicit-GEMM convolution on the gfx950 matrix cores (MFMA):
// weight packing, the split-K sum, the tile table, the planner and the launch.
// The kernel itself is igemm_kernel.h.
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
#include "igemm_kernel.h"

namespace libconv {
namespace {

using namespace igk;

// ------------------------------------------------------------ weight packing
// w [K][C][TS] -> wp [Kp/64][G = ceil(C/SE)][TS][64][SE] (16 bytes per
// entry), zero for channels >= C and output channels >= K.  A block of 64
// output channels is contiguous: an MFMA tile streams its weights from one
// range instead of 1 KB pieces at a stride of Kp entries, which spread a
// tile's weights over a fraction of the L2 sets.  One thread per (output
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
  store_packed<SE, TS, 0>(pr, (((co >> 6) * a.G + g) * TS * 64 + (co & 63)) * 16, 64 * 16, v);
}

// The same packing when C is a multiple of the channel group: one workgroup
// per block of 64 output channels x one channel group.  The block's 64 rows
// of SE * TS contiguous elements are read whole (consecutive lanes read
// consecutive 16-byte pieces of a row) into LDS, rows one dword apart in
// banks; then each thread takes one output channel and every fourth tap,
// gathers the SE channels of each of its taps from the row and writes the
// slot vector.  Lanes hold consecutive output channels, so each store of a
// wave writes 1 KB contiguous, as above.
template <int DT, int TS>
__global__ __launch_bounds__(kThreads) void pack_rows_kernel(PackArgs a) {
  using E = Elem<DT>;
  constexpr int SE = Mma<DT>::SE;
  constexpr int EB = E::bytes;
  constexpr int ROWW = SE * TS * EB / 4 + 1;  // row pitch in dwords (odd: no bank conflicts)
  __shared__ uint32_t rows[64 * ROWW];
  const int g = blockIdx.x % a.G, cb = blockIdx.x / a.G;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.w, a.w_bytes);
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.wp, a.wp_bytes);
#pragma unroll
  for (int v0 = 0; v0 < 64 * TS; v0 += kThreads) {
    const int v = v0 + tid;
    if (v < 64 * TS) {
      const int row = v / TS, k = v % TS;
      const int co = cb * 64 + row;
      const u32x4_t x = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                       wr, guard_offset(co < a.K, (co * a.C + g * SE) * TS * EB + k * 16), 0, 0));
#pragma unroll
      for (int m = 0; m < 4; ++m) rows[row * ROWW + k * 4 + m] = x[m];
    }
  }
  __syncthreads();
  const int co_l = tid & 63;
  const uint32_t* r = rows + co_l * ROWW;
  auto elem = [&](int c, int t) -> uint32_t {  // element (channel c, tap t) of the row
    const int e = c * TS + t;
    if constexpr (EB == 4) {
      return r[e];
    } else {
      const uint32_t d = r[e >> 1];
      return (e & 1) ? (d >> 16) : (d & 0xffffu);
    }
  };
#pragma unroll
  for (int t = tid >> 6; t < TS; t += kThreads / 64) {
    u32x4_t o;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      o[m] = EB == 4 ? elem(m, t) : (elem(2 * m, t) | (elem(2 * m + 1, t) << 16));
    __builtin_amdgcn_raw_buffer_store_b128(o, pr, (((cb * a.G + g) * TS + t) * 64 + co_l) * 16, 0,
                                           0);
  }
}

// ------------------------------------------------------------ split-K sum
// y[e] = act(b[co] + sum_{s < S} part[s][e]) rounded once to the storage
// dtype, the slices added in order s = 0, 1, ... (so the result does not
// depend on timing).  Thread i takes 4 consecutive outputs of one channel
// plane when the plane length is a multiple of 4, else one output.
struct ReduceArgs {
  const float* part;
  const void* b;
  void* y;
  int S, K, plane, relu;
  // output channels written: K, or for channel-packed y (the _cpack kernel)
  // K rounded up to whole groups (the channels past K are written as 0)
  int K_out;
  long long n_out;  // N * K_out * plane
  uint32_t part_bytes, b_bytes, y_bytes;
};

template <int DT, int V>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(ReduceArgs a) {
  using E = Elem<DT>;
  const long long e0 = ((long long)blockIdx.x * kThreads + threadIdx.x) * V;
  if (e0 >= a.n_out) return;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.part, a.part_bytes);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.b, a.b_bytes);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, a.y_bytes);
  const int co = (int)((e0 / a.plane) % a.K);
  const float bias = E::load(br, guard_offset(a.b != nullptr, co * E::bytes));
  float v[V];
#pragma unroll
  for (int m = 0; m < V; ++m) v[m] = 0.0f;
  for (int sp = 0; sp < a.S; ++sp) {
    const int off = (int)((sp * a.n_out + e0) * 4);
    if constexpr (V == 4) {
      const float4_t q = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(pr, off, 0, 0));
#pragma unroll
      for (int m = 0; m < 4; ++m) v[m] += q[m];
    } else {
      v[0] += Elem<DT_F32>::load(pr, off);
    }
  }
#pragma unroll
  for (int m = 0; m < V; ++m)
    E::store_out(epilogue(v[m], bias, a.relu), yr, (int)((e0 + m) * E::bytes));
}

// The same sum for channel-packed y: one thread per output channel group of
// one pixel, u = (n, group, s); lanes walk s, so each channel's partial sums
// are read as contiguous runs across the wave and the 16-byte groups are
// written contiguously.  Channels past K read nothing and are written as 0.
template <int DT>
__global__ __launch_bounds__(kThreads) void splitk_reduce_cpack_kernel(ReduceArgs a) {
  using E = Elem<DT>;
  constexpr int SE = 16 / E::bytes;
  const long long u = (long long)blockIdx.x * kThreads + threadIdx.x;
  const int groups = a.K_out / SE;
  if (u >= (long long)a.n_out / SE) return;
  const int s = (int)(u % a.plane);
  const long long ng = u / a.plane;
  const int g = (int)(ng % groups);
  const long long n = ng / groups;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.part, a.part_bytes);
  const __amdgpu_buffer_rsrc_t br = make_rsrc(a.b, a.b_bytes);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(a.y, a.y_bytes);
  const long long part_elems = (long long)a.part_bytes / 4 / a.S;
  float v[SE];
#pragma unroll
  for (int j = 0; j < SE; ++j) {
    const int co = g * SE + j;
    const bool real = co < a.K;
    float acc = 0.0f;
    for (int sp = 0; sp < a.S; ++sp) {
      const long long e = sp * part_elems + (n * a.K + co) * a.plane + s;
      acc += Elem<DT_F32>::load(pr, guard_offset(real, (int)(e * 4)));
    }
    v[j] = epilogue(acc, E::load(br, guard_offset(a.b != nullptr && real, co * E::bytes)), a.relu);
  }
  u32x4_t w;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if constexpr (SE == 4)
      w[m] = __builtin_bit_cast(uint32_t, v[m]);
    else
      w[m] = (uint32_t)E::from_f32(v[2 * m]) | ((uint32_t)E::from_f32(v[2 * m + 1]) << 16);
  }
  __builtin_amdgcn_raw_buffer_store_b128(w, yr, (int)(u * 16), 0, kOutPolicy);
}

// ------------------------------------------------------------------ tiles
struct TileDesc {
  int id;
  int wide;       // 0: fp32 operands, 1: 16-bit operands
  int KT, KH, KW, SH, SW;
  int flat;       // 1: 1x1 stride-1 pad-0 layer viewed as one long row per plane
  int BM, TH, TW, CG;
  int packed;     // 1: reads packed weights
  int vx;         // 1: reads the input as aligned 16-byte runs (W a multiple of the run);
                  // 2: channel-packed activations (input copied straight to LDS)
  int eff;        // fraction of MFMA peak one CU reaches on this tile, in percent
                  // (measured on MI355X on large grids; used to rank tiles)
  int occ;        // workgroups one CU holds at once (registers and LDS of the
                  // built kernel; checked against the runtime by a GPU test)
  int one;        // 1: single-stage tile (the layer's input channels fit one stage)
  int pool;       // 1: can fuse the 2x2 max pooling into its epilogue
  int w1;         // 1: OIHW weights through one register set (read one stage ahead)
  int lds;
  const char* name;
  LaunchFn fn[3];  // by libconv_dtype
  OccFn occ_fn[3];
};

// Launcher of a tile for one storage dtype, or null when the tile's operand
// width does not match the dtype.
template <int DT, int WIDE, int KT, int KH, int KW, int SH, int SW, int BM, int TH, int TW,
          int WM, int WN, int CG, int PK, int VX>
constexpr LaunchFn launcher() {
  if constexpr ((DT == DT_F32) == (WIDE == 0))
    return &launch_cfg<Cfg<DT, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>>;
  else
    return nullptr;
}
template <int DT, int WIDE, int KT, int KH, int KW, int SH, int SW, int BM, int TH, int TW,
          int WM, int WN, int CG, int PK, int VX>
constexpr OccFn occupier() {
  if constexpr ((DT == DT_F32) == (WIDE == 0))
    return &occupancy_cfg<Cfg<DT, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>>;
  else
    return nullptr;
}

#define LIBCONV_TILE(ID, WIDE, KT, KH, KW, SH, SW, FLAT, BM, TH, TW, WM, WN, CG, PK, VX, EFF,   \
                     OCC, NAME)                                                                 \
  {ID, WIDE, KT, KH, KW, SH, SW, FLAT, BM, TH, TW, CG, (PK) & 1, VX, EFF, OCC, ((PK) >> 1) & 1, \
   !(FLAT) && Cfg<WIDE ? DT_F16 : DT_F32, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK,       \
                  VX>::POOLABLE,                                                                \
   ((PK) >> 2) & 1,                                                                             \
   Cfg<WIDE ? DT_F16 : DT_F32, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>::LDS, NAME, \
   {launcher<DT_F32, WIDE, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>(),               \
    launcher<DT_F16, WIDE, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>(),               \
    launcher<DT_BF16, WIDE, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>()},              \
   {occupier<DT_F32, WIDE, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>(),               \
    occupier<DT_F16, WIDE, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>(),               \
    occupier<DT_BF16, WIDE, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>()}},

const TileDesc kTiles[] = {
#include "igemm_tiles_a.def"
#include "igemm_tiles_b.def"
#include "igemm_tiles_c.def"
#include "igemm_tiles_d.def"
#include "igemm_tiles_e.def"
};

#undef LIBCONV_TILE

const TileDesc* find_tile(int id) {
  for (const auto& t : kTiles)
    if (t.id == id) return &t;
  return nullptr;
}

bool is_flat(const Problem& p) {
  return p.KT == 1 && p.KH == 1 && p.KW == 1 && p.st == 1 && p.sh == 1 && p.sw == 1 &&
         p.pt == 0 && p.ptb == 0 && p.ph == 0 && p.pw == 0;
}

bool tile_fits(const TileDesc& t, const Problem& p) {
  const int wide = p.dtype == LIBCONV_F32 ? 0 : 1;
  if (t.wide != wide) return false;
  const int se = wide ? 8 : 4;
  // 16-byte weight vectors read from OIHW must not straddle channels; packed
  // weights are zero-padded to whole groups instead.
  if (!t.packed && p.C % se != 0) return false;
  // channel-packed activations only on the tiles made for them; their
  // copies and stores move 16-byte channel groups
  if ((t.vx == 2) != p.cpack) return false;
  if (t.vx == 2 && ((reinterpret_cast<uintptr_t>(p.x) | reinterpret_cast<uintptr_t>(p.y)) & 15))
    return false;
  // 16-byte runs (8 pixels of a 16-bit type, 4 of fp32): rows (flattened
  // planes for 1x1 tiles) of whole runs, and an input aligned for 16-byte reads
  if (t.vx == 1) {
    const long long row = t.flat ? (long long)p.H * p.W : p.W;
    if (row % (16 / dtype_bytes(p.dtype)) != 0 || (reinterpret_cast<uintptr_t>(p.x) & 15) != 0)
      return false;
  }
  if (t.one && (p.C > t.CG * se || p.KT != 1)) return false;
  if (p.pool && !t.pool) return false;
  if (t.flat) return is_flat(p);
  return p.KT == t.KT && p.KH == t.KH && p.KW == t.KW && p.sh == t.SH && p.sw == t.SW &&
         (t.KT > 1 || (p.st == 1 && p.pt == 0 && p.ptb == 0));
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
  if (a.C % Mma<DT>::SE == 0)  // whole groups: block-wise, rows read whole
    hipLaunchKernelGGL((pack_rows_kernel<DT, TS>), dim3(a.Kp / 64 * a.G), dim3(kThreads), 0, s, a);
  else
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

int igemm_tile_occupancy(int id, int dtype, bool measured) {
  const TileDesc* t = find_tile(id);
  if (!t || dtype < 0 || dtype > 2 || !t->fn[dtype]) return -1;
  return measured ? t->occ_fn[dtype]() : t->occ;
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

// Output elements and fp32 partial-sum bytes of a split-K launch.
static long long out_elems(const Problem& p) { return (long long)p.N * p.K * p.OT * p.OH * p.OW; }
static long long part_bytes(const Problem& p, int ksplit) { return ksplit * out_elems(p) * 4; }

// Chunks of channels per split, and whether a split count is usable: every
// split gets at least two chunks and the partial sums stay addressable.
static int chunks_of(const TileDesc& t, const Problem& p) {
  const int ck = t.CG * (t.wide ? 8 : 4);
  return (p.C + ck - 1) / ck;
}
static bool split_ok(const TileDesc& t, const Problem& p, int ksplit) {
  if (ksplit == 1) return true;
  const int chunks = chunks_of(t, p);
  const int cps = (chunks + ksplit - 1) / ksplit;
  return cps >= 2 && (long long)(ksplit - 1) * cps < chunks && part_bytes(p, ksplit) < 0x7fff0000LL;
}

// Estimated time of a tile and split on this shape, in microseconds.  The
// busiest compute unit runs ceil(units / CUs) work units (tiles, times the
// split count), occ of them at a time (one round).  A round takes the longer
// of (a) the MFMA work of its units, which share the CU's matrix cores, at the
// tile's measured efficiency, and (b) the latency chain of one workgroup:
// about kFirstUs (launch, first reads, last stores) plus kStageUs per stage,
// the time a stage's reads take to arrive when no MFMA work hides them
// (fitted to single-round launches on MI355X: a one-stage 1x1 tile takes 5-7
// us, a four-stage 3x3 tile 10-12 us).  Packed tiles on OIHW weights add the
// pack kernel into the caller's workspace (a launch, plus reading and
// writing the weights once; fitted to the pack kernel's measured times, 6 us
// for 0.9 MB and 9 us for 14 MB).  A split adds the sum kernel: a launch, plus
// writing and reading the fp32 partial sums once and writing the output.
constexpr double kFirstUs = 4.5;
constexpr double kStageUs = 1.6;
// A one-weight-set tile reads the next stage's weights within the stage, so
// a stage's chain is longer when no other workgroup hides it (fitted to the
// 1280-channel UNet layer, 160 tiles: 140 vs 100 us for the two-set tile).
constexpr double kStageUsW1 = 2.2;
static double estimate_us(const TileDesc& t, const Problem& p, const TileCounts& c, int ksplit) {
  const double ck = t.CG * (t.wide ? 8 : 4);
  const int chunks = chunks_of(t, p);
  const double cps = std::ceil((double)chunks / ksplit);
  const double unit_flop = 2.0 * t.BM * t.TH * t.TW * cps * ck * p.KT * p.KH * p.KW;
  const double cu_flop_per_us = (t.wide ? 4096.0 : 256.0) * 2400.0 * (t.eff / 100.0);
  const double unit_us = unit_flop / cu_flop_per_us;
  const double latency_us = kFirstUs + (t.w1 ? kStageUsW1 : kStageUs) * cps * p.KT;
  const double cus = p.cus > 0 ? p.cus : 256.0;
  const double per_cu = std::ceil(c.total * ksplit / cus);
  const double full_rounds = std::floor(per_cu / t.occ);
  const double rest = per_cu - full_rounds * t.occ;
  double us = full_rounds * std::max(t.occ * unit_us, latency_us);
  if (rest > 0) us += std::max(rest * unit_us, latency_us);
  if (t.packed && !p.wp) {
    const double wbytes = (double)packed_weight_bytes(p.C, p.K, p.KT, p.KH, p.KW, p.dtype);
    us += 5.0 + 2.0 * wbytes / 6.5e6;
  }
  if (ksplit > 1)
    us += 8.0 + (2.0 * part_bytes(p, ksplit) + out_elems(p) * dtype_bytes(p.dtype)) / 4.0e6;
  return us;
}

// Workspace layout of a plan: the packed copy of OIHW weights (when the tile
// reads packed weights and the caller passed none) at offset 0, then the
// split-K partial sums at the next 256-byte boundary.
static long long align256(long long b) { return (b + 255) / 256 * 256; }
static long long packed_part(const TileDesc& t, const Problem& p) {
  return t.packed && !p.wp ? align256(packed_weight_bytes(p.C, p.K, p.KT, p.KH, p.KW, p.dtype))
                           : 0;
}
static long long ws_need(const TileDesc& t, const Problem& p, int ksplit) {
  return packed_part(t, p) + (ksplit > 1 ? align256(part_bytes(p, ksplit)) : 0);
}

// Split count forced for tests and A/B runs (LIBCONV_FORCE_KSPLIT), else 0.
static int forced_ksplit() {
  const char* e = std::getenv("LIBCONV_FORCE_KSPLIT");
  return e ? std::atoi(e) : 0;
}

// Among the tiles that fit (packed or not, as asked) and the split counts
// 1..4, the pair with the smallest estimated time.
static bool plan_among(const Problem& p, int want_packed, Plan* plan) {
  const TileDesc* best = nullptr;
  double best_cost = 0.0;
  long long best_total = 0;
  int best_split = 1;
  const int fk = forced_ksplit();
  for (const auto& t : kTiles) {
    if (want_packed >= 0 && t.packed != want_packed) continue;
    if (!tile_fits(t, p) || !t.fn[p.dtype]) continue;
    if (ws_need(t, p, 1) > p.ws_bytes) continue;  // would pack without room to pack into
    const TileCounts c = counts(t, p);
    for (int ks = 1; ks <= (p.pool ? 1 : 4); ++ks) {
      if ((fk > 0 && ks != fk && ws_need(t, p, fk) <= p.ws_bytes) || !split_ok(t, p, ks) ||
          ws_need(t, p, ks) > p.ws_bytes)
        continue;
      const double cost = estimate_us(t, p, c, ks);
      if (!best || cost < best_cost) {
        best = &t;
        best_cost = cost;
        best_total = c.total;
        best_split = ks;
      }
    }
  }
  if (!best) return false;
  plan->algo = LIBCONV_ALGO_IGEMM;
  plan->tile = best->id;
  plan->ksplit = best_split;
  plan->grid = best_total * best_split;
  return true;
}

bool igemm_plan(const Problem& p, Plan* plan) { return plan_among(p, -1, plan); }

long long plan_workspace(const Problem& p, const Plan& plan) {
  if (plan.algo != LIBCONV_ALGO_IGEMM) return 0;
  const TileDesc* t = find_tile(plan.tile);
  return t ? ws_need(*t, p, plan.ksplit > 1 ? plan.ksplit : 1) : 0;
}

bool igemm_plan_packed(const Problem& p, Plan* plan) { return plan_among(p, 1, plan); }

bool igemm_plan_tile(const Problem& p, int tile_id, Plan* plan) {
  const TileDesc* t = find_tile(tile_id);
  if (!t || !tile_fits(*t, p) || !t->fn[p.dtype]) return false;
  if (ws_need(*t, p, 1) > p.ws_bytes) return false;
  const int fk = p.pool ? 1 : forced_ksplit();
  plan->algo = LIBCONV_ALGO_IGEMM;
  plan->tile = t->id;
  plan->ksplit = fk > 1 && split_ok(*t, p, fk) && ws_need(*t, p, fk) <= p.ws_bytes ? fk : 1;
  plan->grid = counts(*t, p).total * plan->ksplit;
  return true;
}

using ReduceFn = hipError_t (*)(const ReduceArgs&, unsigned, hipStream_t);
template <int DT, int V>
hipError_t launch_reduce(const ReduceArgs& a, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((splitk_reduce_kernel<DT, V>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}
template <int DT>
hipError_t launch_reduce_cpack(const ReduceArgs& a, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL((splitk_reduce_cpack_kernel<DT>), dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

libconv_status igemm_launch(const Problem& p, const Plan& plan) {
  const TileDesc* t = find_tile(plan.tile);
  if (!t || !tile_fits(*t, p)) return LIBCONV_ERR_UNSUPPORTED;
  const LaunchFn fn = t->fn[p.dtype];
  if (!fn) return LIBCONV_ERR_UNSUPPORTED;
  const int ks = plan.ksplit > 1 ? plan.ksplit : 1;
  if (!split_ok(*t, p, ks) || (ks > 1 && p.pool)) return LIBCONV_ERR_UNSUPPORTED;
  if (ws_need(*t, p, ks) > p.ws_bytes || (ws_need(*t, p, ks) > 0 && !p.ws))
    return LIBCONV_ERR_UNSUPPORTED;
  if (p.pool && !t->pool) return LIBCONV_ERR_UNSUPPORTED;
  const TileCounts c = counts(*t, p);
  if (c.total * ks > 0x7fffffffLL) return LIBCONV_ERR_UNSUPPORTED;
  // The tile reads packed weights but the caller passed OIHW weights: pack
  // them into the head of the workspace first, on the call's stream.
  const void* wpk = p.wp;
  if (t->packed && !wpk) {
    const libconv_status st = pack_launch(p.w, p.ws, p.C, p.K, p.KT, p.KH, p.KW, p.dtype,
                                          p.stream);
    if (st != LIBCONV_OK) return st;
    wpk = p.ws;
  }
  IgemmArgs a;
  a.x = p.x; a.w = t->packed ? wpk : p.w; a.b = p.b; a.y = p.y;
  a.N = p.N; a.C = p.C; a.T = p.T; a.K = p.K; a.OT = p.OT;
  if (t->flat) {  // a 1x1 layer: each plane is one row of H*W pixels
    a.H = 1; a.W = p.H * p.W; a.OH = 1; a.OW = p.OH * p.OW;
  } else {
    a.H = p.H; a.W = p.W; a.OH = p.OH; a.OW = p.OW;
  }
  a.pt = p.pt; a.ph = p.ph; a.pw = p.pw; a.st = p.st;
  a.relu = p.act == LIBCONV_ACT_RELU;
  a.chunks = chunks_of(*t, p);
  a.ksplit = ks;
  a.cps = (a.chunks + ks - 1) / ks;
  a.wblk = (p.C + (t->wide ? 8 : 4) - 1) / (t->wide ? 8 : 4) * p.KT * p.KH * p.KW * 64;
  a.co_tiles = (int)c.co; a.row_tiles = (int)c.rows; a.col_tiles = (int)c.cols;
  const int eb = dtype_bytes(p.dtype);
  // as many output-channel tiles side by side as keep their weights (of one
  // split) within about 4 MB (one XCD's L2).  Measured against 2, 8 and 16 MB
  // on the video-VAE and UNet layers: the 512-channel 3x3x3 layer reads 38 %
  // fewer bytes past L2 and runs 1-3 % faster, and the 640-channel 3x3 layer
  // 16 % fewer and 3 % faster; wider groups thrash the weights.
  const long long w_tile = (long long)t->BM * std::min(p.C, a.cps * t->CG * (t->wide ? 8 : 4)) *
                           p.KT * p.KH * p.KW * eb;
  a.co_group = (int)std::max(1LL, std::min<long long>(c.co, (4LL << 20) / std::max(1LL, w_tile)));
  a.x_bytes = (uint32_t)(p.cpack ? cpack_bytes(p.N, p.C, (long long)p.T * p.H * p.W, p.dtype)
                                 : (long long)p.N * p.C * p.T * p.H * p.W * eb);
  a.w_bytes = t->packed ? (uint32_t)packed_weight_bytes(p.C, p.K, p.KT, p.KH, p.KW, p.dtype)
                        : (uint32_t)((long long)p.K * p.C * p.KT * p.KH * p.KW * eb);
  a.b_bytes = p.b ? (uint32_t)(p.K * eb) : 0u;
  a.y_bytes = (uint32_t)(p.cpack ? cpack_bytes(p.N, p.K, (long long)p.OT * p.OH * p.OW, p.dtype)
                                 : (long long)p.N * p.K * p.OT * p.OH * p.OW * eb);
  a.part = nullptr;
  a.part_bytes = 0;
  a.vec_out = (a.OW % (16 / eb)) == 0 && (reinterpret_cast<uintptr_t>(p.y) & 15) == 0;
  a.pool = p.pool ? 1 : 0;
  // Output frames that share input frames side by side only pay while the
  // tile's weights stay in L2 as well: the edge frames have fewer frame taps
  // (time padding), so the tiles of one wave drift apart in the channel loop
  // and stop sharing each weight read.  Measured on the 3x3x3 video-VAE
  // layers: 442 KB of weights per tile, 8-10% faster; 1.8 MB, 3-6% slower.
  a.frame_fast = (p.KT > 1 && p.OT > 1 && w_tile <= (1LL << 20)) ? 1 : 0;
  if (p.pool) {  // y holds the pooled output
    a.y_bytes = (uint32_t)((long long)p.N * p.K * (p.OH / 2) * (p.OW / 2) * eb);
    a.vec_out = ((p.OW / 2) % (16 / eb)) == 0 && (reinterpret_cast<uintptr_t>(p.y) & 15) == 0;
  }
  if (ks == 1) {
    const hipError_t e = fn(a, (unsigned)c.total, p.stream);
    return e == hipSuccess ? LIBCONV_OK : LIBCONV_ERR_LAUNCH;
  }
  // split-K: partial sums in the workspace (after any packed weights), then
  // the sum kernel
  const long long pb = part_bytes(p, ks);
  void* part = static_cast<char*>(p.ws) + packed_part(*t, p);
  a.part = static_cast<float*>(part);
  a.part_bytes = (uint32_t)pb;
  libconv_status st = LIBCONV_OK;
  if (fn(a, (unsigned)(c.total * ks), p.stream) != hipSuccess) st = LIBCONV_ERR_LAUNCH;
  if (st == LIBCONV_OK) {
    ReduceArgs r;
    r.part = a.part; r.b = p.b; r.y = p.y;
    r.S = ks; r.K = p.K; r.plane = p.OT * p.OH * p.OW; r.relu = a.relu;
    const int se = 16 / eb;
    r.K_out = p.cpack ? (p.K + se - 1) / se * se : p.K;
    r.n_out = (long long)p.N * r.K_out * r.plane;
    r.part_bytes = a.part_bytes; r.b_bytes = a.b_bytes; r.y_bytes = a.y_bytes;
    const bool v4 = r.plane % 4 == 0;
    const int V = p.cpack ? se : v4 ? 4 : 1;
    const unsigned grid = (unsigned)((r.n_out / V + kThreads - 1) / kThreads);
    ReduceFn rf = nullptr;
    switch (p.dtype) {
      case LIBCONV_F32:
        rf = p.cpack ? &launch_reduce_cpack<DT_F32>
                     : v4 ? &launch_reduce<DT_F32, 4> : &launch_reduce<DT_F32, 1>;
        break;
      case LIBCONV_F16:
        rf = p.cpack ? &launch_reduce_cpack<DT_F16>
                     : v4 ? &launch_reduce<DT_F16, 4> : &launch_reduce<DT_F16, 1>;
        break;
      default:
        rf = p.cpack ? &launch_reduce_cpack<DT_BF16>
                     : v4 ? &launch_reduce<DT_BF16, 4> : &launch_reduce<DT_BF16, 1>;
        break;
    }
    if (rf(r, grid, p.stream) != hipSuccess) st = LIBCONV_ERR_LAUNCH;
  }
  return st;
}

}  // namespace libconv
