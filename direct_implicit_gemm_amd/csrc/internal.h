// internal.h -- types shared by the host side of libconv (validation,
// dispatch) and the two kernel families.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "libconv.h"

namespace libconv {

// One convolution call, normalised to the 3-D form (2-D: T = KT = 1,
// pt = 0, st = 1).  K is C_out.  pt pads the frame axis before the first
// frame and ptb after the last (equal unless the caller asked otherwise).
// Output extents are filled by validation.
struct Problem {
  int N, C, T, H, W;
  int K, KT, KH, KW;
  int pt, ph, pw;
  int ptb;
  int st, sh, sw;
  int OT, OH, OW;
  int dtype;  // libconv_dtype
  int act;    // libconv_act
  const void* x;
  const void* w;   // OIHW / OIDHW weights (null when only packed weights are given)
  const void* wp;  // packed weights (libconv_pack_weights layout), or null
  const void* b;   // may be null
  void* y;
  hipStream_t stream;
  int cus;         // compute units of the current device (filled before a launch)
  // Caller-owned device workspace (256-byte aligned) for a plan that packs
  // OIHW weights per call or splits the reduction (split-K partial sums);
  // ws_bytes == 0 (ws null): neither.  Plans depend on ws_bytes, never on
  // whether the stream is being captured into a graph.
  void* ws;
  long long ws_bytes;
  bool pool;       // y is the 2x2 stride-2 max pool of the activated conv output (2-D only)
  // x and y are channel-packed: [N][ceil(C/g)][T][H][W][g] (g channels = 16
  // bytes, zero past C) and likewise y over C_out; else plain NC(T)HW
  bool cpack;
};

// What the dispatcher decided.
struct Plan {
  int algo;         // LIBCONV_ALGO_DIRECT or LIBCONV_ALGO_IGEMM
  int tile;         // tile configuration id (see tile_name)
  long long grid;   // workgroups (of the convolution kernel)
  int ksplit = 1;   // MFMA tiles: workgroups sharing one tile's reduction (split-K)
};

// Workspace bytes a plan needs: the packed copy of OIHW weights when the
// tile reads packed weights and the caller passed OIHW ones, then (256-byte
// aligned) the fp32 partial sums of a split-K plan.  0 for direct plans.
long long plan_workspace(const Problem& p, const Plan& plan);

inline int dtype_bytes(int dt) { return dt == LIBCONV_F32 ? 4 : 2; }

// Direct (vector ALU) family: every shape is supported.
bool direct_plan(const Problem& p, Plan* plan);
// A specific direct tile (the fixed-geometry tap tiles), if it fits the shape.
bool direct_plan_tile(const Problem& p, int tile_id, Plan* plan);
libconv_status direct_launch(const Problem& p, const Plan& plan);

// Implicit-GEMM (MFMA) family: a fixed set of geometries; returns false
// when the shape is not one of them.
bool igemm_plan(const Problem& p, Plan* plan);
// Best tile among those that read packed weights.
bool igemm_plan_packed(const Problem& p, Plan* plan);
// A specific MFMA tile, if it fits the shape.
bool igemm_plan_tile(const Problem& p, int tile_id, Plan* plan);
// Workgroups per compute unit of an MFMA tile for a dtype: the value the
// dispatcher assumes, or (measured) the runtime's figure for the built
// kernel; -1 for an unknown tile or dtype.
int igemm_tile_occupancy(int id, int dtype, bool measured);
// Whether a tile reads packed weights (p.wp) instead of OIHW weights.
bool igemm_tile_packed(int tile_id);
libconv_status igemm_launch(const Problem& p, const Plan& plan);

// Packed weights: [round_up(K, 128) / 64][ceil(C/g)][KT*KH*KW][64][g] 16-byte entries,
// g = 8 channels (16-bit dtypes) or 4 (fp32).
long long packed_weight_bytes(int C, int K, int KT, int KH, int KW, int dtype);
bool pack_supported(int KT, int KH, int KW, int dtype);
libconv_status pack_launch(const void* w, void* wp, int C, int K, int KT, int KH, int KW,
                           int dtype, hipStream_t stream);

// Channel-packed activations: bytes of a tensor, and the conversions from and
// to the plain layout (spatial = T*H*W elements per channel).
long long cpack_bytes(int N, int C, long long spatial, int dtype);
libconv_status layout_launch(const void* src, void* dst, int N, int C, long long spatial,
                             int dtype, bool to_packed, hipStream_t stream);

const char* direct_tile_name(int id);
const char* igemm_tile_name(int id);

}  // namespace libconv
