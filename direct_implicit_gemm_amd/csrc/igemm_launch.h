// igemm_launch.h -- the host launch and occupancy query of an implicit-GEMM
// tile kernel, and the macros that instantiate them for a tile list
// (igemm_tiles_*.def).  Included only by the igemm_inst_*.hip units.
#pragma once

#include "igemm_kernel.h"

namespace libconv {
namespace igk {

template <class G>
hipError_t launch_cfg(const IgemmArgs& a, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL(igemm_kernel<G>, dim3(grid), dim3(G::NT), 0, s, a);
  return hipGetLastError();
}

// Workgroups of a tile kernel one compute unit holds at once, from the
// runtime (registers and LDS of the built kernel); -1 if the query fails.
template <class G>
int occupancy_cfg() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, igemm_kernel<G>, G::NT, 0) !=
      hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return n;
}

}  // namespace igk
}  // namespace libconv

// One tile of a igemm_tiles_*.def list: instantiate its kernel for the
// storage dtypes of its operand width (fp32, or f16 and bf16).
#define LIBCONV_INST_ONE(DT, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX)              \
  template hipError_t libconv::igk::launch_cfg<                                                \
      libconv::igk::Cfg<DT, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>>(             \
      const libconv::igk::IgemmArgs&, unsigned, hipStream_t);                                 \
  template int libconv::igk::occupancy_cfg<                                                    \
      libconv::igk::Cfg<DT, KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX>>();
#define LIBCONV_INST_W0(...) LIBCONV_INST_ONE(libconv::DT_F32, __VA_ARGS__)
#define LIBCONV_INST_W1(...) \
  LIBCONV_INST_ONE(libconv::DT_F16, __VA_ARGS__) LIBCONV_INST_ONE(libconv::DT_BF16, __VA_ARGS__)
#define LIBCONV_TILE(ID, WIDE, KT, KH, KW, SH, SW, FLAT, BM, TH, TW, WM, WN, CG, PK, VX, EFF,  \
                     OCC, NAME)                                                                \
  LIBCONV_INST_W##WIDE(KT, KH, KW, SH, SW, BM, TH, TW, WM, WN, CG, PK, VX)
