// igemm_inst_d.hip -- instantiates the implicit-GEMM kernel for the tiles of
// igemm_tiles_d.def (16-bit operands, 2-D, packed weights).
#include "igemm_launch.h"

#include "igemm_tiles_d.def"
