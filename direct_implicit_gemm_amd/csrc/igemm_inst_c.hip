// igemm_inst_c.hip -- instantiates the implicit-GEMM kernel for the tiles of
// igemm_tiles_c.def (16-bit operands, 3x3x3: packed weights, and OIDHW weights transposed in the kernel).
#include "igemm_launch.h"

#include "igemm_tiles_c.def"
