// igemm_inst_a.hip -- instantiates the implicit-GEMM kernel for the tiles of
// igemm_tiles_a.def (16-bit operands, 2-D, OIHW weights transposed in the kernel).
#include "igemm_launch.h"

#include "igemm_tiles_a.def"
