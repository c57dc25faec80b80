// igemm_inst_b.hip -- instantiates the implicit-GEMM kernel for the tiles of
// igemm_tiles_b.def (fp32 operands, 2-D, OIHW weights transposed in the kernel).
#include "igemm_launch.h"

#include "igemm_tiles_b.def"
