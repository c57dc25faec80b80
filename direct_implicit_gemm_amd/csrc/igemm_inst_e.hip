// igemm_inst_e.hip -- instantiates the implicit-GEMM kernel for the tiles of
// igemm_tiles_e.def (channel-packed activations (packed weights; input halo copied straight to LDS)).
#include "igemm_launch.h"

#include "igemm_tiles_e.def"
