// tile2_mx_f8.hip -- instantiations of the pipelined tile kernel with fp8 (E4M3)
// output for block-scaled fp8 (MX) inputs (one translation unit per input dtype, so that they
// compile in parallel).
#include "tile2_kernel.h"

namespace ge {

Tile2Fn pick_tile2_mx_f8_f8(int op_b, int tile_id) { return pick_op2_mx<GE_F8_E4M3>(op_b, tile_id); }

}  // namespace ge
