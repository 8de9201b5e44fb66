// tile2_f16_f8.hip -- instantiations of the pipelined tile kernel with fp8 (E4M3)
// output for fp16 inputs (one translation unit per input dtype, so that they
// compile in parallel).
#include "tile2_kernel.h"

namespace ge {

Tile2Fn pick_tile2_f16_f8(int op_b, int tile_id) { return pick_op2_out8<GE_F16>(op_b, tile_id); }

}  // namespace ge
