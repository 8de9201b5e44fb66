// tile2_bf16_bf16.hip -- instantiations of the pipelined tile kernel for
// bf16 inputs and bf16 output (one translation unit per dtype pair, so
// that they compile in parallel).
#include "tile2_kernel.h"

namespace ge {

Tile2Fn pick_tile2_bf16_bf16(int op_b, int tile_id) { return pick_op2<GE_BF16, GE_BF16>(op_b, tile_id); }

}  // namespace ge
