// tile2_f16_f32.hip -- instantiations of the pipelined tile kernel for
// fp16 inputs and fp32 output (one translation unit per dtype pair, so
// that they compile in parallel).
#include "tile2_kernel.h"

namespace ge {

Tile2Fn pick_tile2_f16_f32(int op_b, int tile_id) { return pick_op2<GE_F16, GE_F32>(op_b, tile_id); }

}  // namespace ge
