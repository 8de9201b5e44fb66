// tile2_mx_f32.hip -- instantiations of the pipelined tile kernel for MX
// block-scaled fp8 inputs (OCP E4M3 elements, one E8M0 scale per 32 K values)
// and f32 output (one translation unit per output dtype, so that they compile
// in parallel).
#include "tile2_kernel.h"

namespace ge {

Tile2Fn pick_tile2_mx_f8_f32(int op_b, int tile_id) { return pick_op2_mx<GE_F32>(op_b, tile_id); }

}  // namespace ge
