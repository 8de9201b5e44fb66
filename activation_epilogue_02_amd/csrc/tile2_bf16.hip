// tile2_bf16.hip -- instantiations of the pipelined tile kernel for bf16 inputs.
#include "tile2_kernel.h"

namespace ge {

TileFn pick_tile2_bf16(int d_type, int op_b, int tile_id) {
    if (d_type == GE_BF16) return pick_op2<GE_BF16, GE_BF16>(op_b, tile_id);
    if (d_type == GE_F32) return pick_op2<GE_BF16, GE_F32>(op_b, tile_id);
    return nullptr;
}

}  // namespace ge
