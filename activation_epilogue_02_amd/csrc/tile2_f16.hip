// tile2_f16.hip -- instantiations of the pipelined tile kernel for f16 inputs.
#include "tile2_kernel.h"

namespace ge {

TileFn pick_tile2_f16(int d_type, int op_b, int tile_id) {
    if (d_type == GE_F16) return pick_op2<GE_F16, GE_F16>(op_b, tile_id);
    if (d_type == GE_F32) return pick_op2<GE_F16, GE_F32>(op_b, tile_id);
    return nullptr;
}

}  // namespace ge
