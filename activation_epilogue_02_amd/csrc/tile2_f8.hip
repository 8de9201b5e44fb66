// tile2_f8.hip -- instantiations of the pipelined tile kernel for fp8 (OCP
// E4M3) inputs.
#include "tile2_kernel.h"

namespace ge {

TileFn pick_tile2_f8(int d_type, int op_b, int tile_id) {
    if (d_type == GE_BF16) return pick_op2<GE_F8_E4M3, GE_BF16>(op_b, tile_id);
    if (d_type == GE_F16) return pick_op2<GE_F8_E4M3, GE_F16>(op_b, tile_id);
    if (d_type == GE_F32) return pick_op2<GE_F8_E4M3, GE_F32>(op_b, tile_id);
    return nullptr;
}

}  // namespace ge
