// tile_f32.hip -- instantiations of the MFMA tile kernel for f32 inputs.
#include "tile_kernel.h"

namespace ge {

TileFn pick_tile_f32(int d_type, int op_b, int tile_id) {
    if (d_type == GE_F32) return pick_op<GE_F32, GE_F32>(op_b, tile_id);
    return nullptr;
}

}  // namespace ge
