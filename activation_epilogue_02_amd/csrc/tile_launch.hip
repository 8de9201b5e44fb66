// tile_launch.hip -- launch table of the MFMA tile kernel.
#include "tile2_kernel.h"

namespace ge {

int launch_tile(int tile_id, int a_type, int d_type, int op_b, const KernelArgs& args, unsigned grid,
                void* stream) {
    const TileShape* t = nullptr;
    for (int i = 0; i < kNumTiles; ++i)
        if (kTiles[i].id == tile_id) t = &kTiles[i];
    if (!t) return (int)hipErrorInvalidDeviceFunction;
    const int threads = t->wm * t->wn * 64;
    const unsigned slices = t->kernel == 5 ? (unsigned)args.split_k : 1u;   // split-K tiles: K slices in z
    if (t->kernel >= 2) {
        Tile2Fn fn = nullptr;
        if (a_type == GE_F16 && d_type == GE_F16) fn = pick_tile2_f16_f16(op_b, tile_id);
        else if (a_type == GE_F16 && d_type == GE_F32) fn = pick_tile2_f16_f32(op_b, tile_id);
        else if (a_type == GE_BF16 && d_type == GE_BF16) fn = pick_tile2_bf16_bf16(op_b, tile_id);
        else if (a_type == GE_BF16 && d_type == GE_F32) fn = pick_tile2_bf16_f32(op_b, tile_id);
        else if (a_type == GE_F8_E4M3 && d_type == GE_BF16) fn = pick_tile2_f8_bf16(op_b, tile_id);
        else if (a_type == GE_F8_E4M3 && d_type == GE_F16) fn = pick_tile2_f8_f16(op_b, tile_id);
        else if (a_type == GE_F8_E4M3 && d_type == GE_F32) fn = pick_tile2_f8_f32(op_b, tile_id);
        else if (a_type == GE_BF16 && d_type == GE_F8_E4M3) fn = pick_tile2_bf16_f8(op_b, tile_id);
        else if (a_type == GE_F16 && d_type == GE_F8_E4M3) fn = pick_tile2_f16_f8(op_b, tile_id);
        else if (a_type == GE_F8_E4M3 && d_type == GE_F8_E4M3) fn = pick_tile2_f8_f8(op_b, tile_id);
        if (!fn) return (int)hipErrorInvalidDeviceFunction;
        const MxArgs none = {nullptr, nullptr, 0, 0, 0, 0};
        hipLaunchKernelGGL(fn, dim3(grid, args.batch, slices), dim3(threads), 0, (hipStream_t)stream, args, none);
        return (int)hipGetLastError();
    }
    TileFn fn = nullptr;
    switch (a_type) {
    case GE_F32: fn = pick_tile_f32(d_type, op_b, tile_id); break;
    case GE_F16: fn = pick_tile_f16(d_type, op_b, tile_id); break;
    case GE_BF16: fn = pick_tile_bf16(d_type, op_b, tile_id); break;
    case GE_F8_E4M3: fn = pick_tile_f8(d_type, op_b, tile_id); break;
    }
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    hipLaunchKernelGGL(fn, dim3(grid, args.batch, slices), dim3(threads), 0, (hipStream_t)stream, args);
    return (int)hipGetLastError();
}

int launch_tile_mx(int tile_id, int d_type, int op_b, const KernelArgs& args, const MxArgs& mx, unsigned grid,
                   void* stream) {
    const TileShape* t = nullptr;
    for (int i = 0; i < kNumTiles; ++i)
        if (kTiles[i].id == tile_id) t = &kTiles[i];
    if (!t) return (int)hipErrorInvalidDeviceFunction;
    Tile2Fn fn = nullptr;
    if (d_type == GE_BF16) fn = pick_tile2_mx_f8_bf16(op_b, tile_id);
    else if (d_type == GE_F16) fn = pick_tile2_mx_f8_f16(op_b, tile_id);
    else if (d_type == GE_F32) fn = pick_tile2_mx_f8_f32(op_b, tile_id);
    else if (d_type == GE_F8_E4M3) fn = pick_tile2_mx_f8_f8(op_b, tile_id);
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    hipLaunchKernelGGL(fn, dim3(grid, args.batch, 1), dim3(t->wm * t->wn * 64), 0, (hipStream_t)stream, args, mx);
    return (int)hipGetLastError();
}

}  // namespace ge
