// ge_params.h -- kernel argument block and launch-table interface shared by
// the C-ABI front end (api.cpp) and the kernel translation units.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/gemm_epilog.h"

namespace ge {

// Everything a kernel needs, passed by value as the kernel argument.
struct KernelArgs {
    const void* A;
    const void* B;
    const void* bias;      // NULL for GE_EPILOG_NONE
    void* D;
    uint32_t* aux;         // RELU_AUX_BIAS/DRELU: mask words; GELU_AUX_BIAS/DGELU:
                           // pre-activation matrix in D's dtype; else NULL
    const float* scale_a;  // NULL = 1.0
    const float* scale_b;  // NULL = 1.0
    float* partial;        // fp32 partials: split-K (small-m path) or bias gradient, or NULL
    uint32_t* counters;    // split-K arrival counters (small-m path), or NULL
    int32_t m, n, k;
    int32_t epilog, axis;
    int32_t ldaux;         // aux row stride: 32-bit words (mask) or elements (matrix)
    int64_t lda, ldb, ldd;
    int32_t tiles_m, tiles_n;
    int32_t group_m;       // tile-rows per group in the launch order
    int32_t split_k;       // K slices (small-m path)
    int32_t k_per_split;   // K elements per slice, multiple of the k step
    int32_t k_stagger;     // pipelined tiles: full K steps of rotation per
                           // position in the tile group (0 = none)
    // batched launches: the product's index z comes from the launch grid;
    // product z's buffers start z * bs_* bytes after product 0's (a stride
    // of 0 shares one input between all products); counters: elements
    int32_t batch;
    int64_t bs_part, bs_cnt;
    int64_t bs_a, bs_b, bs_bias, bs_d, bs_aux, bs_c;
    // the added input term beta*C (gemm_epilog_execute_c): C in D's dtype
    // with row stride ldc elements, beta a device scalar; cin NULL = none
    const void* cin;
    const float* beta;
    int64_t ldc;
    // fp8 output (E4M3 D): D = E4M3(y * *scale_d) (NULL = 1); amax, if not
    // NULL, receives the largest |y| of each product (one float per product)
    const float* scale_d;
    float* amax;
};
// The arguments of product z of a batched launch: each buffer advanced by
// its per-product stride (bytes; counters in elements).  (The block is
// passed by value; the copy batch_slice makes is taken apart by the
// compiler, since only z == 0 skips the offsets.)
__host__ __device__ inline KernelArgs batch_slice(const KernelArgs& p, int64_t z) {
    KernelArgs q = p;
    if (z == 0) return q;
    q.A = p.A ? (const void*)((const uint8_t*)p.A + z * p.bs_a) : nullptr;
    q.B = p.B ? (const void*)((const uint8_t*)p.B + z * p.bs_b) : nullptr;
    q.bias = p.bias ? (const void*)((const uint8_t*)p.bias + z * p.bs_bias) : nullptr;
    q.D = p.D ? (void*)((uint8_t*)p.D + z * p.bs_d) : nullptr;
    q.aux = p.aux ? (uint32_t*)((uint8_t*)p.aux + z * p.bs_aux) : nullptr;
    q.partial = p.partial ? (float*)((uint8_t*)p.partial + z * p.bs_part) : nullptr;
    q.counters = p.counters ? p.counters + z * p.bs_cnt : nullptr;
    q.cin = p.cin ? (const void*)((const uint8_t*)p.cin + z * p.bs_c) : nullptr;
    q.amax = p.amax ? p.amax + z : nullptr;
    return q;
}

// Block scales of MX (block-scaled) fp8 operands, a second kernel argument of
// the MX instantiations of the pipelined tile kernel: one E8M0 byte per 32
// consecutive K values, for each row of A (sa: m rows) and each column of B
// (sb: n rows, whichever layout B has), rows of `ld` bytes (a multiple of
// 16); kb = ceil(k / 32) blocks are valid in a row.  Product z of a batch
// reads sa + z*bs_sa and sb + z*bs_sb (bytes).
struct MxArgs {
    const uint8_t* sa;
    const uint8_t* sb;
    int32_t ld;
    int32_t kb;
    int64_t bs_sa, bs_sb;
};

// Kernel families.
enum Path : int32_t { PATH_TILE = 1, PATH_SMALLM = 2 };

// Tile shapes of the MFMA tile kernels: block tile BM x BN, waves WM x WN.
// Kernel 1 (tile_kernel.h): register-staged, two LDS stages, every dtype.
// Kernel 2 (tile2_kernel.h): direct-to-LDS copies through up to `stages`
// LDS stages (as many as fit in 160 KiB), fp16/bf16/fp8 inputs.
// Kernel 3: the same kernel with register-staged copies (global loads two
// steps ahead into registers, then LDS writes; two LDS stages).
// Kernel 4: the same kernel with 128-byte K steps for 16-bit inputs (64 k
// per step, four MFMA sub-steps, two 64 KiB stages at 256 x 256).
// Kernel 5: kernel 4 with split-K: K slices in the launch grid's z, fp32
// partials and an arrival counter per tile in the workspace.
// Kernel 6: kernel 2 for fp8 inputs with 64-byte K steps (one MFMA sub-step
// per step, 32 KiB stages at 256 x 256).
struct TileShape {
    int32_t id, bm, bn, wm, wn, kernel, stages;
};
constexpr int kNumTiles = 16;
constexpr TileShape kTiles[kNumTiles] = {
    {1, 64, 64, 2, 2, 1, 2},     // 4 waves, 32 x 32 per wave
    {2, 128, 128, 2, 2, 1, 2},   // 4 waves, 64 x 64 per wave
    {3, 256, 256, 2, 2, 1, 2},   // 4 waves, 128 x 128 per wave
    {4, 256, 128, 2, 2, 1, 2},   // 4 waves, 128 x 64 per wave
    {5, 256, 256, 2, 2, 2, 4},   // 4 waves, 128 x 128 per wave
    {6, 256, 256, 2, 4, 2, 4},   // 8 waves, 128 x 64 per wave
    {7, 256, 128, 2, 2, 2, 4},   // 4 waves, 128 x 64 per wave
    {8, 128, 128, 2, 2, 2, 4},   // 4 waves, 64 x 64 per wave
    {9, 256, 256, 2, 4, 3, 2},   // register-staged copies: 8 waves
    {10, 256, 256, 2, 2, 3, 2},  // register-staged copies: 4 waves
    {11, 256, 256, 2, 4, 4, 2},  // 128-byte K steps for 16-bit inputs: 8 waves
    {12, 256, 256, 2, 2, 4, 2},  // 128-byte K steps for 16-bit inputs: 4 waves
    {13, 64, 64, 2, 2, 4, 4},    // 128-byte K steps, 16-bit inputs only: 4 waves, 32 x 32 per wave
    {14, 64, 64, 2, 2, 5, 4},    // tile 13 with split-K (kernel 5): small problems with long K
    {15, 256, 128, 4, 2, 2, 4},  // 8 waves, 64 x 64 per wave (two waves per SIMD; fp8's fastest)
    {16, 256, 256, 2, 4, 6, 4},  // fp8 only: 8 waves, 128 x 64 per wave, 64-byte K steps
};

// LDS stages the pipelined kernel uses: a stage holds BM + BN rows of 64
// bytes (16-bit inputs in kernel 2; fp8 in kernel 6) or 128 bytes (fp8 in
// kernel 2, 16-bit inputs in kernels 4 and 5); at most 160 KiB in total.
constexpr int tile2_stages(const TileShape& t, int elem_size) {
    const int stage = (t.bm + t.bn) * (t.kernel == 6 ? 64 : elem_size == 1 || t.kernel >= 4 ? 128 : 64);
    return t.stages * stage <= 160 * 1024 ? t.stages : (160 * 1024) / stage;
}

// Launch one fused (or NONE-epilogue) tile-kernel GEMM.  Returns a hipError_t.
int launch_tile(int tile_id, int a_type, int d_type, int op_b, const KernelArgs& args,
                unsigned grid, void* stream);

// Launch the MX instantiation of a pipelined tile (fp8 elements with block
// scales).  Returns a hipError_t.
int launch_tile_mx(int tile_id, int d_type, int op_b, const KernelArgs& args, const MxArgs& mx,
                   unsigned grid, void* stream);

// Launch the small-m streaming kernel with rg (1, 2 or 4) groups of 16 W
// rows per wave; args.tiles_n counts column blocks of 16 * rg rows.
int launch_smallm(int a_type, int d_type, int op_b, int rg, const KernelArgs& args, unsigned grid,
                  void* stream);

// Zero n split-K arrival counters on `stream` (a kernel, graph-capturable).
int launch_clear_counters(uint32_t* p, int n, void* stream);

// Bias gradient.  launch_bgrad_sum: the unfused pair's partial sums of the
// stored D over blocks of 256 rows (COL) or columns (ROW) into args.partial
// (`parts` blocks).  launch_bgrad_reduce: sum `parts` partials per entry, in
// order, into args.bias (D's dtype); parts = 0 writes zeros.
int launch_bgrad_sum(int d_type, const KernelArgs& args, int parts, void* stream);
int launch_bgrad_reduce(int d_type, const KernelArgs& args, int parts, void* stream);

// Launch the unfused pair's elementwise kernel: D = act(C + bias) (+ mask),
// reading C (d_type, leading dimension ldd) from `c`.
int launch_elementwise(int d_type, const KernelArgs& args, const void* c, void* stream);

}  // namespace ge
