// tile_kernel.hip -- the fused GEMM + epilogue MFMA tile kernel for gfx950.
//
// D = act(s * A*B + bias) (+ ReLU sign mask), one workgroup per BM x BN tile
// of D.  The epilogue runs on the fp32 accumulators in registers right after
// the K loop, and D is written once: the fusion the pages describe (cuBLASLt
// page, paragraph 2: the bias add happens inside the matmul kernel and the
// intermediate never goes back to memory; NVGEMM page, section "What NVGEMM
// changes": matmul + bias + activation written back once).
//
// Design (gfx950 / CDNA4):
//  * K is consumed in steps of 128 bytes (BK = 32 fp32, 64 fp16/bf16, 128 fp8
//    elements).  A and B tiles are staged in LDS, two stages (double buffer),
//    with one barrier per step: the next step's global loads are issued
//    before the current step's MFMAs and written to the other stage after.
//  * LDS holds both operands "K-contiguous": one 128-byte row per M row of A
//    and per N column of B, split into eight 16-byte chunks whose order is
//    XOR-swizzled by the row so that 8 lanes reading the same chunk of 8
//    consecutive rows hit distinct banks.
//  * Global loads are 16 bytes per lane.  A (and B given n x k) are copied
//    chunk for chunk.  B given k x n (row-major, N-contiguous) is read as
//    KB x 16-byte blocks and transposed in registers before the LDS write, so
//    that MFMA operands for both A and B are 16-byte LDS reads.
//  * MFMA: 32x32x16 bf16/f16, 32x32x64 fp8 (f8f6f4, E4M3), 32x32x2 fp32.
//    Operands are swapped (src0 = B columns, src1 = A rows), so a lane's
//    accumulators hold one row of D; after a cross-half lane swap
//    (v_permlane32_swap) each lane owns 8 consecutive columns of one row and
//    stores them with one 16-byte store.  Any assignment of K values to
//    lanes is valid as long as A and B use the same one; the chunk order
//    below is chosen so that each lane's LDS reads are whole chunks.
//  * The aux mask: 8 bits per lane per 8 columns, combined across the two
//    lane halves into one 32-bit word per row of a 32 x 32 block.
//  * Launch order is XCD-aware: consecutive workgroup ids land on different
//    XCDs (round-robin), so ids are remapped to give each XCD a contiguous
//    range of tiles, traversed in groups of `group_m` tile-rows for L2 reuse.
#pragma once
#include "ge_device.h"

namespace ge {

constexpr int kRowBytes = 128;

__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ lds_swz(row)) << 4);
}

template <int DIN, int DOUT, int OPB, int BM, int BN, int WM, int WN>
struct TileCfg {
    static constexpr int ESZ = Elem<DIN>::size;
    static constexpr int BK = kRowBytes / ESZ;   // K elements per step
    static constexpr int E = 16 / ESZ;           // elements per 16-byte chunk
    static constexpr int NT = WM * WN * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int A_CHUNKS = BM * 8;
    static constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT;
    static constexpr int BT_CHUNKS = BN * 8;
    static constexpr int BT_PER_T = (BT_CHUNKS + NT - 1) / NT;
    // B given k x n: blocks of KB k-rows x one 16-byte chunk (E n-values)
    static constexpr int KB = (ESZ == 4) ? 4 : 8;
    static constexpr int KBLK = BK / KB;
    static constexpr int NBLK = BN / E;
    static constexpr int BN_BLOCKS = KBLK * NBLK;
    static constexpr int BN_PER_T = (BN_BLOCKS + NT - 1) / NT;
    static constexpr int B_REGS = OPB == GE_OP_T ? BT_PER_T : BN_PER_T * KB;
    static constexpr int STAGE = (BM + BN) * kRowBytes;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
};

// 16-byte chunk at element (row, col) of a row-major matrix with `ld`
// elements per row, of which `ncols` are valid (col a multiple of 16/ESZ,
// nrows and ncols >= 1); elements of rows >= nrows or columns >= ncols read
// as zero.  No per-lane branch: the load always reads a chunk that holds a
// valid element (the row clamped to the last, the chunk to the last one
// with valid columns), so its 16-byte-aligned bytes lie on a mapped page
// even where the matrix ends mid-row, and the invalid elements are masked
// off afterwards.  (Divergent branches here made the register allocator
// spill and reload values for the active lanes only.)
template <int ESZ>
__device__ __forceinline__ u32x4 load_chunk(const uint8_t* base, int64_t ld, int row, int nrows,
                                            int col, int ncols) {
    constexpr int E = 16 / ESZ;
    const int rr = max(min(row, nrows - 1), 0);
    const int cc = min(col, max((ncols - 1) / E * E, 0));
    u32x4 v = *(const u32x4*)(base + ((int64_t)rr * ld + cc) * ESZ);
    const int nb = (row < nrows ? min(max(ncols - col, 0), E) : 0) * ESZ;   // valid bytes
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int b = min(max(nb - 4 * d, 0), 4);
        v[d] &= b >= 4 ? 0xffffffffu : ((1u << (8 * b)) - 1u);
    }
    return v;
}

template <int DIN, int DOUT, int OPB, int BM, int BN, int WM, int WN>
__device__ __forceinline__ void tile_coords(const KernelArgs& p, int& tm, int& tn) {
    int b = blockIdx.x;
    const int T = p.tiles_m * p.tiles_n;
    int lin = b;
    if ((T & 7) == 0) lin = (b & 7) * (T >> 3) + (b >> 3);   // contiguous range per XCD
    const int per_group = p.group_m * p.tiles_n;
    const int g = lin / per_group;
    const int first = g * p.group_m;
    const int gm = min(p.tiles_m - first, p.group_m);
    const int r = lin - g * per_group;
    tm = first + r % gm;
    tn = r / gm;
}

template <int DIN, int DOUT, int OPB, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(WM* WN * 64)
ge_tile_kernel(KernelArgs p_all) {
    const KernelArgs p = batch_slice(p_all, blockIdx.y);   // this product of a batch
    using C = TileCfg<DIN, DOUT, OPB, BM, BN, WM, WN>;
    constexpr int ESZ = C::ESZ, BK = C::BK, E = C::E, NT = C::NT;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

    int tm, tn;
    tile_coords<DIN, DOUT, OPB, BM, BN, WM, WN>(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.m, N = p.n, K = p.k;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int r32 = lane & 31, h = lane >> 5;
    const uint8_t* gA = (const uint8_t*)p.A;
    const uint8_t* gB = (const uint8_t*)p.B;

    u32x4 ra[C::A_PER_T];
    u32x4 rb[C::B_REGS];

    // ---- global -> registers for K step starting at k0 ----
    auto load_regs = [&](int k0) {
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i) {
            const int c = tid + i * NT;
            const int row = c >> 3, ch = c & 7;
            if (C::A_CHUNKS % NT == 0 || c < C::A_CHUNKS)
                ra[i] = load_chunk<ESZ>(gA, p.lda, m0 + row, M, k0 + ch * E, K);
        }
        if constexpr (OPB == GE_OP_T) {
#pragma unroll
            for (int i = 0; i < C::BT_PER_T; ++i) {
                const int c = tid + i * NT;
                const int row = c >> 3, ch = c & 7;
                if (C::BT_CHUNKS % NT == 0 || c < C::BT_CHUNKS)
                    rb[i] = load_chunk<ESZ>(gB, p.ldb, n0 + row, N, k0 + ch * E, K);
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::BN_PER_T; ++i) {
                const int bid = tid + i * NT;
                const int kb = bid % C::KBLK, nb = bid / C::KBLK;
                if (C::BN_BLOCKS % NT == 0 || bid < C::BN_BLOCKS) {
#pragma unroll
                    for (int r = 0; r < C::KB; ++r)
                        rb[i * C::KB + r] =
                            load_chunk<ESZ>(gB, p.ldb, k0 + kb * C::KB + r, K, n0 + nb * E, N);
                }
            }
        }
    };

    // ---- registers -> LDS stage ----
    auto store_lds = [&](int stage) {
        uint8_t* sA = smem + stage * C::STAGE;
        uint8_t* sB = sA + BM * kRowBytes;
#pragma unroll
        for (int i = 0; i < C::A_PER_T; ++i) {
            const int c = tid + i * NT;
            if (C::A_CHUNKS % NT == 0 || c < C::A_CHUNKS)
                *(u32x4*)(sA + lds_off(c >> 3, c & 7)) = ra[i];
        }
        if constexpr (OPB == GE_OP_T) {
#pragma unroll
            for (int i = 0; i < C::BT_PER_T; ++i) {
                const int c = tid + i * NT;
                if (C::BT_CHUNKS % NT == 0 || c < C::BT_CHUNKS)
                    *(u32x4*)(sB + lds_off(c >> 3, c & 7)) = rb[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::BN_PER_T; ++i) {
                const int bid = tid + i * NT;
                const int kb = bid % C::KBLK, nb = bid / C::KBLK;
                if (!(C::BN_BLOCKS % NT == 0 || bid < C::BN_BLOCKS)) continue;
                const u32x4* v = rb + i * C::KB;
                if constexpr (ESZ == 2) {
                    // 8 k-rows x 8 n-values -> 8 n-rows of 8 k-values
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        u32x4 o;
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t lo = v[2 * j][c >> 1], hi = v[2 * j + 1][c >> 1];
                            o[j] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                           : ((lo & 0xffffu) | (hi << 16));
                        }
                        *(u32x4*)(sB + lds_off(nb * 8 + c, kb)) = o;
                    }
                } else if constexpr (ESZ == 4) {
                    // 4 k-rows x 4 n-values
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        u32x4 o = {v[0][c], v[1][c], v[2][c], v[3][c]};
                        *(u32x4*)(sB + lds_off(nb * 4 + c, kb)) = o;
                    }
                } else {
                    // fp8: 8 k-rows x 16 n-values -> 16 n-rows of 8 bytes
#pragma unroll
                    for (int c = 0; c < 16; ++c) {
                        u32x2 o;
#pragma unroll
                        for (int j = 0; j < 2; ++j) {
                            uint32_t w = 0;
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                w |= ((v[4 * j + t][c >> 2] >> (8 * (c & 3))) & 0xffu) << (8 * t);
                            o[j] = w;
                        }
                        *(u32x2*)(sB + lds_off(nb * 16 + c, kb >> 1) + ((kb & 1) << 3)) = o;
                    }
                }
            }
        }
    };

    f32x16 acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};

    // per-lane LDS row offsets of this wave's fragments
    int rowA[C::FM], rowB[C::FN];
#pragma unroll
    for (int f = 0; f < C::FM; ++f) rowA[f] = wm * C::TM + f * 32 + r32;
#pragma unroll
    for (int f = 0; f < C::FN; ++f) rowB[f] = wn * C::TN + f * 32 + r32;

    auto compute = [&](int stage) {
        const uint8_t* sA = smem + stage * C::STAGE;
        const uint8_t* sB = sA + BM * kRowBytes;
        if constexpr (ESZ == 1) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                i32x8 af[C::FM], bfr[C::FN];
#pragma unroll
                for (int f = 0; f < C::FM; ++f) {
                    const u32x4 lo = *(const u32x4*)(sA + lds_off(rowA[f], h + 4 * kk));
                    const u32x4 hi = *(const u32x4*)(sA + lds_off(rowA[f], h + 4 * kk + 2));
                    af[f] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
#pragma unroll
                for (int f = 0; f < C::FN; ++f) {
                    const u32x4 lo = *(const u32x4*)(sB + lds_off(rowB[f], h + 4 * kk));
                    const u32x4 hi = *(const u32x4*)(sB + lds_off(rowB[f], h + 4 * kk + 2));
                    bfr[f] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int j = 0; j < C::FM; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            bfr[i], af[j], acc[i][j], 0, 0, 0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                u32x4 af[C::FM], bfr[C::FN];
#pragma unroll
                for (int f = 0; f < C::FM; ++f) af[f] = *(const u32x4*)(sA + lds_off(rowA[f], h + 2 * kk));
#pragma unroll
                for (int f = 0; f < C::FN; ++f) bfr[f] = *(const u32x4*)(sB + lds_off(rowB[f], h + 2 * kk));
                if constexpr (ESZ == 2) {
#pragma unroll
                    for (int i = 0; i < C::FN; ++i)
#pragma unroll
                        for (int j = 0; j < C::FM; ++j) {
                            if constexpr (DIN == GE_BF16)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    __builtin_bit_cast(bf16x8, bfr[i]), __builtin_bit_cast(bf16x8, af[j]),
                                    acc[i][j], 0, 0, 0);
                            else
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                    __builtin_bit_cast(f16x8, bfr[i]), __builtin_bit_cast(f16x8, af[j]),
                                    acc[i][j], 0, 0, 0);
                        }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int i = 0; i < C::FN; ++i)
#pragma unroll
                            for (int j = 0; j < C::FM; ++j)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                    __uint_as_float(bfr[i][e]), __uint_as_float(af[j][e]), acc[i][j], 0, 0, 0);
                }
            }
        }
    };

    // ---- main loop: double-buffered LDS, one barrier per K step ----
    const int KT = (K + BK - 1) / BK;
    load_regs(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) load_regs((kt + 1) * BK);
        compute(cur);
        if (more) store_lds(cur ^ 1);
        __syncthreads();
    }

    // ---- fused epilogue on the accumulators ----
    // the product's scale: fp8 dequantisation factors, or an alpha for any dtype
    float s = 1.0f;
    if (p.scale_a) s *= *p.scale_a;
    if (p.scale_b) s *= *p.scale_b;
    const int ep = p.epilog;
    const bool has_bias = epilog_has_bias(ep);
    const bool row_bias = p.axis == GE_BIAS_ROW;
    const bool want_aux = ep == GE_EPILOG_RELU_AUX_BIAS;
    const bool want_pre = ep == GE_EPILOG_GELU_AUX_BIAS;                    // aux <- P
    const bool want_grad = epilog_is_grad(ep);                              // D = C * f(aux)
    const bool want_bgrad = epilog_is_bgrad(ep);                            // + bias gradient
    // + beta * C; with beta = 0 C is not read (so it may hold anything)
    const float beta = p.cin ? *p.beta : 0.0f;
    const bool with_c = p.cin != nullptr && beta != 0.0f;
    const bool bgrad_col = p.axis == GE_BIAS_COL;
    BgradAcc<C::FM, C::FN> bg;
    bg.clear();

#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
        const int m = m0 + wm * C::TM + fm * 32 + r32;
        const bool mok = m < M;
        float brow = 0.0f;
        if (has_bias && row_bias && mok) brow = load_scalar<DOUT>(p.bias, m);
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
            const int nb = n0 + wn * C::TN + fn * 32;
            const f32x16 a = acc[fn][fm];
            // lane half h holds columns nb + 8G + 4h + e of row m in a[4G + e];
            // swap halves so that lane half h holds nb + 16g + 8h + j, j = 0..7
            float v[2][8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[8 * g + e]),
                                                               __float_as_uint(a[8 * g + 4 + e]), false, false);
                    v[g][e] = __uint_as_float(sw[0]);
                    v[g][4 + e] = __uint_as_float(sw[1]);
                }
            }
            uint32_t bits = 0;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int nc = nb + 16 * g + 8 * h;
                const bool full = nc + 8 <= N;
                float bc[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) bc[j] = brow;
                if (has_bias && !row_bias) {
                    if (full) load8<DOUT>(p.bias, nc, bc);
                    else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) bc[j] = (nc + j < N) ? load_scalar<DOUT>(p.bias, nc + j) : 0.0f;
                    }
                }
                float gf[8], pre[8], cb[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) cb[j] = 0.0f;
                if (with_c && mok) beta_c8<DOUT>(p, beta, m, nc, cb);
                if (want_grad) {
                    if (mok) grad_factor8<DOUT>(p, ep, m, nc, gf);
                    else {
#pragma unroll
                        for (int j = 0; j < 8; ++j) gf[j] = 0.0f;
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float x = (v[g][j] * s + cb[j]) + bc[j];
                    pre[j] = x;
                    if (want_aux && x > 0.0f && nc + j < N) bits |= 1u << (16 * g + 8 * h + j);
                    v[g][j] = want_grad ? grad_apply(ep, x, gf[j]) : activate(ep, x);
                }
                if (want_bgrad) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float val = (mok && nc + j < N) ? v[g][j] : 0.0f;
                        if (bgrad_col) bg.col[fn][g][j] += val;
                        else bg.row[fm] += val;
                    }
                }
                if (mok) {
                    const int64_t idx = (int64_t)m * p.ldd + nc;
                    if (full) store8<DOUT>(p.D, idx, v[g]);
                    else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (nc + j < N) store_one<DOUT>(p.D, idx + j, v[g][j]);
                    }
                    if (want_pre) store_pre8<DOUT>(p, m, nc, pre);
                }
            }
            if (want_aux) {
                bits |= (uint32_t)__shfl_xor((int)bits, 32);
                if (h == 0 && mok && (nb >> 5) < p.ldaux) p.aux[(int64_t)m * p.ldaux + (nb >> 5)] = bits;
            }
        }
    }
    // mask padding words that no tile covers (row stride rounded up to 128 bits)
    if (want_bgrad)
        bgrad_tile<BM, BN, WM, WN, C::FM, C::FN>(p, bg, (float*)smem, tm, tn, wm, wn, lane, tid, NT);
    if (want_aux && tn == p.tiles_n - 1) {
        const int w0 = (p.tiles_n * BN) >> 5;
        const int nw = p.ldaux - w0;
        if (nw > 0) {
            for (int idx = tid; idx < BM * nw; idx += NT) {
                const int row = m0 + idx / nw;
                if (row < M) p.aux[(int64_t)row * p.ldaux + w0 + idx % nw] = 0u;
            }
        }
    }
}

typedef void (*TileFn)(KernelArgs);

template <int DIN, int DOUT, int OPB>
TileFn pick_tile(int tile_id) {
    switch (tile_id) {
    case 1: return ge_tile_kernel<DIN, DOUT, OPB, 64, 64, 2, 2>;
    case 2: return ge_tile_kernel<DIN, DOUT, OPB, 128, 128, 2, 2>;
    case 3: return ge_tile_kernel<DIN, DOUT, OPB, 256, 256, 2, 2>;
    case 4: return ge_tile_kernel<DIN, DOUT, OPB, 256, 128, 2, 2>;
    }
    return nullptr;
}

template <int DIN, int DOUT>
TileFn pick_op(int op_b, int tile_id) {
    return op_b == GE_OP_T ? pick_tile<DIN, DOUT, GE_OP_T>(tile_id) : pick_tile<DIN, DOUT, GE_OP_N>(tile_id);
}

// per-input-dtype tables, each compiled in its own translation unit
TileFn pick_tile_f32(int d_type, int op_b, int tile_id);
TileFn pick_tile_f16(int d_type, int op_b, int tile_id);
TileFn pick_tile_bf16(int d_type, int op_b, int tile_id);
TileFn pick_tile_f8(int d_type, int op_b, int tile_id);
// the pipelined kernels take the MX block-scale arguments besides (unused
// and zero unless the instantiation is a block-scaled one)
typedef void (*Tile2Fn)(KernelArgs, MxArgs);
Tile2Fn pick_tile2_f16_f16(int op_b, int tile_id);
Tile2Fn pick_tile2_f16_f32(int op_b, int tile_id);
Tile2Fn pick_tile2_bf16_bf16(int op_b, int tile_id);
Tile2Fn pick_tile2_bf16_f32(int op_b, int tile_id);
Tile2Fn pick_tile2_f8_bf16(int op_b, int tile_id);
Tile2Fn pick_tile2_f8_f16(int op_b, int tile_id);
Tile2Fn pick_tile2_f8_f32(int op_b, int tile_id);
Tile2Fn pick_tile2_mx_f8_bf16(int op_b, int tile_id);
Tile2Fn pick_tile2_mx_f8_f16(int op_b, int tile_id);
Tile2Fn pick_tile2_mx_f8_f32(int op_b, int tile_id);
Tile2Fn pick_tile2_bf16_f8(int op_b, int tile_id);   // fp8 (E4M3) output
Tile2Fn pick_tile2_f16_f8(int op_b, int tile_id);
Tile2Fn pick_tile2_f8_f8(int op_b, int tile_id);
Tile2Fn pick_tile2_mx_f8_f8(int op_b, int tile_id);

}  // namespace ge
