// tile2_kernel.h -- the pipelined fused GEMM + epilogue tile kernel for
// 16-bit inputs (fp16, bf16) on gfx950.
//
// Computes the same thing as the baseline tile kernel (tile_kernel.h):
// D = act(A*B + bias) (+ ReLU sign mask), one workgroup per BM x BN tile,
// the epilogue applied to the fp32 accumulators in registers and D written
// once (cuBLASLt page, paragraph 2; NVGEMM page, section "What NVGEMM
// changes").  What differs is how A and B reach the matrix cores:
//
//  * K is consumed 32 elements (64 bytes of a row) per step, through S LDS
//    stages.  Full steps are copied global -> LDS by the direct-to-LDS loads
//    of gfx950 (global_load_lds_dwordx4: each lane's 16 bytes land at
//    M0 + 16*lane), so the copy costs no VGPRs and no VALU, and S-1 steps are
//    in flight while the matrix cores work on the current one.  A wave waits
//    for its own copies with s_waitcnt vmcnt(n) and the workgroup meets at a
//    plain s_barrier (no memory fence, which would drain every copy).
//  * Since the LDS address of a lane is fixed by the lane id, the layout is
//    chosen on the global side: lane (row R, slot s) fetches chunk
//    s ^ g(R) of its row, which XOR-swizzles the 16-byte chunks of each LDS
//    row so that the fragment reads below hit distinct banks.
//  * A (m x k) and B given n x k are stored one 64-byte row per M (N) index
//    and read as 16-byte k-runs (ds_read_b128).  B given k x n keeps its
//    natural [k][n] layout in LDS and is read with the transposing LDS load
//    of gfx950 (ds_read_b64_tr_b16): in each 16-lane group, lanes 4r..4r+3
//    address the four 8-byte pieces of row r of a 4 x 16 block and lane i
//    receives column i, i.e. 4 consecutive k values of one n.  No transpose
//    in registers.
//  * Tails: rows of A beyond m and columns of B beyond n only feed outputs
//    that are never stored, so their addresses are clamped to the last valid
//    row / 16-byte chunk (memory safety only).  A ragged last K step is
//    loaded through registers with the elements beyond k zeroed (in both A
//    and B, since 0 * NaN would not vanish) and written to the same LDS
//    positions.
//  * MFMA 32x32x16 with swapped operands and the epilogue exactly as in
//    tile_kernel.h: after a lane-half swap each lane owns 8 consecutive
//    columns of one row of D and stores them with one 16-byte store.
#pragma once
#include "tile_kernel.h"

namespace ge {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row (A and B given
// n x k): lanes reading the same chunk of 8 or 16 consecutive rows hit
// distinct banks (64-byte rows repeat the bank pattern every 2 or 4 rows).
__device__ __forceinline__ int swz64(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// XOR swizzle of the chunks of a [k][n] LDS row (B given k x n), indexed by
// k mod 4: the transposing reads of four consecutive k rows then cover
// distinct banks whether a pass serves 16 or 32 lanes.
__device__ __forceinline__ int swz_kn(int k) {
    constexpr int t = (0 << 0) | (4 << 5) | (10 << 10) | (14 << 15);
    return (t >> (5 * (k & 3))) & 31;
}

// One direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// LDS byte address lds + 16*l (lds must be the same for the whole wave; it
// goes to M0, and one wait state separates the M0 write from its use).
// Written as inline assembly on purpose: the compiler's wait-count pass
// would otherwise make every later LDS read wait for all copies in flight,
// which defeats the pipeline.  Completion is tracked by hand instead
// (wait_vm + barrier).  The compiler's own vmcnt waits for ordinary loads
// stay correct: copies it does not count only make them wait longer.
__device__ __forceinline__ void copy_to_lds16(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

// Wait until at most n of this wave's vector-memory operations are
// outstanding (the other counters are left alone).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int DIN, int DOUT, int OPB, int BM, int BN, int WM, int WN, int S>
struct Tile2Cfg {
    static constexpr int NW = WM * WN, NT = NW * 64;
    static constexpr int BK = 32;                    // elements per K step
    static constexpr int ROWB = 64;                  // bytes per LDS row (A, B n x k)
    static constexpr int A_BYTES = BM * ROWB;
    static constexpr int B_BYTES = BK * BN * 2;      // same for both B layouts
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int A_INS = A_BYTES / 1024 / NW;   // 1 KiB copies per wave per step
    static constexpr int B_INS = B_BYTES / 1024 / NW;
    static constexpr int VM_PER_STEP = A_INS + B_INS;
    static constexpr int KN_ROWB = BN * 2;           // bytes per [k][n] LDS row
    static constexpr int KN_CPR = BN / 8;            // 16-byte chunks per [k][n] row
    static constexpr int KN_RPI = 1024 / KN_ROWB;    // [k][n] rows per 1 KiB copy
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static_assert(DIN == GE_F16 || DIN == GE_BF16, "16-bit inputs only");
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole copies per wave");
    static_assert(KN_CPR >= 16 && KN_ROWB <= 1024, "[k][n] swizzle needs 16..64 chunks per row");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(S >= 2 && S * STAGE <= 160 * 1024, "LDS budget");
    static_assert((S - 2) * VM_PER_STEP < 64, "vmcnt range");
};

template <int DIN, int DOUT, int OPB, int BM, int BN, int WM, int WN, int S>
__global__ void __launch_bounds__(WM* WN * 64)
ge_tile2_kernel(KernelArgs p) {
    using C = Tile2Cfg<DIN, DOUT, OPB, BM, BN, WM, WN, S>;
    constexpr int BK = C::BK;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S * C::STAGE];

    int tm, tn;
    tile_coords<DIN, DOUT, OPB, BM, BN, WM, WN>(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.m, N = p.n, K = p.k;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int wm = wave % WM, wn = wave / WM;
    const int r32 = lane & 31, h = lane >> 5;
    const uint8_t* gA = (const uint8_t*)p.A;
    const uint8_t* gB = (const uint8_t*)p.B;
    const int KT = (K + BK - 1) / BK;       // K steps
    const int KF = K / BK;                  // full K steps (direct copies)

    // ---- per-lane sources of this wave's 1 KiB copies, at K step 0 ----
    // A: copy i covers LDS rows R = (wave*A_INS + i)*16 + lane/4, slot lane%4
    const uint8_t* srcA[C::A_INS];
    int rowA_cp[C::A_INS], chA_cp[C::A_INS];
#pragma unroll
    for (int i = 0; i < C::A_INS; ++i) {
        const int R = (wave * C::A_INS + i) * 16 + (lane >> 2);
        const int c = (lane & 3) ^ swz64(R);
        const int gm = min(m0 + R, max(M - 1, 0));
        rowA_cp[i] = m0 + R;
        chA_cp[i] = c;
        srcA[i] = gA + ((int64_t)gm * p.lda + c * 8) * 2;
    }
    const uint8_t* srcB[C::B_INS];
    int rowB_cp[C::B_INS], chB_cp[C::B_INS];
    const int nlast = N > 0 ? ((N - 1) / 8) * 8 : 0;   // start of the last chunk holding valid columns
#pragma unroll
    for (int i = 0; i < C::B_INS; ++i) {
        if constexpr (OPB == GE_OP_T) {
            const int R = (wave * C::B_INS + i) * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz64(R);
            const int gn = min(n0 + R, max(N - 1, 0));
            rowB_cp[i] = n0 + R;
            chB_cp[i] = c;
            srcB[i] = gB + ((int64_t)gn * p.ldb + c * 8) * 2;
        } else {
            const int kr = (wave * C::B_INS + i) * C::KN_RPI + lane / C::KN_CPR;
            const int c = (lane % C::KN_CPR) ^ swz_kn(kr);
            const int gn = min(n0 + c * 8, nlast);
            rowB_cp[i] = kr;
            chB_cp[i] = n0 + c * 8;
            srcB[i] = gB + ((int64_t)kr * p.ldb + gn) * 2;
        }
    }
    const int64_t stepB = (OPB == GE_OP_T) ? (int64_t)BK * 2 : (int64_t)BK * p.ldb * 2;

    // issue the direct copies of full K step t into stage t % S
    auto issue_direct = [&](int t) {
        uint8_t* st = smem + (t % S) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::A_INS; ++i)
            copy_to_lds16(srcA[i] + (int64_t)t * BK * 2, lds_addr(st + (wave * C::A_INS + i) * 1024));
#pragma unroll
        for (int i = 0; i < C::B_INS; ++i)
            copy_to_lds16(srcB[i] + (int64_t)t * stepB, lds_addr(st + C::A_BYTES + (wave * C::B_INS + i) * 1024));
    };

    // the ragged last K step t: through registers, elements at k >= K zeroed
    auto issue_tail = [&](int t) {
        uint8_t* st = smem + (t % S) * C::STAGE;
        const int k0 = t * BK;
        u32x4 va[C::A_INS], vb[C::B_INS];
#pragma unroll
        for (int i = 0; i < C::A_INS; ++i)
            va[i] = load_chunk<2>(gA, p.lda, min(rowA_cp[i], max(M - 1, 0)), M, k0 + chA_cp[i] * 8, K);
#pragma unroll
        for (int i = 0; i < C::B_INS; ++i) {
            if constexpr (OPB == GE_OP_T)
                vb[i] = load_chunk<2>(gB, p.ldb, min(rowB_cp[i], max(N - 1, 0)), N, k0 + chB_cp[i] * 8, K);
            else
                vb[i] = load_chunk<2>(gB, p.ldb, k0 + rowB_cp[i], K, min(chB_cp[i], nlast), N);
        }
#pragma unroll
        for (int i = 0; i < C::A_INS; ++i) *(u32x4*)(st + (wave * C::A_INS + i) * 1024 + lane * 16) = va[i];
#pragma unroll
        for (int i = 0; i < C::B_INS; ++i)
            *(u32x4*)(st + C::A_BYTES + (wave * C::B_INS + i) * 1024 + lane * 16) = vb[i];
    };

    auto issue = [&](int t) {
        if (t < KF) issue_direct(t);
        else issue_tail(t);
    };

    f32x16 acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};

    // per-lane LDS read offsets within a stage
    int offA[C::FM][2];
#pragma unroll
    for (int f = 0; f < C::FM; ++f) {
        const int row = wm * C::TM + f * 32 + r32;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) offA[f][kk] = row * C::ROWB + (((2 * kk + h) ^ swz64(row)) << 4);
    }
    // B given n x k: as A.  B given k x n: two transposing reads per fragment
    // and k16 sub-step; lane (group G, i): k = 16kk + 8(G/2) + 4*half + i/4,
    // n = wave col + 32f + 16(G%2) + 4(i%4).
    int offB[C::FN][2][2];
#pragma unroll
    for (int f = 0; f < C::FN; ++f) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                if constexpr (OPB == GE_OP_T) {
                    const int row = wn * C::TN + f * 32 + r32;
                    offB[f][kk][hf] = C::A_BYTES + row * C::ROWB + (((2 * kk + h) ^ swz64(row)) << 4);
                } else {
                    const int G = lane >> 4, i = lane & 15;
                    const int k = 16 * kk + 8 * (G >> 1) + 4 * hf + (i >> 2);
                    const int n = wn * C::TN + f * 32 + 16 * (G & 1) + 4 * (i & 3);
                    offB[f][kk][hf] =
                        C::A_BYTES + k * C::KN_ROWB + (((n >> 3) ^ swz_kn(k)) << 4) + ((n & 4) << 1);
                }
            }
        }
    }

    // fragments of one k16 sub-step (kk) of the step held in `stage`
    auto load_frags = [&](int stage, int kk, u32x4 (&af)[C::FM], u32x4 (&bfr)[C::FN]) {
        const uint8_t* st = smem + stage * C::STAGE;
#pragma unroll
        for (int f = 0; f < C::FN; ++f) {
            if constexpr (OPB == GE_OP_T) {
                bfr[f] = *(const u32x4*)(st + offB[f][kk][0]);
            } else {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_t*)((lds_void_t*)(st + offB[f][kk][0])));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_t*)((lds_void_t*)(st + offB[f][kk][1])));
                bfr[f] = u32x4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                               (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                               (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                               (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
            }
        }
#pragma unroll
        for (int f = 0; f < C::FM; ++f) af[f] = *(const u32x4*)(st + offA[f][kk]);
    };
    auto mfmas = [&](const u32x4 (&af)[C::FM], const u32x4 (&bfr)[C::FN]) {
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
            for (int j = 0; j < C::FM; ++j) {
                if constexpr (DIN == GE_BF16)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, bfr[i]), __builtin_bit_cast(bf16x8, af[j]), acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(f16x8, bfr[i]), __builtin_bit_cast(f16x8, af[j]), acc[i][j], 0, 0, 0);
            }
    };
    // Wait until this wave's copies of step t are done, given that the
    // copies of steps t+1 .. last_issued were issued after them.
    auto wait_step = [&](int later) {
        static_assert(S <= 5, "wait ladder covers up to 4 later steps");
        if (later >= 4) wait_vm<(4 * C::VM_PER_STEP < 64 ? 4 * C::VM_PER_STEP : 63)>();
        else if (later == 3) wait_vm<(3 * C::VM_PER_STEP < 64 ? 3 * C::VM_PER_STEP : 63)>();
        else if (later == 2) wait_vm<2 * C::VM_PER_STEP>();
        else if (later == 1) wait_vm<C::VM_PER_STEP>();
        else wait_vm<0>();
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): own LDS reads and tail writes done
        // workgroup barrier without a memory fence (a fence would wait for
        // every copy in flight); the clobber keeps LDS accesses on their side
        asm volatile("s_barrier" ::: "memory");
    };

    // ---- main loop ----
    // All S stages start filling at once; afterwards the copy of step
    // kt + S goes into the stage step kt used, as soon as every wave has
    // read its last fragments from it.  The barrier sits between the two
    // k16 halves of a step, so the first fragments of step kt + 1 are read
    // while the matrix cores still work on step kt.
#pragma unroll
    for (int t = 0; t < S; ++t)
        if (t < KT) issue(t);
    u32x4 a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
    if (KT > 0) {
        wait_step(min(S - 1, KT - 1));
        load_frags(0, 0, a0, b0);
    }
    // (the last step is peeled off so that the loop body always passes the
    // barrier: a merged path would make the compiler's wait analysis hold
    // the second-half MFMAs until the next step's fragment reads return)
    for (int kt = 0; kt < KT - 1; ++kt) {
        // each group of fragment reads is issued ahead of the MFMAs that do
        // not need it (the scheduler would otherwise sink the last reads to
        // the end of the block and stall the next MFMAs on them)
        load_frags(kt % S, 1, a1, b1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(a0, b0);
        wait_step(min(S - 2, KT - 2 - kt));
        if (kt + S < KT) issue(kt + S);
        load_frags((kt + 1) % S, 0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(a1, b1);
    }
    if (KT > 0) {
        load_frags((KT - 1) % S, 1, a1, b1);
        mfmas(a0, b0);
        mfmas(a1, b1);
    }

    // ---- fused epilogue on the accumulators (as in tile_kernel.h) ----
    const int ep = p.epilog;
    const bool has_bias = ep != GE_EPILOG_NONE;
    const bool row_bias = p.axis == GE_BIAS_ROW;
    const bool want_aux = ep == GE_EPILOG_RELU_AUX_BIAS;

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
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float x = v[g][j] + bc[j];
                    if (want_aux && x > 0.0f && nc + j < N) bits |= 1u << (16 * g + 8 * h + j);
                    v[g][j] = activate(ep, x);
                }
                if (mok) {
                    const int64_t idx = (int64_t)m * p.ldd + nc;
                    if (full) store8<DOUT>(p.D, idx, v[g]);
                    else {
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            if (nc + j < N) store_one<DOUT>(p.D, idx + j, v[g][j]);
                    }
                }
            }
            if (want_aux) {
                bits |= (uint32_t)__shfl_xor((int)bits, 32);
                if (h == 0 && mok && (nb >> 5) < p.ldaux) p.aux[(int64_t)m * p.ldaux + (nb >> 5)] = bits;
            }
        }
    }
    if (want_aux && tn == p.tiles_n - 1) {
        const int w0 = (p.tiles_n * BN) >> 5;
        const int nw = p.ldaux - w0;
        if (nw > 0) {
            for (int idx = tid; idx < BM * nw; idx += C::NT) {
                const int row = m0 + idx / nw;
                if (row < M) p.aux[(int64_t)row * p.ldaux + w0 + idx % nw] = 0u;
            }
        }
    }
}

template <int DIN, int DOUT, int OPB>
TileFn pick_tile2(int tile_id) {
    switch (tile_id) {
    case 5: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 256, 2, 2, 4>;
    case 6: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 256, 2, 4, 4>;
    case 7: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 128, 2, 2, 4>;
    case 8: return ge_tile2_kernel<DIN, DOUT, OPB, 128, 128, 2, 2, 4>;
    }
    return nullptr;
}

template <int DIN, int DOUT>
TileFn pick_op2(int op_b, int tile_id) {
    return op_b == GE_OP_T ? pick_tile2<DIN, DOUT, GE_OP_T>(tile_id) : pick_tile2<DIN, DOUT, GE_OP_N>(tile_id);
}

}  // namespace ge
