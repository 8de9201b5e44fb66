// tile2_kernel.h -- the pipelined fused GEMM + epilogue tile kernel for
// 16-bit (fp16, bf16) and 8-bit (OCP E4M3) inputs on gfx950.
//
// Computes the same thing as the baseline tile kernel (tile_kernel.h):
// D = act(A*B + bias) (+ ReLU sign mask), one workgroup per BM x BN tile,
// the epilogue applied to the fp32 accumulators in registers and D written
// once (cuBLASLt page, paragraph 2; NVGEMM page, section "What NVGEMM
// changes").  What differs is how A and B reach the matrix cores:
//
//  * K is consumed 64 bytes of a row per step for 16-bit inputs (32
//    elements) and 128 bytes for fp8 (128 elements), through as many LDS
//    stages as fit (up to S).  Full steps are copied global -> LDS by the direct-to-LDS loads
//    of gfx950 (global_load_lds_dwordx4: each lane's 16 bytes land at
//    M0 + 16*lane), so the copy costs no VGPRs and no VALU, and S-1 steps are
//    in flight while the matrix cores work on the current one.  A wave waits
//    for its own copies with s_waitcnt vmcnt(n) and the workgroup meets at a
//    plain s_barrier (no memory fence, which would drain every copy).
//  * LDS holds the A stages first, then the B stages, so consecutive stages
//    of one operand are A_BYTES (or B_BYTES) apart -- 32 KiB at 256 x 256 --
//    within the 16-bit immediate offset of the LDS reads; the main loop takes
//    one step per stage per iteration, so each stage's base becomes such an
//    immediate instead of a per-read address add.
//  * Since the LDS address of a lane is fixed by the lane id, the layout is
//    chosen on the global side: lane (row R, slot s) fetches chunk
//    s ^ g(R) of its row, which XOR-swizzles the 16-byte chunks of each LDS
//    row so that the fragment reads below hit distinct banks.
//  * A (m x k) and B given n x k are stored one 64-byte row per M (N) index
//    and read as 16-byte k-runs (ds_read_b128).  B given k x n keeps its
//    natural [k][n] layout in LDS and is read with the transposing LDS load
//    of gfx950 (ds_read_b64_tr_b16): in each 16-lane group, lanes 4r..4r+3
//    address the four 8-byte pieces of row r of a 4 x 16 block and lane i
//    receives column i, i.e. 4 consecutive k values of one n.  For fp8 the
//    byte form (ds_read_b64_tr_b8) does the same on an 8 x 16-byte block:
//    lanes 2r, 2r+1 address the halves of row r, lane i receives 8
//    consecutive k values of column i.  No transpose in registers.
//  * Tails: rows of A beyond m and columns of B beyond n only feed outputs
//    that are never stored, so their addresses are clamped to the last valid
//    row / 16-byte chunk (memory safety only).  A ragged last K step is
//    loaded through registers with the elements beyond k zeroed (in both A
//    and B, since 0 * NaN would not vanish) and written to the same LDS
//    positions.
//  * MFMA 32x32x16 (16-bit) or 32x32x64 (fp8, per-tensor scales applied to
//    the accumulator) with swapped operands and the epilogue exactly as in
//    tile_kernel.h: after a lane-half swap each lane owns 8 consecutive
//    columns of one row of D and stores them with one 16-byte store.
#pragma once
#include <type_traits>

#include "tile_kernel.h"

namespace ge {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

// XOR swizzle of the four 16-byte chunks of a 64-byte LDS row (A and B given
// n x k): lanes reading the same chunk of 8 or 16 consecutive rows hit
// distinct banks (64-byte rows repeat the bank pattern every 2 or 4 rows).
__device__ __forceinline__ int swz64(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

// XOR swizzle of the chunks of a [k][n] LDS row of 16-bit B (given k x n),
// indexed by k mod 4: the transposing reads of four consecutive k rows then
// cover distinct banks whether a pass serves 16 or 32 lanes.  Rows of 256
// bytes or more use the table; 128-byte rows (which alternate between the
// halves of a 256-byte bank window) use 2 * (k mod 4).
__device__ __forceinline__ int swz_kn(int k, int cpr) {
    if (cpr == 8) return 2 * (k & 3);
    constexpr int t = (0 << 0) | (4 << 5) | (10 << 10) | (14 << 15);
    return (t >> (5 * (k & 3))) & 31;
}


// XOR swizzle of the chunks of a [k][n] LDS row of 8-bit B (given k x n),
// indexed by k mod 8.  The transposing byte reads take 8 consecutive k rows
// and one 16-byte chunk per 16-lane group (two adjacent chunks per 32
// lanes); with 256-byte rows the table keeps both the chunk index mod 8 and
// its upper three bits distinct over the 8 rows, with 128-byte rows (where
// the rows alternate between bank halves) the identity does.
__device__ __forceinline__ int swz_kn8(int k, int cpr) {
    const int r = k & 7;
    return cpr == 16 ? 2 * r + (r >> 2) : r;
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2_t;

template <int DIN, int DOUT, int OPB, int BM, int BN, int WM, int WN, int S, bool REG, int RB, bool MX = false>
struct Tile2Cfg {
    static constexpr int NW = WM * WN, NT = NW * 64;
    static constexpr int ESZ = Elem<DIN>::size;
    // bytes of an A (or n x k B) row per K step: RB (64 or 128) for 16-bit
    // inputs; fp8 rows are 128 bytes, or 64 with RB = 32
    static constexpr int ROWB = ESZ == 1 ? (RB == 32 ? 64 : 128) : RB;
    static constexpr int BK = ROWB / ESZ;             // K elements per step: 32/64 (16-bit) or 64/128 (fp8)
    // MFMA k sub-steps per step: even, or one (fp8 64-byte rows), when the
    // two fragment register sets alternate from step to step
    static constexpr int NKK = ESZ == 1 ? ROWB / 64 : ROWB / 32;
    static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row: 4 or 8
    static constexpr int RPC = 1024 / ROWB;           // rows per 1 KiB copy
    static constexpr int EPC = 16 / ESZ;              // elements per 16-byte chunk
    static constexpr int A_BYTES = BM * ROWB;
    static constexpr int B_BYTES = BK * BN * ESZ;     // same for both B layouts
    // MX block scales: each wave stages the 4 E8M0 bytes of a step (128 K
    // values) for each of its TM rows of A and TN columns of B, one 4-byte
    // direct copy (64 lanes) per 64 rows or columns
    static constexpr int SCA = MX ? (BM / WM) / 64 : 0;
    static constexpr int SCB = MX ? (BN / WN) / 64 : 0;
    static constexpr int SC_WAVE = (SCA + SCB) * 256;   // bytes per wave per stage
    static constexpr int SC_BYTES = NW * SC_WAVE;
    static constexpr int STAGE = A_BYTES + B_BYTES + SC_BYTES;
    // stages that fit; the register-staged copy uses two (its lookahead is
    // in registers)
    static constexpr int SE = REG ? 2 : (S * STAGE <= 160 * 1024 ? S : (160 * 1024) / STAGE);
    static constexpr int A_INS = A_BYTES / 1024 / NW;   // 1 KiB copies per wave per step
    static constexpr int B_INS = B_BYTES / 1024 / NW;
    static constexpr int VM_PER_STEP = A_INS + B_INS + SCA + SCB;
    // Direct copies spread among the MFMAs: the copies of a step start
    // while the stage they fill is two steps from being read, each sub-step
    // region taking an equal share.  With three stages that leaves them
    // about one step to land, less than the burst loop's two: measured
    // slower (fp8 256 x 128), so it takes four or more.
    static constexpr bool SPREAD = !REG && SE >= 4 && VM_PER_STEP % NKK == 0;
    static constexpr int KN_ROWB = BN * ESZ;          // bytes per [k][n] LDS row
    static constexpr int KN_CPR = KN_ROWB / 16;       // 16-byte chunks per [k][n] row
    static constexpr int KN_RPI = 1024 / KN_ROWB;     // [k][n] rows per 1 KiB copy
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    // LDS reads per fragment and k sub-step: 16-bit A 1 x 16 B; fp8 A 2 x 16 B;
    // k x n B: 2 transposing 16-bit reads or 4 transposing byte reads
    static constexpr int NRA = ESZ == 1 ? 2 : 1;
    static constexpr int NRB = OPB == GE_OP_T ? NRA : (ESZ == 1 ? 4 : 2);
    static_assert(DIN == GE_F16 || DIN == GE_BF16 || DIN == GE_F8_E4M3, "16-bit or fp8 inputs");
    static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "whole copies per wave");
    static_assert(OPB == GE_OP_T || (ESZ == 2 ? (KN_CPR >= 8 && KN_CPR <= 64) : (KN_CPR == 8 || KN_CPR == 16)),
                  "[k][n] swizzles cover 128..1024-byte (16-bit) or 128/256-byte (fp8) rows");
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(SE >= 2, "LDS budget");
    static_assert(ROWB == 64 || ROWB == 128, "64- or 128-byte rows");
    static_assert(NKK % 2 == 0 || (NKK == 1 && SPREAD && SE % 2 == 0 && !MX),
                  "fragment sets alternate over an even number of sub-steps, or from step to step over an "
                  "even number of stages with spread copies");
    static_assert(!MX || (ESZ == 1 && !REG && (BM / WM) % 64 == 0 && (BN / WN) % 64 == 0),
                  "MX scales: fp8 elements, direct copies, wave tiles of whole 64-row groups");
    static_assert((SE - 1) * VM_PER_STEP < 64, "vmcnt range");
    static_assert(!SPREAD || (SE - 3) * VM_PER_STEP + (NKK - 1) * (VM_PER_STEP / NKK) < 64, "vmcnt range");
};

// swizzle of the chunks of a ROWB-byte row (A, or B given n x k).  Both
// depend on row bits 0-4 only: a fragment read covers 32 consecutive rows,
// and rows 32 apart then share the swizzle, so the fragments of a wave tile
// lie at constant offsets from each other (immediate offsets of the reads
// rather than one address register per fragment)
template <int ROWB>
__device__ __forceinline__ int swz_row(int row) {
    if constexpr (ROWB == 64) return swz64(row);
    else return lds_swz(row & 31);   // 128-byte rows: eight rows cover the 8 chunk slots
}

// One kernel template for the plain and the block-scaled (MX) instantiations.
// Its body stays in the __global__ function itself: moved into a force-inlined
// device function, the same code compiled to 3x the scalar-register spills
// and 768 bytes of scratch per lane on the 256 x 256 tile (10x slower).
template <int DIN, int DOUT, int OPB, int BM, int BN, int WM, int WN, int S, bool REG, int RB, bool SPLIT = false,
          bool MX = false>
__global__ void __launch_bounds__(WM* WN * 64) ge_tile2_kernel(KernelArgs p_all, MxArgs mx_all) {
    const KernelArgs p = batch_slice(p_all, blockIdx.y);   // this product of a batch
    using C = Tile2Cfg<DIN, DOUT, OPB, BM, BN, WM, WN, S, REG, RB, MX>;
    constexpr int BK = C::BK, SE = C::SE, ESZ = C::ESZ, EPC = C::EPC;
    using Frag = typename std::conditional<ESZ == 1, i32x8, u32x4>::type;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[SE * C::STAGE];

    int tm, tn;
    tile_coords<DIN, DOUT, OPB, BM, BN, WM, WN>(p, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int M = p.m, N = p.n;
    // split-K (SPLIT): this workgroup takes K slice blockIdx.z of k_per_split
    // elements; its partial accumulators are summed in slice order by the
    // last slice to finish the tile, which then runs the epilogue
    const int slice = SPLIT ? (int)blockIdx.z : 0;
    const int ks = SPLIT ? slice * p.k_per_split : 0;
    const int K = SPLIT ? max(0, min(p.k - ks, p.k_per_split)) : p.k;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int wm = wave % WM, wn = wave / WM;
    const int r32 = lane & 31, h = lane >> 5;
    const uint8_t* gA = (const uint8_t*)p.A + (int64_t)ks * ESZ;
    const uint8_t* gB = (const uint8_t*)p.B + (OPB == GE_OP_T ? (int64_t)ks * ESZ : (int64_t)ks * p.ldb * ESZ);
    const int KT = (K + BK - 1) / BK;       // K steps
    const int KF = K / BK;                  // full K steps (direct copies)
    // The full steps are taken in a rotated order, step t reading K position
    // kpos(t) = (t + koff) mod KF (the ragged step, if any, stays last), with
    // koff growing by k_stagger per tile row and column of the group, so that
    // the tiles sharing a panel of A or B do not request its lines at the
    // same moment.
    const int koff = (p.k_stagger > 0 && KF > 1)
                         ? (int)(((int64_t)(tm % max(p.group_m, 1) + tn) * p.k_stagger) % KF)
                         : 0;
    auto kpos = [&](int t) __attribute__((always_inline)) {
        const int q = t + koff;
        return q >= KF ? q - KF : q;
    };

    // ---- per-lane sources of this wave's 1 KiB copies, at K step 0 ----
    // A: copy i covers LDS rows R = (wave*A_INS + i)*RPC + lane/CPR, slot lane%CPR
    // srcA/srcB: per-lane addresses (register-staged copies); voA/voB: the
    // same as 32-bit offsets from the tile's wave-uniform bases baseA/baseB
    // (direct copies).  The planner keeps a tile's span of A rows (and of B
    // given n x k) below 4 GiB.
    const uint8_t* srcA[C::A_INS];
    uint32_t voA[C::A_INS], voB[C::B_INS];
    int rowA_cp[C::A_INS], chA_cp[C::A_INS];
#pragma unroll
    for (int i = 0; i < C::A_INS; ++i) {
        const int R = (wave * C::A_INS + i) * C::RPC + lane / C::CPR;
        const int c = (lane % C::CPR) ^ swz_row<C::ROWB>(R);
        const int gm = min(m0 + R, max(M - 1, 0));
        rowA_cp[i] = m0 + R;
        chA_cp[i] = c;
        srcA[i] = gA + ((int64_t)gm * p.lda + c * EPC) * ESZ;
        voA[i] = (uint32_t)(((int64_t)(gm - m0) * p.lda + c * EPC) * ESZ);
    }
    const uint8_t* srcB[C::B_INS];
    int rowB_cp[C::B_INS], chB_cp[C::B_INS];
    const int nlast = N > 0 ? ((N - 1) / EPC) * EPC : 0;   // start of the last chunk holding valid columns
#pragma unroll
    for (int i = 0; i < C::B_INS; ++i) {
        if constexpr (OPB == GE_OP_T) {
            const int R = (wave * C::B_INS + i) * C::RPC + lane / C::CPR;
            const int c = (lane % C::CPR) ^ swz_row<C::ROWB>(R);
            const int gn = min(n0 + R, max(N - 1, 0));
            rowB_cp[i] = n0 + R;
            chB_cp[i] = c;
            srcB[i] = gB + ((int64_t)gn * p.ldb + c * EPC) * ESZ;
            voB[i] = (uint32_t)(((int64_t)(gn - n0) * p.ldb + c * EPC) * ESZ);
        } else {
            const int kr = (wave * C::B_INS + i) * C::KN_RPI + lane / C::KN_CPR;
            const int c = (lane % C::KN_CPR) ^ (ESZ == 1 ? swz_kn8(kr, C::KN_CPR) : swz_kn(kr, C::KN_CPR));
            const int gn = min(n0 + c * EPC, nlast);
            rowB_cp[i] = kr;
            chB_cp[i] = n0 + c * EPC;
            srcB[i] = gB + ((int64_t)kr * p.ldb + gn) * ESZ;
            voB[i] = (uint32_t)(((int64_t)kr * p.ldb + (gn - n0)) * ESZ);
        }
    }
    const int64_t stepA = (int64_t)BK * ESZ;
    const uint8_t* baseA = gA + (int64_t)m0 * p.lda * ESZ;
    const uint8_t* baseB = OPB == GE_OP_T ? gB + (int64_t)n0 * p.ldb * ESZ : gB + (int64_t)n0 * ESZ;
    const int64_t stepB = (OPB == GE_OP_T) ? (int64_t)BK * ESZ : (int64_t)BK * p.ldb * ESZ;

    // MX block scales: lane l of scale copy c fetches, at step t, the 4 bytes
    // 4t .. 4t+3 (blocks of 32 K values) of row wm*TM + 64c + l of A, or of
    // column wn*TN + 64c + l of B; rows and columns past the edge are clamped
    // (their outputs are never stored)
    const uint8_t* srcSA[C::SCA > 0 ? C::SCA : 1];
    const uint8_t* srcSB[C::SCB > 0 ? C::SCB : 1];
    if constexpr (MX) {
        const uint8_t* sa = mx_all.sa + (int64_t)blockIdx.y * mx_all.bs_sa;
        const uint8_t* sb = mx_all.sb + (int64_t)blockIdx.y * mx_all.bs_sb;
#pragma unroll
        for (int c = 0; c < C::SCA; ++c)
            srcSA[c] = sa + (int64_t)min(m0 + wm * C::TM + 64 * c + lane, max(M - 1, 0)) * mx_all.ld;
#pragma unroll
        for (int c = 0; c < C::SCB; ++c)
            srcSB[c] = sb + (int64_t)min(n0 + wn * C::TN + 64 * c + lane, max(N - 1, 0)) * mx_all.ld;
    }
    // this wave's scale words of the step held in `stage`
    auto sc_base = [&](int stage) {
        return smem + SE * (C::A_BYTES + C::B_BYTES) + stage * C::SC_BYTES + wave * C::SC_WAVE;
    };

    // direct copy c (A copies first, then B, then the MX scale words) of full
    // K step t into stage t % SE
    auto copy_one = [&](int t, int c) __attribute__((always_inline)) {
        uint8_t* sa = smem + (t % SE) * C::A_BYTES;                      // A stages first,
        uint8_t* sb = smem + SE * C::A_BYTES + (t % SE) * C::B_BYTES;    // then B stages
        if (c < C::A_INS)
            copy_to_lds16_sb(voA[c], baseA + (int64_t)kpos(t) * stepA, lds_addr(sa + (wave * C::A_INS + c) * 1024));
        else if (c < C::A_INS + C::B_INS)
            copy_to_lds16_sb(voB[c - C::A_INS], baseB + (int64_t)kpos(t) * stepB,
                             lds_addr(sb + (wave * C::B_INS + c - C::A_INS) * 1024));
        else if constexpr (MX) {
            const int sc = c - C::A_INS - C::B_INS;   // scale copy: A rows first, then B columns
            const uint8_t* src = sc < C::SCA ? srcSA[sc] : srcSB[sc - C::SCA];
            copy_to_lds4(src + 4 * kpos(t), lds_addr(sc_base(t % SE) + sc * 256));
        }
    };
    // issue the direct copies of full K step t into stage t % SE
    auto issue_direct = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < C::VM_PER_STEP; ++c) copy_one(t, c);
    };

    // the ragged last K step t: through registers, elements at k >= K zeroed
    // (the staging lambdas are forced inline: left to the inliner, the 4-wave
    // 256 x 256 tile called this path as a function, with KernelArgs copied to
    // a 2 KiB stack frame in scratch memory)
    auto issue_tail = [&](int t) __attribute__((always_inline)) {
        uint8_t* sa = smem + (t % SE) * C::A_BYTES;
        uint8_t* sb = smem + SE * C::A_BYTES + (t % SE) * C::B_BYTES;
        const int k0 = t * BK;
        u32x4 va[C::A_INS], vb[C::B_INS];
#pragma unroll
        for (int i = 0; i < C::A_INS; ++i)
            va[i] = load_chunk<ESZ>(gA, p.lda, min(rowA_cp[i], max(M - 1, 0)), M, k0 + chA_cp[i] * EPC, K);
#pragma unroll
        for (int i = 0; i < C::B_INS; ++i) {
            if constexpr (OPB == GE_OP_T)
                vb[i] = load_chunk<ESZ>(gB, p.ldb, min(rowB_cp[i], max(N - 1, 0)), N, k0 + chB_cp[i] * EPC, K);
            else
                vb[i] = load_chunk<ESZ>(gB, p.ldb, k0 + rowB_cp[i], K, min(chB_cp[i], nlast), N);
        }
#pragma unroll
        for (int i = 0; i < C::A_INS; ++i) *(u32x4*)(sa + (wave * C::A_INS + i) * 1024 + lane * 16) = va[i];
#pragma unroll
        for (int i = 0; i < C::B_INS; ++i)
            *(u32x4*)(sb + (wave * C::B_INS + i) * 1024 + lane * 16) = vb[i];
        if constexpr (MX) {
            // blocks at or past ceil(k/32) hold no data (their elements were
            // zeroed above) and their bytes may be anything, NaN codes
            // included: they become 127 (a factor of 1)
            uint32_t keep = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (4 * t + j < mx_all.kb) keep |= 0xffu << (8 * j);
#pragma unroll
            for (int sc = 0; sc < C::SCA + C::SCB; ++sc) {
                const uint8_t* src = sc < C::SCA ? srcSA[sc] : srcSB[sc - C::SCA];
                const uint32_t w = *(const uint32_t*)(src + 4 * t);
                *(uint32_t*)(sc_base(t % SE) + sc * 256 + lane * 4) = (w & keep) | (0x7f7f7f7fu & ~keep);
            }
        }
    };

    auto issue = [&](int t) __attribute__((always_inline)) {
        if (t < KF) issue_direct(t);
        else issue_tail(t);
    };

    f32x16 acc[C::FN][C::FM];
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};

    // Per-lane LDS read offsets within a stage.  Any assignment of K values
    // to (lane half, operand element) is valid as long as A and B use the
    // same one.  16-bit: sub-step kk, lane half h reads k 16kk + 8h .. +7.
    // fp8: sub-step kk, lane half h reads k 64kk + 16h .. +15 into its bytes
    // 0-15 and k 64kk + 32 + 16h .. +15 into bytes 16-31.  That is the
    // assignment the block-scaled instruction needs: it scales bytes 0-15 of
    // every lane by the E8M0 value of the row's lane half 0 and bytes 16-31 by
    // that of lane half 1 (measured), so each 32-value K block of the
    // instruction must be the two lane halves' 16-byte pieces.
    // (fragment f of A sits 32 rows below fragment f - 1: offset
    // offA[kk][e] + f * 32 * ROWB, the swizzle repeating every 32 rows)
    int offA[C::NKK][C::NRA];
    {
        const int row = wm * C::TM + r32;
#pragma unroll
        for (int kk = 0; kk < C::NKK; ++kk)
#pragma unroll
            for (int e = 0; e < C::NRA; ++e) {
                const int chunk = ESZ == 1 ? 4 * kk + h + 2 * e : 2 * kk + h;
                offA[kk][e] = row * C::ROWB + ((chunk ^ swz_row<C::ROWB>(row)) << 4);
            }
    }
    // B given n x k: as A.  B given k x n, transposing reads:
    //  16-bit, read e of 2: group G, lane i: k = 16kk + 8(G/2) + 4e + i/4,
    //          n = wave col + 32f + 16(G%2) + 4(i%4);
    //  fp8, read e of 4:    group G, lane i: k = 64kk + 16(G/2) + 32(e/2) +
    //          8(e%2) + i/2, n = wave col + 32f + 16(G%2) + 8(i%2)
    //          (the lane halves' K pieces as for A).
    // (n x k: fragment f at offB[0][kk][e] + f * 32 * ROWB, as for A.
    // k x n: the swizzles depend on k mod 4 (16-bit) or mod 8 (fp8) only, so
    // the sub-steps and reads of a fragment lie at constant k-row offsets
    // from its first read (kn_koff); one base per fragment, offB[f][0][0])
    constexpr int NBF = OPB == GE_OP_T ? 1 : C::FN;
    constexpr int NBK = OPB == GE_OP_T ? C::NKK : 1;
    constexpr int NBE = OPB == GE_OP_T ? C::NRB : 1;
    int offB[NBF][NBK][NBE];
#pragma unroll
    for (int f = 0; f < NBF; ++f) {
#pragma unroll
        for (int kk = 0; kk < NBK; ++kk) {
#pragma unroll
            for (int e = 0; e < NBE; ++e) {
                if constexpr (OPB == GE_OP_T) {
                    const int row = wn * C::TN + r32;
                    const int chunk = ESZ == 1 ? 4 * kk + h + 2 * e : 2 * kk + h;
                    offB[f][kk][e] = row * C::ROWB + ((chunk ^ swz_row<C::ROWB>(row)) << 4);
                } else if constexpr (ESZ == 2) {
                    const int G = lane >> 4, i = lane & 15;
                    const int k = 8 * (G >> 1) + (i >> 2);
                    const int n = wn * C::TN + f * 32 + 16 * (G & 1) + 4 * (i & 3);
                    offB[f][kk][e] =
                        k * C::KN_ROWB + (((n >> 3) ^ swz_kn(k, C::KN_CPR)) << 4) + ((n & 4) << 1);
                } else {
                    const int G = lane >> 4, i = lane & 15;
                    const int k = 16 * (G >> 1) + (i >> 1);
                    const int n = wn * C::TN + f * 32 + 16 * (G & 1) + 8 * (i & 1);
                    offB[f][kk][e] = k * C::KN_ROWB +
                                     (((n >> 4) ^ swz_kn8(k, C::KN_CPR)) << 4) + (n & 8);
                }
            }
        }
    }
    // k-row offset of read e of sub-step kk of a k x n fragment:
    //  16-bit: k = 16kk + 8(G/2) + 4e + i/4;  fp8: k = 64kk + 16(G/2) +
    //  32(e/2) + 8(e%2) + i/2 (the lane halves' K pieces as for A)
    auto kn_koff = [](int kk, int e) {
        return ESZ == 2 ? 16 * kk + 4 * e : 64 * kk + 32 * (e >> 1) + 8 * (e & 1);
    };
    auto offB_at = [&](int f, int kk, int e) __attribute__((always_inline)) {
        if constexpr (OPB == GE_OP_T) return offB[0][kk][e] + f * 32 * C::ROWB;
        else return offB[f][0][0] + kn_koff(kk, e) * C::KN_ROWB;
    };

    auto read16 = [&](const uint8_t* a) { return *(const u32x4*)a; };
    // fragment f of B (or of A) for k sub-step kk of the step held in `stage`
    auto load_fragB = [&](int stage, int kk, int f, Frag (&bfr)[C::FN]) {
        const uint8_t* st = smem + SE * C::A_BYTES + stage * C::B_BYTES;   // B stage
        if constexpr (OPB == GE_OP_T && ESZ == 2) {
            bfr[f] = read16(st + offB_at(f, kk, 0));
        } else if constexpr (OPB == GE_OP_T) {
            const u32x4 lo = read16(st + offB_at(f, kk, 0)), hi = read16(st + offB_at(f, kk, 1));
            bfr[f] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                           (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else if constexpr (ESZ == 2) {
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t*)((lds_void_t*)(st + offB_at(f, kk, 0))));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_t*)((lds_void_t*)(st + offB_at(f, kk, 1))));
            bfr[f] = u32x4{(uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                           (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                           (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                           (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16)};
        } else {
            i32x2 v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (lds_i32x2_t*)((lds_void_t*)(st + offB_at(f, kk, e))));
            bfr[f] = i32x8{v[0][0], v[0][1], v[1][0], v[1][1], v[2][0], v[2][1], v[3][0], v[3][1]};
        }
    };
    auto load_fragA = [&](int stage, int kk, int f, Frag (&af)[C::FM]) {
        const uint8_t* st = smem + stage * C::A_BYTES;   // A stage
        if constexpr (ESZ == 2) {
            af[f] = read16(st + offA[kk][0] + f * 32 * C::ROWB);
        } else {
            const u32x4 lo = read16(st + offA[kk][0] + f * 32 * C::ROWB),
                        hi = read16(st + offA[kk][1] + f * 32 * C::ROWB);
            af[f] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    };
    // MX: the scale word of this lane's row (A) or column (B) for the step
    // held in `stage`, shifted so that its byte 0 is the scale of the lane's
    // block: sub-step kk, lane half h reads the 32 K values of block 2kk + h
    // (the MFMA's lane half h is its K block h; op_sel then stays 0)
    auto load_scale = [&](int stage, int kk, int slot) -> uint32_t {
        const uint32_t w = *(const uint32_t*)(sc_base(stage) + slot * 4);
        return w >> (8 * h + 16 * kk);
    };
    // all fragments (and MX scale words) of one k sub-step (kk) of the step
    // held in `stage`
    auto load_frags = [&](int stage, int kk, Frag (&af)[C::FM], Frag (&bfr)[C::FN], uint32_t (&sca)[C::FM],
                          uint32_t (&scb)[C::FN]) {
#pragma unroll
        for (int f = 0; f < C::FN; ++f) load_fragB(stage, kk, f, bfr);
#pragma unroll
        for (int f = 0; f < C::FM; ++f) load_fragA(stage, kk, f, af);
        if constexpr (MX) {
#pragma unroll
            for (int f = 0; f < C::FM; ++f) sca[f] = load_scale(stage, kk, f * 32 + r32);
#pragma unroll
            for (int f = 0; f < C::FN; ++f) scb[f] = load_scale(stage, kk, C::SCA * 64 + f * 32 + r32);
        }
    };
    // MFMA number idx (B fragment idx / FM, A fragment idx % FM) of a sub-step
    auto mfma_one = [&](int idx, const Frag (&af)[C::FM], const Frag (&bfr)[C::FN], const uint32_t (&sca)[C::FM],
                        const uint32_t (&scb)[C::FN]) {
        const int i = idx / C::FM, j = idx % C::FM;
        if constexpr (DIN == GE_BF16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, bfr[i]), __builtin_bit_cast(bf16x8, af[j]), acc[i][j], 0, 0, 0);
        else if constexpr (DIN == GE_F16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, bfr[i]), __builtin_bit_cast(f16x8, af[j]), acc[i][j], 0, 0, 0);
        else if constexpr (MX)   // E4M3 operands with E8M0 block scales: src0 = B's, src1 = A's
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[i], af[j], acc[i][j], 0, 0, 0,
                                                                         (int)scb[i], 0, (int)sca[j]);
        else   // OCP E4M3 operands (format code 0 for both), no block scales
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[i], af[j], acc[i][j], 0, 0, 0, 0,
                                                                         0, 0);
    };
    auto mfmas = [&](const Frag (&af)[C::FM], const Frag (&bfr)[C::FN], const uint32_t (&sca)[C::FM],
                     const uint32_t (&scb)[C::FN]) {
#pragma unroll
        for (int idx = 0; idx < C::FM * C::FN; ++idx) mfma_one(idx, af, bfr, sca, scb);
    };
    // Scheduling order for a region holding one sub-step's MFMAs and the
    // next sub-step's fragment reads: LDS read and MFMA alternate, so the
    // matrix core is never left waiting behind a burst of reads.  With fewer
    // than four MFMAs per sub-step (the 64 x 64 tile) there is nothing to
    // alternate with, and the reads simply go first.
    auto interleave = [&]() {
        constexpr int NMF = C::FM * C::FN;
        constexpr int NDS = C::FM * C::NRA + C::FN * C::NRB + (MX ? C::FM + C::FN : 0);
        if constexpr (NMF >= 4) {
#pragma unroll
            for (int i = 0; i < (NMF > NDS ? NMF : NDS); ++i) {
                if (i < NDS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                if (i < NMF) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // Wait until this wave's copies of step t are done, given that the
    // copies of `later` further steps were issued after them.
    auto wait_step = [&](int later) {
        static_assert(SE <= 5, "wait ladder covers up to 4 later steps");
        if (later >= 4) wait_vm<(4 * C::VM_PER_STEP < 64 ? 4 * C::VM_PER_STEP : 63)>();
        else if (later == 3) wait_vm<(3 * C::VM_PER_STEP < 64 ? 3 * C::VM_PER_STEP : 63)>();
        else if (later == 2) wait_vm<(2 * C::VM_PER_STEP < 64 ? 2 * C::VM_PER_STEP : 63)>();
        else if (later == 1) wait_vm<C::VM_PER_STEP>();
        else wait_vm<0>();
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): own LDS reads and tail writes done
        // workgroup barrier without a memory fence (a fence would wait for
        // every copy in flight); the clobber keeps LDS accesses on their side
        asm volatile("s_barrier" ::: "memory");
    };

    if constexpr (REG) {
        static_assert(C::NKK == 2, "the register-staged loop takes two sub-steps per step");
        // ---- main loop, register-staged copies ----
        // Step t is fetched from global memory into register set t % 2 two
        // steps before it is written to LDS stage t % 2, right after the
        // barrier that frees that stage; it is read after the next barrier.
        // The compiler tracks these loads itself (no hand-counted waits).
        u32x4 ra0[C::A_INS], rb0[C::B_INS], ra1[C::A_INS], rb1[C::B_INS];
        auto fetch = [&](int t, u32x4 (&ra)[C::A_INS], u32x4 (&rb)[C::B_INS]) {
            if (t >= KT) return;
            if (t < KF) {
#pragma unroll
                for (int i = 0; i < C::A_INS; ++i) ra[i] = *(const u32x4*)(srcA[i] + (int64_t)kpos(t) * stepA);
#pragma unroll
                for (int i = 0; i < C::B_INS; ++i) rb[i] = *(const u32x4*)(srcB[i] + (int64_t)kpos(t) * stepB);
            } else {
                const int k0 = t * BK;
#pragma unroll
                for (int i = 0; i < C::A_INS; ++i)
                    ra[i] = load_chunk<ESZ>(gA, p.lda, min(rowA_cp[i], max(M - 1, 0)), M, k0 + chA_cp[i] * EPC, K);
#pragma unroll
                for (int i = 0; i < C::B_INS; ++i) {
                    if constexpr (OPB == GE_OP_T)
                        rb[i] = load_chunk<ESZ>(gB, p.ldb, min(rowB_cp[i], max(N - 1, 0)), N,
                                                k0 + chB_cp[i] * EPC, K);
                    else
                        rb[i] = load_chunk<ESZ>(gB, p.ldb, k0 + rowB_cp[i], K, min(chB_cp[i], nlast), N);
                }
            }
        };
        auto commit = [&](int t, const u32x4 (&ra)[C::A_INS], const u32x4 (&rb)[C::B_INS]) {
            if (t >= KT) return;
            uint8_t* st = smem + (t % 2) * C::A_BYTES;
            uint8_t* stb = smem + SE * C::A_BYTES + (t % 2) * C::B_BYTES;
#pragma unroll
            for (int i = 0; i < C::A_INS; ++i) *(u32x4*)(st + (wave * C::A_INS + i) * 1024 + lane * 16) = ra[i];
#pragma unroll
            for (int i = 0; i < C::B_INS; ++i)
                *(u32x4*)(stb + (wave * C::B_INS + i) * 1024 + lane * 16) = rb[i];
        };
        auto barrier = [&]() {
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): own LDS reads and writes done
            asm volatile("s_barrier" ::: "memory");
        };
        fetch(0, ra0, rb0);
        fetch(1, ra1, rb1);
        commit(0, ra0, rb0);
        commit(1, ra1, rb1);
        fetch(2, ra0, rb0);
        fetch(3, ra1, rb1);
        Frag a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
        uint32_t sa0[C::FM], sb0[C::FN], sa1[C::FM], sb1[C::FN];
        if (KT > 0) {
            barrier();
            load_frags(0, 0, a0, b0, sa0, sb0);
        }
        auto body = [&](int kt, u32x4 (&ra)[C::A_INS], u32x4 (&rb)[C::B_INS]) {
            load_frags(kt % 2, 1, a1, b1, sa1, sb1);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(a0, b0, sa0, sb0);
            barrier();
            commit(kt + 2, ra, rb);   // into stage kt % 2, free since the barrier
            fetch(kt + 4, ra, rb);
            load_frags((kt + 1) % 2, 0, a0, b0, sa0, sb0);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(a1, b1, sa1, sb1);
        };
        int kt = 0;
        for (; kt + 2 <= KT - 1; kt += 2) {
            body(kt, ra0, rb0);
            body(kt + 1, ra1, rb1);
        }
        if (kt < KT - 1) {
            body(kt, ra0, rb0);
            ++kt;
        }
        if (KT > 0) {
            load_frags((KT - 1) % 2, 1, a1, b1, sa1, sb1);
            mfmas(a0, b0, sa0, sb0);
            mfmas(a1, b1, sa1, sb1);
        }
    } else {
    if constexpr (C::SPREAD) {
    // ---- main loop, copies spread among the MFMAs ----
    // Step kt reads stage kt % SE.  Its sub-step regions also issue the
    // copies of step kt + SE - 1 into stage (kt - 1) % SE, which every wave
    // finished reading before the barrier of step kt - 1.  Each region puts
    // its share of the copies between its fragment reads, so that the
    // address unit takes them while the matrix cores run: issued in one
    // burst, they hold back every wave's next MFMA behind the copy queue.
    // The prologue starts SE - 1 steps; the last steps fall back to one
    // burst per step with the counted waits of the burst loop.
    constexpr int VM = C::VM_PER_STEP;
    constexpr int CPR = VM / C::NKK;   // copies per sub-step region
#pragma unroll
    for (int t = 0; t < SE - 1; ++t)
        if (t < KT) issue(t);
    Frag a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
    uint32_t sa0[C::FM], sb0[C::FN], sa1[C::FM], sb1[C::FN];   // MX scale words of each set
    if (KT > 0) {
        wait_step(min(SE - 2, KT - 1));
        load_frags(0, 0, a0, b0, sa0, sb0);
    }
    auto reads_first = [&]() {
        if constexpr (C::FM * C::FN < 4) __builtin_amdgcn_sched_barrier(0);
    };
    // one region: the fragment reads of sub-step rkk of stage rst into
    // (ra, rb), with NC copies of step ct (numbers c0 ..) placed evenly
    // between them, then the MFMAs of (ma, mb)
    auto region = [&](auto nc_c, int rst, int rkk, Frag (&ra)[C::FM], Frag (&rb)[C::FN], uint32_t (&rsa)[C::FM],
                      uint32_t (&rsb)[C::FN], const Frag (&ma)[C::FM], const Frag (&mb)[C::FN],
                      const uint32_t (&msa)[C::FM], const uint32_t (&msb)[C::FN], int ct, int c0)
        __attribute__((always_inline)) {
        constexpr int NC = decltype(nc_c)::value;
        constexpr int R = C::FN + C::FM;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (r < C::FN) load_fragB(rst, rkk, r, rb);
            else load_fragA(rst, rkk, r - C::FN, ra);
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                const int pos = min(max((j + 1) * R / (NC + 1) - 1, 0), R - 1);
                if (pos == r) copy_one(ct, c0 + j);
            }
        }
        if constexpr (MX) {
#pragma unroll
            for (int f = 0; f < C::FM; ++f) rsa[f] = load_scale(rst, rkk, f * 32 + r32);
#pragma unroll
            for (int f = 0; f < C::FN; ++f) rsb[f] = load_scale(rst, rkk, C::SCA * 64 + f * 32 + r32);
        }
        reads_first();
        mfmas(ma, mb, msa, msb);
        interleave();
    };
    auto step_spread = [&](int kt, int stage) __attribute__((always_inline)) {
        const int ct = kt + SE - 1;
        if constexpr (C::NKK == 1) {
            // one sub-step per step: step kt's fragments are in set kt & 1
            // (stage has kt's parity: SE is even); after the barrier the
            // region reads step kt + 1's into the other set, issues every
            // copy of step kt + SE - 1 and runs step kt's MFMAs
            wait_vm<(SE - 3) * VM>();
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): own LDS reads done
            asm volatile("s_barrier" ::: "memory");
            if ((stage & 1) == 0)
                region(std::integral_constant<int, VM>{}, (stage + 1) % SE, 0, a1, b1, sa1, sb1, a0, b0, sa0, sb0,
                       ct, 0);
            else
                region(std::integral_constant<int, VM>{}, (stage + 1) % SE, 0, a0, b0, sa0, sb0, a1, b1, sa1, sb1,
                       ct, 0);
            return;
        }
#pragma unroll
        for (int kk = 0; kk < C::NKK - 1; ++kk) {
            if (kk % 2 == 0)
                region(std::integral_constant<int, CPR>{}, stage, kk + 1, a1, b1, sa1, sb1, a0, b0, sa0, sb0, ct,
                       kk * CPR);
            else
                region(std::integral_constant<int, CPR>{}, stage, kk + 1, a0, b0, sa0, sb0, a1, b1, sa1, sb1, ct,
                       kk * CPR);
        }
        // step kt + 1 has landed once only the copies issued after it are
        // outstanding: steps kt + 2 .. kt + SE - 2 and this step's regions'
        // share of step kt + SE - 1
        wait_vm<(SE - 3) * VM + (C::NKK - 1) * CPR>();
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): own LDS reads done
        asm volatile("s_barrier" ::: "memory");
        region(std::integral_constant<int, VM - (C::NKK - 1) * CPR>{}, (stage + 1) % SE, 0, a0, b0, sa0, sb0, a1,
               b1, sa1, sb1, ct, (C::NKK - 1) * CPR);
    };
    auto inner = [&](int stage) {
#pragma unroll
        for (int kk = 0; kk < C::NKK - 1; ++kk) {
            if (kk % 2 == 0) {
                load_frags(stage, kk + 1, a1, b1, sa1, sb1);
                reads_first();
                mfmas(a0, b0, sa0, sb0);
            } else {
                load_frags(stage, kk + 1, a0, b0, sa0, sb0);
                reads_first();
                mfmas(a1, b1, sa1, sb1);
            }
            interleave();
        }
    };
    // (odd_c: with one sub-step per step, whether kt is odd, i.e. which set
    // holds step kt's fragments)
    auto step_last = [&](int kt, int stage, auto odd_c) __attribute__((always_inline)) {
        if (kt + SE - 1 < KT) issue(kt + SE - 1);
        __builtin_amdgcn_sched_barrier(0);
        inner(stage);
        wait_step(min(SE - 2, KT - 2 - kt));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (C::NKK == 1 && !decltype(odd_c)::value) {
            load_frags((stage + 1) % SE, 0, a1, b1, sa1, sb1);
            reads_first();
            mfmas(a0, b0, sa0, sb0);
        } else {
            load_frags((stage + 1) % SE, 0, a0, b0, sa0, sb0);
            reads_first();
            mfmas(a1, b1, sa1, sb1);   // the last sub-step (NKK - 1 is odd), or step kt of odd kt
        }
        interleave();
    };
    int kt = 0;
    // SE steps per iteration (constant stage offsets), each issuing the
    // copies of a full step
    for (; kt + 2 * SE - 2 < KF; kt += SE) {
#pragma unroll
        for (int u = 0; u < SE; ++u) step_spread(kt + u, u);
    }
    if constexpr (C::NKK == 1) {
        // kt is even here (a multiple of SE): steps in pairs, so that each
        // call knows its set; the last step's MFMAs use the set the final
        // reads went to
        for (; kt + 2 <= KT - 1; kt += 2) {
            step_last(kt, kt % SE, std::false_type{});
            step_last(kt + 1, (kt + 1) % SE, std::true_type{});
        }
        // one final MFMA call on set 0 (an odd tail moves its last
        // fragments there): with a call per path, the two paths' ends left
        // the accumulators in different registers and the join spilled them
        if (kt < KT - 1) {
            step_last(kt, kt % SE, std::false_type{});
#pragma unroll
            for (int f = 0; f < C::FM; ++f) {
                a0[f] = a1[f];
                sa0[f] = sa1[f];
            }
#pragma unroll
            for (int f = 0; f < C::FN; ++f) {
                b0[f] = b1[f];
                sb0[f] = sb1[f];
            }
        }
        if (KT > 0) mfmas(a0, b0, sa0, sb0);
    } else {
        for (; kt < KT - 1; ++kt) step_last(kt, kt % SE, std::false_type{});
        if (KT > 0) {
            inner((KT - 1) % SE);
            mfmas(a1, b1, sa1, sb1);
        }
    }
    } else {
    static_assert(C::NKK % 2 == 0, "the burst loop alternates the sets within a step");
    // ---- main loop ----
    // All SE stages start filling at once; afterwards the copy of step
    // kt + SE goes into the stage step kt used, as soon as every wave has
    // read its last fragments from it.  The barrier sits between the two
    // k sub-steps of a step, so the first fragments of step kt + 1 are read
    // while the matrix cores still work on step kt.
#pragma unroll
    for (int t = 0; t < SE; ++t)
        if (t < KT) issue(t);
    Frag a0[C::FM], b0[C::FN], a1[C::FM], b1[C::FN];
    uint32_t sa0[C::FM], sb0[C::FN], sa1[C::FM], sb1[C::FN];   // MX scale words of each set
    if (KT > 0) {
        wait_step(min(SE - 1, KT - 1));
        load_frags(0, 0, a0, b0, sa0, sb0);
    }
    // (the last step is peeled off so that the loop body always passes the
    // barrier: a merged path would make the compiler's wait analysis hold
    // the second-half MFMAs until the next step's fragment reads return)
    // sub-steps kk = 0 .. NKK-2 of step kt: the fragments of sub-step kk+1
    // are read (into the other register set) ahead of the MFMAs of kk
    // (small tiles: a fence between the reads and the MFMAs, as above)
    auto reads_first = [&]() {
        if constexpr (C::FM * C::FN < 4) __builtin_amdgcn_sched_barrier(0);
    };
    auto inner = [&](int stage) {
#pragma unroll
        for (int kk = 0; kk < C::NKK - 1; ++kk) {
            // each group of fragment reads is issued ahead of the MFMAs that
            // do not need it (the scheduler would otherwise sink the last
            // reads to the end of the block and stall the next MFMAs on them)
            if (kk % 2 == 0) {
                load_frags(stage, kk + 1, a1, b1, sa1, sb1);
                reads_first();
                mfmas(a0, b0, sa0, sb0);
            } else {
                load_frags(stage, kk + 1, a0, b0, sa0, sb0);
                reads_first();
                mfmas(a1, b1, sa1, sb1);
            }
            interleave();
        }
    };
    auto step_body = [&](int kt, int stage) {
        inner(stage);
        wait_step(min(SE - 2, KT - 2 - kt));
        if (kt + SE < KT) issue(kt + SE);
        // the copies stay ahead of the reads below; the last sub-step's
        // MFMAs interleave with the reads of step kt + 1's first fragments
        __builtin_amdgcn_sched_barrier(0);
        load_frags((stage + 1) % SE, 0, a0, b0, sa0, sb0);
        reads_first();
        mfmas(a1, b1, sa1, sb1);   // the last sub-step (NKK - 1 is odd)
        interleave();
    };
    {
        // SE steps per iteration, so that each stage's LDS base is a
        // constant the fragment reads can take as an immediate offset
        int kt = 0;
        for (; kt + SE <= KT - 1; kt += SE) {
#pragma unroll
            for (int u = 0; u < SE; ++u) step_body(kt + u, u);
        }
        for (int u = 0; kt < KT - 1; ++kt, ++u) step_body(kt, u);
    }
    if (KT > 0) {
        inner((KT - 1) % SE);
        mfmas(a1, b1, sa1, sb1);
    }
    }   // spread or burst copies
    }   // copy mode

    if constexpr (SPLIT) {
        if (p.split_k > 1) {
            // publish this slice's accumulators, count the arrival, and let
            // the last slice sum them.  Device-scope atomic accesses keep the
            // partials coherent across the dies' separate L2s without a
            // cache-wide fence; they write through to memory one dword per
            // lane, so accumulator element r of thread t sits at r * NT + t
            // and each instruction covers 256 contiguous bytes (with each
            // thread's elements contiguous instead, an instruction touched
            // 64 separate 64-byte pieces, and two slices of 1024 x 512 x
            // 2048 took 27.5 us against 9.9 us unsplit)
            constexpr int PER = 16 * C::FM * C::FN;   // floats per thread
            const int64_t tile_lin = blockIdx.x;
            float* mine = p.partial + (tile_lin * p.split_k + slice) * (int64_t)(C::NT * PER) + tid;
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
                for (int j = 0; j < C::FM; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        __hip_atomic_store(mine + ((i * C::FM + j) * 16 + e) * C::NT, acc[i][j][e],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // every lane's stores are performed before the arrival is counted
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __shared__ int split_last;
            __syncthreads();
            if (tid == 0)
                split_last = (int)__hip_atomic_fetch_add(&p.counters[tile_lin], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT) == p.split_k - 1;
            __syncthreads();
            if (!split_last) return;
            // the loads below depend on the counter's value (the clobber keeps
            // them below the branch)
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
                for (int j = 0; j < C::FM; ++j) acc[i][j] = f32x16{};
            for (int sl = 0; sl < p.split_k; ++sl) {
                const float* ps = p.partial + (tile_lin * p.split_k + sl) * (int64_t)(C::NT * PER) + tid;
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int j = 0; j < C::FM; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            acc[i][j][e] += __hip_atomic_load(ps + ((i * C::FM + j) * 16 + e) * C::NT,
                                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (tid == 0) p.counters[tile_lin] = 0u;   // re-arm for the next launch
        }
    }

    // ---- fused epilogue on the accumulators (as in tile_kernel.h) ----
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
    // fp8 output: the bias is bf16; D = E4M3(y * scale_d), and the largest
    // |y| of the product goes to *amax (inference epilogues only: the host
    // refuses the C input, the aux matrix and the backward epilogues)
    constexpr bool OUT8 = DOUT == GE_F8_E4M3;
    constexpr int DB = OUT8 ? GE_BF16 : DOUT;
    const float sd = (OUT8 && p.scale_d) ? *p.scale_d : 1.0f;
    float amax_l = 0.0f;

    // The epilogue, unrolled over the accumulators, tests the epilogue kind
    // per element: on the 256 x 256 tiles that code holds every kind's
    // branches (130 KB, twice the instruction cache two CUs share) and is
    // fetched cold at the end of every tile (69 KB on the block-scaled
    // 128 x 128 tile).  There NONE, BIAS and the ReLU kinds also get
    // a copy compiled for their kind alone, picked once per tile, and so do
    // GELU_AUX_BIAS, DRELU and DGELU with bf16 input and output on the
    // 8-wave tile.
    auto epilogue = [&](auto ep_c) __attribute__((always_inline)) {
        const int ep = static_cast<int>(ep_c);   // a constant when ep_c is one
        const bool has_bias = epilog_has_bias(ep);
        const bool want_aux = ep == GE_EPILOG_RELU_AUX_BIAS;
        const bool want_pre = ep == GE_EPILOG_GELU_AUX_BIAS;
        const bool want_grad = epilog_is_grad(ep);
        const bool want_bgrad = epilog_is_bgrad(ep);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int m = m0 + wm * C::TM + fm * 32 + r32;
            const bool mok = m < M;
            float brow = 0.0f;
            if (has_bias && row_bias && mok) brow = load_scalar<DB>(p.bias, m);
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
                        if (full) load8<DB>(p.bias, nc, bc);
                        else {
#pragma unroll
                            for (int j = 0; j < 8; ++j) bc[j] = (nc + j < N) ? load_scalar<DB>(p.bias, nc + j) : 0.0f;
                        }
                    }
                    float gf[8], pre[8], cb[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        cb[j] = 0.0f;
                        gf[j] = 0.0f;
                    }
                    if constexpr (!OUT8) {
                        if (with_c && mok) beta_c8<DOUT>(p, beta, m, nc, cb);
                        if (want_grad && mok) grad_factor8<DOUT>(p, ep, m, nc, gf);
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
                    if constexpr (OUT8) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float av = __builtin_fabsf(v[g][j]);   // NaN compares false: not counted
                            if (mok && nc + j < N && av > amax_l) amax_l = av;
                            v[g][j] *= sd;
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
                        if constexpr (!OUT8) {
                            if (want_pre) store_pre8<DOUT>(p, m, nc, pre);
                        }
                    }
                }
                if (want_aux) {
                    bits |= (uint32_t)__shfl_xor((int)bits, 32);
                    if (h == 0 && mok && (nb >> 5) < p.ldaux) p.aux[(int64_t)m * p.ldaux + (nb >> 5)] = bits;
                }
            }
        }
    };
    if constexpr ((BM == 256 && BN == 256 && C::SPREAD && !SPLIT) || MX) {
        switch (p.epilog) {
        // (NONE is the product of the unfused pair: its own copy keeps that
        // baseline from paying the generic code's cost)
        case GE_EPILOG_NONE: epilogue(std::integral_constant<int, GE_EPILOG_NONE>{}); break;
        case GE_EPILOG_BIAS: epilogue(std::integral_constant<int, GE_EPILOG_BIAS>{}); break;
        case GE_EPILOG_RELU_BIAS: epilogue(std::integral_constant<int, GE_EPILOG_RELU_BIAS>{}); break;
        case GE_EPILOG_RELU_AUX_BIAS: epilogue(std::integral_constant<int, GE_EPILOG_RELU_AUX_BIAS>{}); break;
        default: {
            // three training kinds, for bf16 in and out on the 8-wave tile
            // (the planner's choice for the large backward products).  On
            // the 4-wave 256 x 256 tile, whose 128 accumulators per lane
            // leave no registers spare, the copy for DGELU_BGRAD gave a wrong
            // bias gradient, so that tile and the BGRAD kinds keep the
            // generic code.
            bool done = false;
            if constexpr (DIN == GE_BF16 && DOUT == GE_BF16 && WM * WN == 8) {
                done = true;
                switch (p.epilog) {
                case GE_EPILOG_GELU_AUX_BIAS: epilogue(std::integral_constant<int, GE_EPILOG_GELU_AUX_BIAS>{}); break;
                case GE_EPILOG_DRELU: epilogue(std::integral_constant<int, GE_EPILOG_DRELU>{}); break;
                case GE_EPILOG_DGELU: epilogue(std::integral_constant<int, GE_EPILOG_DGELU>{}); break;
                default: done = false; break;
                }
            }
            if (!done) epilogue(ep);
            break;
        }
        }
    } else {
        epilogue(ep);
    }
    if constexpr (OUT8) {
        if (p.amax) {
            // the wave's largest |y|, then one order-free atomic max per wave
            // (the bit patterns of non-negative floats order as the values)
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float o = __shfl_xor(amax_l, d);
                amax_l = o > amax_l ? o : amax_l;
            }
            if (lane == 0 && amax_l > 0.0f)
                __hip_atomic_fetch_max((uint32_t*)p.amax, __float_as_uint(amax_l), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (want_bgrad)
        bgrad_tile<BM, BN, WM, WN, C::FM, C::FN>(p, bg, (float*)smem, tm, tn, wm, wn, lane, tid, C::NT);
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


// MX instantiations: the 128 x 128 tile with four waves of 64 x 64 (tile 8).
// (The larger tiles were compiled too: with the block-scaled MFMA the
// compiler spills 500-1500 bytes per lane in every one of them -- the same
// code with the unscaled instruction does not -- so they are left out.)
template <int DOUT, int OPB>
Tile2Fn pick_tile2_mx(int tile_id) {
    if (tile_id == 8) return ge_tile2_kernel<GE_F8_E4M3, DOUT, OPB, 128, 128, 2, 2, 4, false, 64, false, true>;
    return nullptr;
}

template <int DOUT>
Tile2Fn pick_op2_mx(int op_b, int tile_id) {
    return op_b == GE_OP_T ? pick_tile2_mx<DOUT, GE_OP_T>(tile_id) : pick_tile2_mx<DOUT, GE_OP_N>(tile_id);
}

template <int DIN, int DOUT, int OPB>
Tile2Fn pick_tile2(int tile_id) {
    switch (tile_id) {
    case 5: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 256, 2, 2, 4, false, 64>;
    case 6: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 256, 2, 4, 4, false, 64>;
    case 7: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 128, 2, 2, 4, false, 64>;
    case 8: return ge_tile2_kernel<DIN, DOUT, OPB, 128, 128, 2, 2, 4, false, 64>;
    case 9: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 256, 2, 4, 2, true, 64>;
    case 10: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 256, 2, 2, 2, true, 64>;
    case 11: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 256, 2, 4, 2, false, 128>;
    case 12: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 256, 2, 2, 2, false, 128>;
    case 13:   // 16-bit inputs only (64-byte fp8 k rows have no swizzle here)
        if constexpr (Elem<DIN>::size == 2) return ge_tile2_kernel<DIN, DOUT, OPB, 64, 64, 2, 2, 4, false, 128>;
        else return nullptr;
    case 15: return ge_tile2_kernel<DIN, DOUT, OPB, 256, 128, 4, 2, 4, false, 64>;
    case 16:   // fp8 only: 256 x 256, 8 waves, 64-byte K steps (one sub-step each) in four stages
        if constexpr (Elem<DIN>::size == 1) return ge_tile2_kernel<DIN, DOUT, OPB, 256, 256, 2, 4, 4, false, 32>;
        else return nullptr;
    case 14:   // tile 13 with split-K
        if constexpr (Elem<DIN>::size == 2)
            return ge_tile2_kernel<DIN, DOUT, OPB, 64, 64, 2, 2, 4, false, 128, true>;
        else return nullptr;
    }
    return nullptr;
}

// fp8 output (E4M3 D): the 256 x 256 8-wave tile and the 128 x 128 tile for
// 16-bit inputs; the 256 x 256 tile with 64-byte steps, the 256 x 128 tile
// and the 128 x 128 tile for fp8 inputs
template <int DIN, int OPB>
Tile2Fn pick_tile2_out8(int tile_id) {
    if constexpr (Elem<DIN>::size == 2) {
        if (tile_id == 6) return ge_tile2_kernel<DIN, GE_F8_E4M3, OPB, 256, 256, 2, 4, 4, false, 64>;
    } else {
        if (tile_id == 15) return ge_tile2_kernel<DIN, GE_F8_E4M3, OPB, 256, 128, 4, 2, 4, false, 64>;
        if (tile_id == 16) return ge_tile2_kernel<DIN, GE_F8_E4M3, OPB, 256, 256, 2, 4, 4, false, 32>;
    }
    if (tile_id == 8) return ge_tile2_kernel<DIN, GE_F8_E4M3, OPB, 128, 128, 2, 2, 4, false, 64>;
    return nullptr;
}

template <int DIN>
Tile2Fn pick_op2_out8(int op_b, int tile_id) {
    return op_b == GE_OP_T ? pick_tile2_out8<DIN, GE_OP_T>(tile_id) : pick_tile2_out8<DIN, GE_OP_N>(tile_id);
}

template <int DIN, int DOUT>
Tile2Fn pick_op2(int op_b, int tile_id) {
    return op_b == GE_OP_T ? pick_tile2<DIN, DOUT, GE_OP_T>(tile_id) : pick_tile2<DIN, DOUT, GE_OP_N>(tile_id);
}

}  // namespace ge
