// smallm_kernel.hip -- fused GEMM + epilogue for small batches (m <= 16),
// the bandwidth-bound Linear shape y = act(x W^T + b) with W given n x k.
//
// At m <= 16 every weight element is used at most 16 times, so the kernel is
// bound by streaming W from HBM once; the epilogue is fused as in the tile
// kernel (the small-batch, latency-sensitive case the nvmath page's
// paragraph on the BIAS epilog singles out; the NVGEMM page's
// Linear(4096,4096)+GELU example at batch 16).
//
// Design:
//  * One workgroup per 16 output columns (16 rows of W) and K slice; its
//    waves split the slice further, in spans of 64 K values (128 bytes of a
//    W row).  W is streamed straight from global memory into registers in
//    whole 128-byte lines: for each span, two load instructions cover the
//    16 rows, instruction j giving lane l the 16-byte chunk l/8 of row
//    8j + l%8 (8 lines per instruction).  The MFMA
//    v_mfma_f32_16x16x32_{f16,bf16} wants lane (r = lane % 16, q = lane / 16)
//    to hold row r, so a lane holds its own row's chunk 2q + r/8 in register
//    r/8 and row r^8's chunk in the other register.  Four MFMAs per span,
//    each with the lanes of one half zeroed, add the matching chunks of x
//    (the B operand: x row r, chunks 2q and 2q+1, L2-resident): two into the
//    lane's own row's sums and two into row r^8's, which a lane exchange
//    (lanes l and l^32 hold rows 4q+i and 4(q^2)+i) adds back at the end.
//    The MFMA work doubles, but the matrix cores are idle here anyway, while
//    half-line W requests (16 rows x 64 bytes per instruction) measured 8%
//    slower on the batch-16 Linear.
//  * x is read in the same whole-line pattern (every workgroup reads all of
//    x from L2, as many bytes as its W slab, so x's request count matters as
//    much as W's).  A lane then holds its own row's chunk in one register
//    and row r^8's in the other; one exchange with lane r^8 (a DPP rotation
//    by 8 within each row of 16 lanes) gives every lane both chunks 2q and
//    2q + 1 of x row r, the layout the MFMA's B operand takes.
//  * All of a wave's loads (up to 8 spans of W and x, the whole share at the
//    batch-16 Linear shape) go out before its MFMAs, so the HBM latency is
//    paid once rather than once per span.
//  * The waves' partial 16 x 16 blocks are reduced in LDS in a fixed order.
//    With split_k > 1 each slice publishes its sum to an fp32 workspace with
//    device-scope atomic stores, waits until they have completed (vmcnt(0)),
//    then counts its arrival with a device-scope atomic add; the workgroup
//    that sees the last count reads every slice back with device-scope
//    atomic loads and adds them in slice order, so results are
//    deterministic, and re-arms the counter.  No cache-wide fence is used.
//    The bias, activation, mask and the single store run once, after the
//    full K sum.
#include <type_traits>

#include "ge_device.h"

namespace ge {

constexpr int kSmWaves = 8;

// zeros read in place of the bias by the epilogues that add none
__device__ const uint32_t kSmZeros[4] = {0u, 0u, 0u, 0u};
constexpr int kUnroll = 8;   // spans of 64 K values per load batch

template <int DIN, int DOUT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (DIN == GE_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 16-byte chunk of 8 16-bit elements starting at column `col` of a row,
// elements at col + e >= ncols read as zero (the ragged K step only).
__device__ __forceinline__ u32x4 sm_load_masked(const uint16_t* row, int col, int ncols) {
    if (col >= ncols) return u32x4{0, 0, 0, 0};
    if (col + 8 <= ncols) return *(const u32x4*)(row + col);
    uint16_t t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = (col + e < ncols) ? row[col + e] : (uint16_t)0;
    u32x4 r;
    __builtin_memcpy(&r, t, 16);
    return r;
}

template <int DIN, int DOUT, int RG>
__global__ void __launch_bounds__(kSmWaves * 64) ge_smallm_kernel(KernelArgs p_all) {
    const KernelArgs p = batch_slice(p_all, blockIdx.y);   // this product
    __shared__ f32x4 red[kSmWaves][RG][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int nblk = blockIdx.x % p.tiles_n;   // column block: RG groups of 16 W rows
    const int slice = blockIdx.x / p.tiles_n;  // K slice
    const int n0 = nblk * 16 * RG;
    const int M = p.m, N = p.n, K = p.k;

    // this wave's K range: the slice split evenly over the waves, in spans
    // of 64 (the slice starts on a span boundary: k_per_split is a multiple
    // of 64)
    const int ks = slice * p.k_per_split;
    const int ke = min(K, ks + p.k_per_split);
    const int spans_total = (ke - ks + 63) / 64;
    const int per_wave = (spans_total + kSmWaves - 1) / kSmWaves;
    // Every workgroup reads all of x, so the waves of different workgroups
    // take the K sub-ranges in a rotated order: at any moment neighbouring
    // workgroups read different parts of x rather than all hitting the same
    // L2 lines.  Each output column's summation order is still fixed.
    const int wslot = (wave + nblk) % kSmWaves;
    const int s_begin = min(spans_total, wslot * per_wave);
    const int s_end = min(spans_total, s_begin + per_wave);
    const int s_full = min(s_end, (ke - ks) / 64);   // spans lying wholly below ke

    // Rows beyond n (of W) or m (of x) only feed outputs that are never
    // stored, so their addresses are clamped to the last valid row: the
    // full spans then need no bounds checks at all.
    const int wr = lane & 7, wc = lane >> 3;   // full-line loads: row 8j + wr, chunk wc
    const uint16_t* w0row[RG];
    const uint16_t* w1row[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        w0row[g] = (const uint16_t*)p.B + (int64_t)min(n0 + 16 * g + wr, N - 1) * p.ldb + ks + wc * 8;
        w1row[g] = (const uint16_t*)p.B + (int64_t)min(n0 + 16 * g + 8 + wr, N - 1) * p.ldb + ks + wc * 8;
    }
    const uint16_t* x0row = (const uint16_t*)p.A + (int64_t)min(wr, M - 1) * p.lda + ks + wc * 8;
    const uint16_t* x1row = (const uint16_t*)p.A + (int64_t)min(8 + wr, M - 1) * p.lda + ks + wc * 8;

    // the epilogue's bias values: fetched now so that their latency hides
    // under the W stream instead of adding to the end of the kernel.  The
    // loads are unconditional, with clamped indices (values for columns
    // beyond n or rows beyond m feed outputs that are never stored): a load
    // under a per-element branch makes the compiler wait for it on the spot,
    // which held every wave's W stream back by the bias loads' latency.
    // (The raw elements are kept and converted in the epilogue, so that
    // nothing uses them before then.)
    const int ep = p.epilog;
    const bool has_bias = epilog_has_bias(ep);
    // (No branch either: without a bias the loads read zeros from kSmZeros,
    // so nothing has to be merged, and waited for, where the paths join.)
    // (Both candidates cast to the global address space: a select between a
    // generic pointer and the device array would make these flat loads,
    // which the compiler then waits for everywhere.)
    typedef typename Elem<DOUT>::T BiasT;
    typedef __attribute__((address_space(1))) const BiasT GlobalBiasT;
    GlobalBiasT* bp = has_bias ? (GlobalBiasT*)p.bias : (GlobalBiasT*)kSmZeros;
    BiasT braw[RG][4];
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            braw[g][i] = bp[!has_bias ? 0
                            : p.axis == GE_BIAS_COL ? min(n0 + 16 * g + 4 * q + i, N - 1)
                                                    : min(r, M - 1)];
    __builtin_amdgcn_sched_barrier(0);   // issued here, not sunk to the epilogue

    // per row group: accd, sums of the lane's own row (labels 4q + i); accs,
    // of row r ^ 8
    f32x4 accd[RG], accs[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        accd[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        accs[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const bool rlo = r < 8;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // x rows 0-7 (x0) and 8-15 (x1) as loaded: lane r < 8 holds row r's
    // chunk 2q in x0, lane r >= 8 row r's chunk 2q + 1 in x1; each sends the
    // other register to lane r ^ 8 and takes the missing chunk from it
    auto x_operands = [&](const u32x4& x0, const u32x4& x1, u32x4& xe, u32x4& xo)
                          __attribute__((always_inline)) {
        u32x4 got;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            got[i] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(rlo ? x1[i] : x0[i]), 0x128, 0xf, 0xf, false);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xe[i] = rlo ? x0[i] : got[i];
            xo[i] = rlo ? got[i] : x1[i];
        }
    };
    // one span of one row group: four MFMAs, each with half the lanes of W
    // zeroed, add every chunk into its row's sums
    auto group_mfmas = [&](int g, const u32x4& w0, const u32x4& w1, const u32x4& xe, const u32x4& xo)
                           __attribute__((always_inline)) {
        accd[g] = mfma16<DIN, DOUT>(rlo ? w0 : zero, xe, accd[g]);   // rows 0-7, even chunks
        accd[g] = mfma16<DIN, DOUT>(rlo ? zero : w1, xo, accd[g]);   // rows 8-15, odd chunks
        accs[g] = mfma16<DIN, DOUT>(rlo ? w1 : zero, xe, accs[g]);   // rows 8-15 (as r^8), even chunks
        accs[g] = mfma16<DIN, DOUT>(rlo ? zero : w0, xo, accs[g]);   // rows 0-7 (as r^8), odd chunks
    };
    int s0 = s_begin;
    // U spans at once: all loads first (the scheduler would otherwise
    // trickle them out between the MFMAs), then the MFMAs
    auto batch = [&](auto u_const) __attribute__((always_inline)) {
        constexpr int U = decltype(u_const)::value;
        u32x4 w0[U][RG], w1[U][RG], x0[U], x1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int off = (s0 + u) * 64;
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                w0[u][g] = __builtin_nontemporal_load((const u32x4*)(w0row[g] + off));
                w1[u][g] = __builtin_nontemporal_load((const u32x4*)(w1row[g] + off));
            }
            x0[u] = *(const u32x4*)(x0row + off);
            x1[u] = *(const u32x4*)(x1row + off);
        }
        __builtin_amdgcn_sched_barrier(0);
        // span by span, so that each waits only for its own loads
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4 xe, xo;
            x_operands(x0[u], x1[u], xe, xo);
#pragma unroll
            for (int g = 0; g < RG; ++g) group_mfmas(g, w0[u][g], w1[u][g], xe, xo);
            __builtin_amdgcn_sched_barrier(0);
        }
        s0 += U;
    };
    // spans per load batch: the W registers of a batch stay at 8 spans of
    // one row group's worth
    constexpr int kUnrollRG = kUnroll / RG;
    while (s0 + kUnrollRG <= s_full) batch(std::integral_constant<int, kUnrollRG>{});
    // the rest in descending power-of-two batches, never one load at a time
    // unless a single span is left
    if constexpr (kUnrollRG > 4)
        if (s0 + 4 <= s_full) batch(std::integral_constant<int, 4>{});
    if constexpr (kUnrollRG > 2)
        if (s0 + 2 <= s_full) batch(std::integral_constant<int, 2>{});
    if constexpr (kUnrollRG > 1)
        if (s0 < s_full) batch(std::integral_constant<int, 1>{});
    if (s_full >= s_begin && s_full < s_end) {
        // the ragged last span of the slice, if it falls in this wave's
        // range: elements at k >= ke are zero in both operands (0 * NaN
        // would not vanish)
        const int col = s_full * 64;
        const int lim = ke - ks;
        const u32x4 x0 = sm_load_masked(x0row - wc * 8, col + wc * 8, lim);
        const u32x4 x1 = sm_load_masked(x1row - wc * 8, col + wc * 8, lim);
        u32x4 xe, xo;
        x_operands(x0, x1, xe, xo);
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const u32x4 w0 = sm_load_masked(w0row[g] - wc * 8, col + wc * 8, lim);
            const u32x4 w1 = sm_load_masked(w1row[g] - wc * 8, col + wc * 8, lim);
            group_mfmas(g, w0, w1, xe, xo);
        }
    }
    // row r^8's sums live in lane l^32 (labels 4q + i and 4(q^2) + i);
    // acc: lane holds rows n0 + 16g + 4q + i (i = 0..3) of column m = r of y^T
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = accd[g][i] + __shfl_xor(accs[g][i], 32);
        red[wave][g][lane] = acc;
    }
    __syncthreads();
    if (wave != 0) return;
    f32x4 sum[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        sum[g] = red[0][g][lane];
#pragma unroll
        for (int w = 1; w < kSmWaves; ++w) sum[g] += red[w][g][lane];
    }

    if (p.split_k > 1) {
        // publish this slice's partial, then let the last arriver finish
        // The partials are written and read with device-scope atomic
        // accesses, which are coherent across the XCDs' separate L2s by
        // themselves.  A device-scope fence would do instead, but on this
        // chip it writes back and invalidates the whole L2 of the XCD, and
        // every other workgroup there then re-fetches x from memory.
        // (element i of lane l at i * 64 + l: each store covers 256
        // contiguous bytes)
        float* part = p.partial + ((int64_t)slice * p.tiles_n + nblk) * 256 * RG + lane;
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __hip_atomic_store(part + g * 256 + i * 64, sum[g][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // every lane's stores complete (performed at device scope) before
        // the arrival is counted; the clobber keeps the compiler from
        // moving either across the wait
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int prev = 0;
        if (lane == 0)
            prev = (int)__hip_atomic_fetch_add(&p.counters[nblk], 1u, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        prev = __shfl(prev, 0);
        if (prev != p.split_k - 1) return;
        // the loads below depend on the counter's value, so they issue only
        // after every other slice's stores have been performed (the clobber
        // stops the compiler from hoisting them above the branch)
        asm volatile("" ::: "memory");
#pragma unroll
        for (int g = 0; g < RG; ++g) sum[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int sl = 0; sl < p.split_k; ++sl) {
            float* ps = p.partial + ((int64_t)sl * p.tiles_n + nblk) * 256 * RG + lane;
#pragma unroll
            for (int g = 0; g < RG; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sum[g][i] += __hip_atomic_load(ps + g * 256 + i * 64, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        if (lane == 0) p.counters[nblk] = 0u;   // re-arm for the next launch
    }

    const bool want_aux = ep == GE_EPILOG_RELU_AUX_BIAS;
    float s = 1.0f;   // the product's scale (alpha)
    if (p.scale_a) s *= *p.scale_a;
    if (p.scale_b) s *= *p.scale_b;
    const int m = r;
    const bool mok = m < M;
    const float beta = p.cin ? *p.beta : 0.0f;   // beta = 0: C is not read
    uint16_t* aux16 = (uint16_t*)p.aux;
    const int64_t row_hw = (int64_t)p.ldaux * 2;   // half-words per mask row
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int ng = n0 + 16 * g;   // this group's first column
        float v[4];
        uint32_t bits = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = ng + 4 * q + i;
            float cb = 0.0f;   // the added input term beta * C
            if (beta != 0.0f && mok && n < N) cb = beta * load_scalar<DOUT>(p.cin, (int64_t)m * p.ldc + n);
            float bv = 0.0f;
            if constexpr (DOUT == GE_F32) bv = braw[g][i];
            else if constexpr (DOUT == GE_BF16) bv = bf16_bits_to_f32(braw[g][i]);
            else bv = f16_bits_to_f32(braw[g][i]);
            const float x = (sum[g][i] * s + cb) + bv;
            if (want_aux && x > 0.0f && n < N) bits |= 1u << (4 * q + i);
            v[i] = activate(ep, x);
        }
        if (mok) {
            const int n = ng + 4 * q;
            const int64_t idx = (int64_t)m * p.ldd + n;
            if (n + 4 <= N) {
                if constexpr (DOUT == GE_F32) {
                    *(f32x4*)((float*)p.D + idx) = f32x4{v[0], v[1], v[2], v[3]};
                } else {
                    uint32_t lo, hi;
                    if constexpr (DOUT == GE_BF16) {
                        lo = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
                        hi = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
                    } else {
                        lo = f32_to_f16_bits(v[0]) | ((uint32_t)f32_to_f16_bits(v[1]) << 16);
                        hi = f32_to_f16_bits(v[2]) | ((uint32_t)f32_to_f16_bits(v[3]) << 16);
                    }
                    *(u32x2*)((uint16_t*)p.D + idx) = u32x2{lo, hi};
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n + i < N) store_one<DOUT>(p.D, idx + i, v[i]);
            }
        }
        if (want_aux) {
            // 16 bits per row per group of 16 columns: one half-word of the
            // mask row (groups wholly beyond n store zeros; every group lies
            // below the row's 128-column padding)
            bits |= (uint32_t)__shfl_xor((int)bits, 16);
            bits |= (uint32_t)__shfl_xor((int)bits, 32);
            if (q == 0 && mok) aux16[(int64_t)m * row_hw + nblk * RG + g] = (uint16_t)bits;
        }
    }
    // the last column block also clears the row's padding half-words
    if (want_aux && nblk == p.tiles_n - 1 && q == 0 && mok) {
        for (int64_t hw = (int64_t)(nblk + 1) * RG; hw < row_hw; ++hw) aux16[(int64_t)m * row_hw + hw] = 0;
    }
}

// Clear the split-K arrival counters before a launch.  A kernel rather than
// hipMemsetAsync, so that a caller may capture execute() into a HIP graph.
__global__ void __launch_bounds__(256) ge_clear_u32(uint32_t* p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

int launch_clear_counters(uint32_t* p, int n, void* stream) {
    if (n <= 0) return 0;
    hipLaunchKernelGGL(ge_clear_u32, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, p, n);
    return (int)hipGetLastError();
}

typedef void (*SmFn)(KernelArgs);

template <int RG>
SmFn pick_smallm(int a_type, int d_type) {
    if (a_type == GE_F16 && d_type == GE_F16) return ge_smallm_kernel<GE_F16, GE_F16, RG>;
    if (a_type == GE_F16 && d_type == GE_F32) return ge_smallm_kernel<GE_F16, GE_F32, RG>;
    if (a_type == GE_BF16 && d_type == GE_BF16) return ge_smallm_kernel<GE_BF16, GE_BF16, RG>;
    if (a_type == GE_BF16 && d_type == GE_F32) return ge_smallm_kernel<GE_BF16, GE_F32, RG>;
    return nullptr;
}

int launch_smallm(int a_type, int d_type, int op_b, int rg, const KernelArgs& args, unsigned grid, void* stream) {
    if (op_b != GE_OP_T) return (int)hipErrorInvalidDeviceFunction;
    const SmFn fn = rg == 1 ? pick_smallm<1>(a_type, d_type)
                    : rg == 2 ? pick_smallm<2>(a_type, d_type)
                    : rg == 4 ? pick_smallm<4>(a_type, d_type)
                              : nullptr;
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    hipLaunchKernelGGL(fn, dim3(grid, args.batch), dim3(kSmWaves * 64), 0, (hipStream_t)stream, args);
    return (int)hipGetLastError();
}

}  // namespace ge
