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
//    waves split the slice further.  Lane (r = lane % 16, q = lane / 16)
//    streams 16-byte chunks of W row n0 + r straight from global memory into
//    the A operand of v_mfma_f32_16x16x32_{f16,bf16}; the matching chunk of
//    x row r (L2-resident, read by every workgroup) is the B operand.  Each
//    lane's chunks for one MFMA step cover 32 consecutive K values of its row
//    together with the other three q lanes, so each step reads 64 contiguous
//    bytes per W row.
//  * Loads are issued `kUnroll` steps ahead of the MFMAs that consume them
//    (all of a wave's share of W at the batch-16 Linear shape), so the HBM
//    latency is paid once rather than once per batch.
//  * The waves' partial 16 x 16 blocks are reduced in LDS in a fixed order.
//    With split_k > 1 the per-slice sums go to an fp32 workspace and the last
//    workgroup to arrive for a column block (arrival counter, then a device-
//    scope fence) adds the slices in slice order, so results are
//    deterministic; it re-arms the counter for the next launch.  The bias,
//    activation, mask and the single store run once, after the full K sum.
#include <type_traits>

#include "ge_device.h"

namespace ge {

constexpr int kSmWaves = 8;
constexpr int kUnroll = 16;

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

template <int DIN, int DOUT>
__global__ void __launch_bounds__(kSmWaves * 64) ge_smallm_kernel(KernelArgs p_all) {
    const KernelArgs p = batch_slice<2, Elem<DOUT>::size>(p_all, blockIdx.y, p_all.n);   // this product
    __shared__ f32x4 red[kSmWaves][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, q = lane >> 4;
    const int nblk = blockIdx.x % p.tiles_n;   // column block
    const int slice = blockIdx.x / p.tiles_n;  // K slice
    const int n0 = nblk * 16;
    const int M = p.m, N = p.n, K = p.k;

    // this wave's K range: the slice split evenly over the waves, in steps of 32
    const int ks = slice * p.k_per_split;
    const int ke = min(K, ks + p.k_per_split);
    const int steps_total = (ke - ks + 31) / 32;
    const int per_wave = (steps_total + kSmWaves - 1) / kSmWaves;
    // Every workgroup reads all of x, so the waves of different workgroups
    // take the K sub-ranges in a rotated order: at any moment neighbouring
    // workgroups read different parts of x rather than all hitting the same
    // L2 lines.  Each output column's summation order is still fixed.
    const int wslot = (wave + nblk) % kSmWaves;
    const int s_begin = min(steps_total, wslot * per_wave);
    const int s_end = min(steps_total, s_begin + per_wave);
    const int s_full = min(s_end, (ke - ks) / 32);   // steps lying wholly below ke

    // Rows beyond n (of W) or m (of x) only feed outputs that are never
    // stored, so their addresses are clamped to the last valid row: the
    // full steps then need no bounds checks at all.
    const uint16_t* wrow = (const uint16_t*)p.B + (int64_t)min(n0 + r, N - 1) * p.ldb + ks + q * 8;
    const uint16_t* xrow = (const uint16_t*)p.A + (int64_t)min(r, M - 1) * p.lda + ks + q * 8;

    // the epilogue's bias values (wave 0 runs the epilogue): fetched now so
    // that their latency hides under the W stream instead of adding to the
    // end of the kernel
    const int ep = p.epilog;
    const bool has_bias = epilog_has_bias(ep);
    float bpre[4] = {0.f, 0.f, 0.f, 0.f};
    if (wave == 0 && has_bias) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + 4 * q + i;
            if (p.axis == GE_BIAS_COL) {
                if (n < N) bpre[i] = load_scalar<DOUT>(p.bias, n);
            } else if (r < M) {
                bpre[i] = load_scalar<DOUT>(p.bias, r);
            }
        }
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int s0 = s_begin;
    // U steps at once: all loads first (the scheduler would otherwise
    // trickle them out two per MFMA), then the MFMAs
    auto batch = [&](auto u_const) {
        constexpr int U = decltype(u_const)::value;
        u32x4 wv[U], xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wv[u] = __builtin_nontemporal_load((const u32x4*)(wrow + (s0 + u) * 32));
            xv[u] = *(const u32x4*)(xrow + (s0 + u) * 32);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) acc = mfma16<DIN, DOUT>(wv[u], xv[u], acc);
        s0 += U;
    };
    while (s0 + kUnroll <= s_full) batch(std::integral_constant<int, kUnroll>{});
    // the rest in descending power-of-two batches, never one load at a time
    // unless a single step is left
    if (s0 + 8 <= s_full) batch(std::integral_constant<int, 8>{});
    if (s0 + 4 <= s_full) batch(std::integral_constant<int, 4>{});
    if (s0 + 2 <= s_full) batch(std::integral_constant<int, 2>{});
    if (s0 < s_full) batch(std::integral_constant<int, 1>{});
    if (s_full >= s_begin && s_full < s_end) {
        // the ragged last step of the slice, if it falls in this wave's
        // range: elements at k >= ke are zero in both operands (0 * NaN
        // would not vanish)
        const int col = s_full * 32;
        const int lim = ke - ks - q * 8;
        const u32x4 wv = sm_load_masked(wrow, col, lim);
        const u32x4 xv = sm_load_masked(xrow, col, lim);
        acc = mfma16<DIN, DOUT>(wv, xv, acc);
    }
    // acc: lane holds rows n0 + 4q + i (i = 0..3) of column m = r of y^T
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    f32x4 sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < kSmWaves; ++w) sum += red[w][lane];

    if (p.split_k > 1) {
        // publish this slice's partial, then let the last arriver finish
        // The partials are written and read with device-scope atomic
        // accesses, which are coherent across the XCDs' separate L2s by
        // themselves.  A device-scope fence would do instead, but on this
        // chip it writes back and invalidates the whole L2 of the XCD, and
        // every other workgroup there then re-fetches x from memory.
        float* part = p.partial + ((int64_t)slice * p.tiles_n + nblk) * 256 + lane * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __hip_atomic_store(part + i, sum[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        sum = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int sl = 0; sl < p.split_k; ++sl) {
            float* ps = p.partial + ((int64_t)sl * p.tiles_n + nblk) * 256 + lane * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sum[i] += __hip_atomic_load(ps + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    float v[4];
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = n0 + 4 * q + i;
        float cb = 0.0f;   // the added input term beta * C
        if (beta != 0.0f && mok && n < N) cb = beta * load_scalar<DOUT>(p.cin, (int64_t)m * p.ldc + n);
        const float x = (sum[i] * s + cb) + bpre[i];
        if (want_aux && x > 0.0f && n < N) bits |= 1u << (4 * q + i);
        v[i] = activate(ep, x);
    }
    if (mok) {
        const int n = n0 + 4 * q;
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
        // 16 bits per row per column block: one half-word of the mask row
        bits |= (uint32_t)__shfl_xor((int)bits, 16);
        bits |= (uint32_t)__shfl_xor((int)bits, 32);
        uint16_t* aux16 = (uint16_t*)p.aux;
        const int64_t row_hw = (int64_t)p.ldaux * 2;   // half-words per mask row
        if (q == 0 && mok) aux16[(int64_t)m * row_hw + nblk] = (uint16_t)bits;
        // the last column block also clears the row's padding half-words
        if (nblk == p.tiles_n - 1 && q == 0 && mok) {
            for (int64_t hw = nblk + 1; hw < row_hw; ++hw) aux16[(int64_t)m * row_hw + hw] = 0;
        }
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

int launch_smallm(int a_type, int d_type, int op_b, const KernelArgs& args, unsigned grid, void* stream) {
    if (op_b != GE_OP_T) return (int)hipErrorInvalidDeviceFunction;
    SmFn fn = nullptr;
    if (a_type == GE_F16 && d_type == GE_F16) fn = ge_smallm_kernel<GE_F16, GE_F16>;
    else if (a_type == GE_F16 && d_type == GE_F32) fn = ge_smallm_kernel<GE_F16, GE_F32>;
    else if (a_type == GE_BF16 && d_type == GE_BF16) fn = ge_smallm_kernel<GE_BF16, GE_BF16>;
    else if (a_type == GE_BF16 && d_type == GE_F32) fn = ge_smallm_kernel<GE_BF16, GE_F32>;
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    hipLaunchKernelGGL(fn, dim3(grid, args.batch), dim3(kSmWaves * 64), 0, (hipStream_t)stream, args);
    return (int)hipGetLastError();
}

}  // namespace ge
