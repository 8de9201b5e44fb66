// ew_kernel.hip -- the second kernel of the unfused pair: D = act(C + bias)
// (+ ReLU sign mask or stored pre-activation), or D = C * f(aux) for the
// backward epilogues, reading back the product C that the first kernel (the
// tile or small-m kernel with no epilogue) stored in D's dtype.
//
// This is the separate elementwise pass that epilogue fusion removes (epilog
// page, first body paragraph: the two-kernel form writes the intermediate to
// memory and reads it back).  It exists to measure the fusion gain and to
// cross-check the fused kernels, so it is written to run at the memory's
// speed: HBM-bound, each lane owns 8 consecutive columns of a row (16 bytes
// of 16-bit D), neighbouring lanes own neighbouring chunks, so every load and
// store instruction of a wave covers 1 KiB of one row in whole 128-byte
// lines.  The 32 bits of a mask word come from four neighbouring lanes and
// are combined with two lane exchanges; the first lane of the four stores it.
#include "ge_device.h"

namespace ge {

constexpr int kEwThreads = 256;
constexpr int kEwUnroll = 2;   // chunks per thread: both loads go out before any use

// Work items per row: one per 8 columns, padded to a multiple of four (the
// 32 columns of one mask word) and, when the mask is written, to every word
// of the padded mask row (its padding words are cleared too).
__host__ __device__ inline int64_t ew_chunks_per_row(const KernelArgs& p) {
    if (p.epilog == GE_EPILOG_RELU_AUX_BIAS) return (int64_t)p.ldaux * 4;
    return ((int64_t)(p.n + 7) / 8 + 3) / 4 * 4;
}

template <int DT>
__global__ void __launch_bounds__(kEwThreads) ge_ew_kernel(KernelArgs p_all, const void* c_all) {
    // this product of a batch; its intermediate C sits at D's per-product offset
    const KernelArgs p = batch_slice(p_all, blockIdx.y);
    const void* c = (const uint8_t*)c_all + (int64_t)blockIdx.y * p_all.m * p_all.ldd * Elem<DT>::size;
    const int64_t cpr = ew_chunks_per_row(p);
    const int ep = p.epilog;
    const bool want_aux = ep == GE_EPILOG_RELU_AUX_BIAS;
    const bool want_pre = ep == GE_EPILOG_GELU_AUX_BIAS;
    const bool want_grad = epilog_is_grad(ep);
    const bool has_bias = epilog_has_bias(ep);
    const bool row_bias = p.axis == GE_BIAS_ROW;
    const float beta = p.cin ? *p.beta : 0.0f;
    const int64_t first = (int64_t)blockIdx.x * (kEwUnroll * kEwThreads) + threadIdx.x;

    int64_t row[kEwUnroll];
    int nc[kEwUnroll];
    bool live[kEwUnroll];
    float x[kEwUnroll][8];
    // all loads of C first
#pragma unroll
    for (int u = 0; u < kEwUnroll; ++u) {
        const int64_t t = first + u * kEwThreads;
        row[u] = t / cpr;
        nc[u] = (int)(t - row[u] * cpr) * 8;
        live[u] = row[u] < p.m && nc[u] < p.n;
        if (live[u]) {
            const int64_t idx = row[u] * p.ldd + nc[u];
            if (nc[u] + 8 <= p.n) {
                load8<DT>(c, idx, x[u]);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) x[u][j] = (nc[u] + j < p.n) ? load_scalar<DT>(c, idx + j) : 0.0f;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kEwUnroll; ++u) {
        uint32_t bits = 0;
        if (live[u]) {
            const int n0 = nc[u];
            const bool full = n0 + 8 <= p.n;
            float b[8], gf[8], cb[8];
            const float brow = (has_bias && row_bias) ? load_scalar<DT>(p.bias, row[u]) : 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = brow;
            if (has_bias && !row_bias) {
                if (full) load8<DT>(p.bias, n0, b);
                else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) b[j] = (n0 + j < p.n) ? load_scalar<DT>(p.bias, n0 + j) : 0.0f;
                }
            }
            if (want_grad) grad_factor8<DT>(p, ep, row[u], n0, gf);
#pragma unroll
            for (int j = 0; j < 8; ++j) cb[j] = 0.0f;
            if (beta != 0.0f) beta_c8<DT>(p, beta, row[u], n0, cb);   // beta = 0: C is not read
            float pre[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                pre[j] = (x[u][j] + cb[j]) + b[j];
                if (want_aux && pre[j] > 0.0f && n0 + j < p.n) bits |= 1u << j;
                x[u][j] = want_grad ? grad_apply(ep, pre[j], gf[j]) : activate(ep, pre[j]);
            }
            const int64_t idx = row[u] * p.ldd + n0;
            if (full) store8<DT>(p.D, idx, x[u]);
            else {
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (n0 + j < p.n) store_one<DT>(p.D, idx + j, x[u][j]);
            }
            if (want_pre) store_pre8<DT>(p, row[u], n0, pre);
        }
        if (want_aux) {
            // the four lanes of a mask word hold chunks g = 4w .. 4w+3 of one
            // row (the row length in chunks is a multiple of four, so a group
            // never straddles rows); every lane takes part in the exchange
            const int q = (int)((nc[u] >> 3) & 3);
            uint32_t word = bits << (8 * q);
            word |= (uint32_t)__shfl_xor((int)word, 1);
            word |= (uint32_t)__shfl_xor((int)word, 2);
            if (q == 0 && row[u] < p.m) p.aux[row[u] * p.ldaux + (nc[u] >> 5)] = word;
        }
    }
}

int launch_elementwise(int d_type, const KernelArgs& args, const void* c, void* stream) {
    const int64_t items = (int64_t)args.m * ew_chunks_per_row(args);
    const int64_t per_block = (int64_t)kEwUnroll * kEwThreads;
    const int64_t blocks = (items + per_block - 1) / per_block;
    if (blocks <= 0) return 0;
    if (blocks > 0x7fffffff) return (int)hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks, (unsigned)args.batch);
    switch (d_type) {
    case GE_F32:
        hipLaunchKernelGGL(ge_ew_kernel<GE_F32>, grid, dim3(kEwThreads), 0, (hipStream_t)stream, args, c);
        break;
    case GE_F16:
        hipLaunchKernelGGL(ge_ew_kernel<GE_F16>, grid, dim3(kEwThreads), 0, (hipStream_t)stream, args, c);
        break;
    case GE_BF16:
        hipLaunchKernelGGL(ge_ew_kernel<GE_BF16>, grid, dim3(kEwThreads), 0, (hipStream_t)stream, args, c);
        break;
    default:
        return (int)hipErrorInvalidDeviceFunction;
    }
    return (int)hipGetLastError();
}

// ---- bias gradient: partial sums and their reduction -----------------------------
// Unfused pair: sums of the stored D along the bias-gradient axis over blocks
// of 256 rows (COL: partial[rb * n + j]) or 256 columns (ROW: partial[cb * m + i]).
template <int DT>
__global__ void __launch_bounds__(256) ge_sum_kernel(KernelArgs p_all) {
    const KernelArgs p = batch_slice(p_all, blockIdx.z);   // this product
    const int idx = blockIdx.x * 256 + threadIdx.x;
    const int blk = blockIdx.y;
    if (p.axis == GE_BIAS_COL) {
        if (idx >= p.n) return;
        const int i1 = min(p.m, (blk + 1) * 256);
        float v = 0.0f;
        for (int i = blk * 256; i < i1; ++i) v += load_scalar<DT>(p.D, (int64_t)i * p.ldd + idx);
        p.partial[(int64_t)blk * p.n + idx] = v;
    } else {
        if (idx >= p.m) return;
        const int j1 = min(p.n, (blk + 1) * 256);
        float v = 0.0f;
        for (int j = blk * 256; j < j1; ++j) v += load_scalar<DT>(p.D, (int64_t)idx * p.ldd + j);
        p.partial[(int64_t)blk * p.m + idx] = v;
    }
}

// g[idx] = sum over t = 0 .. parts-1 of partial[t * len + idx], in that
// order, converted to D's dtype and written to the bias pointer (the
// gradient's output).  parts = 0 writes zeros (an empty sum).
template <int DT>
__global__ void __launch_bounds__(256) ge_bgrad_reduce(KernelArgs p_all, int parts) {
    const KernelArgs p = batch_slice(p_all, blockIdx.y);   // this product
    const int len = p.axis == GE_BIAS_COL ? p.n : p.m;
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= len) return;
    float v = 0.0f;
    for (int t = 0; t < parts; ++t) v += p.partial[(int64_t)t * len + idx];
    store_one<DT>((void*)p.bias, idx, v);
}

int launch_bgrad_sum(int d_type, const KernelArgs& args, int parts, void* stream) {
    const int len = args.axis == GE_BIAS_COL ? args.n : args.m;
    if (len <= 0 || parts <= 0) return 0;
    const dim3 grid((unsigned)((len + 255) / 256), (unsigned)parts, (unsigned)args.batch);
    switch (d_type) {
    case GE_F32: hipLaunchKernelGGL(ge_sum_kernel<GE_F32>, grid, dim3(256), 0, (hipStream_t)stream, args); break;
    case GE_F16: hipLaunchKernelGGL(ge_sum_kernel<GE_F16>, grid, dim3(256), 0, (hipStream_t)stream, args); break;
    case GE_BF16: hipLaunchKernelGGL(ge_sum_kernel<GE_BF16>, grid, dim3(256), 0, (hipStream_t)stream, args); break;
    default: return (int)hipErrorInvalidDeviceFunction;
    }
    return (int)hipGetLastError();
}

int launch_bgrad_reduce(int d_type, const KernelArgs& args, int parts, void* stream) {
    const int len = args.axis == GE_BIAS_COL ? args.n : args.m;
    if (len <= 0) return 0;
    const unsigned grid = (unsigned)((len + 255) / 256);
    switch (d_type) {
    case GE_F32:
        hipLaunchKernelGGL(ge_bgrad_reduce<GE_F32>, dim3(grid, args.batch), dim3(256), 0, (hipStream_t)stream, args, parts);
        break;
    case GE_F16:
        hipLaunchKernelGGL(ge_bgrad_reduce<GE_F16>, dim3(grid, args.batch), dim3(256), 0, (hipStream_t)stream, args, parts);
        break;
    case GE_BF16:
        hipLaunchKernelGGL(ge_bgrad_reduce<GE_BF16>, dim3(grid, args.batch), dim3(256), 0, (hipStream_t)stream, args, parts);
        break;
    default:
        return (int)hipErrorInvalidDeviceFunction;
    }
    return (int)hipGetLastError();
}

}  // namespace ge
