// ew_kernel.hip -- the second kernel of the unfused pair: D = act(C + bias)
// (+ ReLU sign mask or stored pre-activation), or D = C * f(aux) for the
// backward epilogues, reading back the product C that the first kernel (the
// tile or small-m kernel with no epilogue) stored in D's dtype.
//
// This is the separate elementwise pass that epilogue fusion removes (epilog
// page, first body paragraph: the two-kernel form writes the intermediate to
// memory and reads it back).  It exists to measure the fusion gain and to
// cross-check the fused kernels.  HBM-bound: one thread per 32 columns of a
// row (one mask word), 16-byte loads and stores.
#include "ge_device.h"

namespace ge {

// Work items per row: one per 32 columns, or per mask word when the mask is
// written (its padding words are cleared too).
__host__ __device__ inline int ew_items_per_row(const KernelArgs& p) {
    return p.epilog == GE_EPILOG_RELU_AUX_BIAS ? p.ldaux : (p.n + 31) / 32;
}

template <int DT>
__global__ void __launch_bounds__(256) ge_ew_kernel(KernelArgs p_all, const void* c_all) {
    // this product of a batch; its intermediate C sits at D's per-product offset
    const KernelArgs p = batch_slice<Elem<DT>::size, Elem<DT>::size>(p_all, blockIdx.y, 0);
    const void* c = (const uint8_t*)c_all + (int64_t)blockIdx.y * p_all.m * p_all.ldd * Elem<DT>::size;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int words = ew_items_per_row(p);
    const int64_t row = t / words;
    const int w = (int)(t - row * words);
    if (row >= p.m) return;
    const int n0 = w * 32;
    const int ep = p.epilog;
    const bool want_aux = ep == GE_EPILOG_RELU_AUX_BIAS;
    const bool want_pre = ep == GE_EPILOG_GELU_AUX_BIAS;
    const bool want_grad = epilog_is_grad(ep);
    if (n0 >= p.n) {
        if (want_aux) p.aux[row * p.ldaux + w] = 0u;   // row padding
        return;
    }
    const bool has_bias = epilog_has_bias(ep);
    const bool row_bias = p.axis == GE_BIAS_ROW;
    const float beta = p.cin ? *p.beta : 0.0f;
    const float brow = (has_bias && row_bias) ? load_scalar<DT>(p.bias, row) : 0.0f;
    uint32_t bits = 0;
    const int64_t base = row * p.ldd;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int nc = n0 + 8 * g;
        if (nc >= p.n) break;
        const bool full = nc + 8 <= p.n;
        float x[8], b[8], gf[8];
        if (full) {
            load8<DT>(c, base + nc, x);
            if (has_bias && !row_bias) load8<DT>(p.bias, nc, b);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                x[j] = (nc + j < p.n) ? load_scalar<DT>(c, base + nc + j) : 0.0f;
                b[j] = (has_bias && !row_bias && nc + j < p.n) ? load_scalar<DT>(p.bias, nc + j) : 0.0f;
            }
        }
        if (want_grad) grad_factor8<DT>(p, ep, row, nc, gf);
        float cb[8];   // the added input term beta * C
#pragma unroll
        for (int j = 0; j < 8; ++j) cb[j] = 0.0f;
        if (beta != 0.0f) beta_c8<DT>(p, beta, row, nc, cb);   // beta = 0: C is not read
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float pre = (x[j] + cb[j]) + (has_bias ? (row_bias ? brow : b[j]) : 0.0f);
            if (want_aux && pre > 0.0f && nc + j < p.n) bits |= 1u << (8 * g + j);
            x[j] = want_grad ? grad_apply(ep, pre, gf[j]) : activate(ep, pre);
            b[j] = pre;
        }
        if (full) store8<DT>(p.D, base + nc, x);
        else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (nc + j < p.n) store_one<DT>(p.D, base + nc + j, x[j]);
        }
        if (want_pre) store_pre8<DT>(p, row, nc, b);
    }
    if (want_aux) p.aux[row * p.ldaux + w] = bits;
}

int launch_elementwise(int d_type, const KernelArgs& args, const void* c, void* stream) {
    const int64_t items = (int64_t)args.m * ew_items_per_row(args);
    const unsigned grid = (unsigned)((items + 255) / 256);
    switch (d_type) {
    case GE_F32:
        hipLaunchKernelGGL(ge_ew_kernel<GE_F32>, dim3(grid, args.batch), dim3(256), 0, (hipStream_t)stream, args, c);
        break;
    case GE_F16:
        hipLaunchKernelGGL(ge_ew_kernel<GE_F16>, dim3(grid, args.batch), dim3(256), 0, (hipStream_t)stream, args, c);
        break;
    case GE_BF16:
        hipLaunchKernelGGL(ge_ew_kernel<GE_BF16>, dim3(grid, args.batch), dim3(256), 0, (hipStream_t)stream, args, c);
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
    const KernelArgs p = batch_slice<Elem<DT>::size, Elem<DT>::size>(p_all, blockIdx.z, 0);   // this product
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
    const KernelArgs p = batch_slice<Elem<DT>::size, Elem<DT>::size>(p_all, blockIdx.y, 0);   // this product
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
