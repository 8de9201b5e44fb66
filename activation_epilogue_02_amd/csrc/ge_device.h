// ge_device.h -- device-side helpers shared by the gfx950 kernels: vector
// types, element-type traits, output conversion and the epilogue activations.
//
// Pages cited: see include/gemm_epilog.h for the page list.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ge_params.h"

namespace ge {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Element-type traits, indexed by the ABI's ge_dtype value.
template <int DT> struct Elem;
template <> struct Elem<GE_F32>     { typedef float    T; static constexpr int size = 4; };
template <> struct Elem<GE_F16>     { typedef uint16_t T; static constexpr int size = 2; };
template <> struct Elem<GE_BF16>    { typedef uint16_t T; static constexpr int size = 2; };
template <> struct Elem<GE_F8_E4M3> { typedef uint8_t  T; static constexpr int size = 1; };

// ---- reading scalars of an output-typed vector (bias) ----------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
    return __uint_as_float(b << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
    _Float16 h;
    uint16_t s = (uint16_t)b;
    __builtin_memcpy(&h, &s, 2);
    return (float)h;
}

template <int DT>
__device__ __forceinline__ float load_scalar(const void* p, int64_t i) {
    if constexpr (DT == GE_F32) return ((const float*)p)[i];
    else if constexpr (DT == GE_BF16) return bf16_bits_to_f32(((const uint16_t*)p)[i]);
    else return f16_bits_to_f32(((const uint16_t*)p)[i]);
}

// ---- fp32 -> output conversion, round to nearest even -----------------------
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 b = (__bf16)x;  // gfx950: hardware RNE conversion
    uint16_t r;
    __builtin_memcpy(&r, &b, 2);
    return r;
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    _Float16 h = (_Float16)x;  // RNE (default rounding mode)
    uint16_t r;
    __builtin_memcpy(&r, &h, 2);
    return r;
}

// fp32 -> OCP E4M3 (E4 M3, bias 7, no infinities, 0x7F = NaN), round to
// nearest even, saturating: magnitudes that round above the largest finite
// value 448 (and infinities) give +-448, NaN gives 0x7F with the sign.
// Written from the format definition: the quantum is 2^(e-3) for a value in
// [2^e, 2^(e+1)), e >= -6, and the subnormal quantum 2^-9 below 2^-6.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = __builtin_fabsf(x);
    if (!(a == a)) return sign | 0x7fu;
    if (a >= 448.0f) return sign | 0x7eu;   // ties at 464 round to 448 too
    int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
    if (e < -6) e = -6;
    int n = (int)__builtin_rintf(__builtin_ldexpf(a, 3 - e));   // exact scaling, RNE
    if (n >= 16) {   // carried into the next binade
        n >>= 1;
        e += 1;
    }
    const uint32_t code = n < 8 ? (uint32_t)n : ((uint32_t)(e + 7) << 3) | (uint32_t)(n - 8);
    return sign | code;
}

// Pack 8 fp32 values into 16 bytes of 16-bit outputs.
template <int DT>
__device__ __forceinline__ u32x4 pack8_16bit(const float* v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo, hi;
        if constexpr (DT == GE_BF16) {
            lo = f32_to_bf16_bits(v[2 * i]);
            hi = f32_to_bf16_bits(v[2 * i + 1]);
        } else {
            lo = f32_to_f16_bits(v[2 * i]);
            hi = f32_to_f16_bits(v[2 * i + 1]);
        }
        r[i] = lo | (hi << 16);
    }
    return r;
}

// Store one converted element.
template <int DT>
__device__ __forceinline__ void store_one(void* D, int64_t idx, float v) {
    if constexpr (DT == GE_F8_E4M3) ((uint8_t*)D)[idx] = (uint8_t)f32_to_e4m3_sat(v);
    else if constexpr (DT == GE_F32) ((float*)D)[idx] = v;
    else if constexpr (DT == GE_BF16) ((uint16_t*)D)[idx] = f32_to_bf16_bits(v);
    else ((uint16_t*)D)[idx] = f32_to_f16_bits(v);
}

// Store 8 consecutive converted elements (16-byte aligned for 16-bit types,
// 32-byte span for fp32).
template <int DT>
__device__ __forceinline__ void store8(void* D, int64_t idx, const float* v) {
    if constexpr (DT == GE_F8_E4M3) {   // 8 bytes
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo |= f32_to_e4m3_sat(v[i]) << (8 * i);
            hi |= f32_to_e4m3_sat(v[4 + i]) << (8 * i);
        }
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        *(u32x2_t*)((uint8_t*)D + idx) = u32x2_t{lo, hi};
    } else if constexpr (DT == GE_F32) {
        u32x4 a, b;
#pragma unroll
        for (int i = 0; i < 4; ++i) { a[i] = __float_as_uint(v[i]); b[i] = __float_as_uint(v[4 + i]); }
        u32x4* p = (u32x4*)((float*)D + idx);
        p[0] = a;
        p[1] = b;
    } else {
        *(u32x4*)((uint16_t*)D + idx) = pack8_16bit<DT>(v);
    }
}

// Load 8 consecutive bias values (aligned as store8).
template <int DT>
__device__ __forceinline__ void load8(const void* p, int64_t idx, float* v) {
    if constexpr (DT == GE_F32) {
        const u32x4* q = (const u32x4*)((const float*)p + idx);
        u32x4 a = q[0], b = q[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) { v[i] = __uint_as_float(a[i]); v[4 + i] = __uint_as_float(b[i]); }
    } else {
        u32x4 a = *(const u32x4*)((const uint16_t*)p + idx);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (DT == GE_BF16) {
                v[2 * i] = bf16_bits_to_f32(a[i] & 0xffffu);
                v[2 * i + 1] = bf16_bits_to_f32(a[i] >> 16);
            } else {
                v[2 * i] = f16_bits_to_f32(a[i] & 0xffffu);
                v[2 * i + 1] = f16_bits_to_f32(a[i] >> 16);
            }
        }
    }
}

// ---- direct global -> LDS copies ---------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;

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

// The same copy with its global address split into a wave-uniform 64-bit
// base (SGPRs) and a 32-bit unsigned per-lane byte offset: advancing the
// copy along K is then one scalar add per step instead of a 64-bit vector
// add per copy in every lane.
__device__ __forceinline__ void copy_to_lds16_sb(uint32_t voff, const void* sbase, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory", "m0");
}

// The same with 4 bytes per lane (global_load_lds_dword): lane l's word
// lands at M0 + 4*l; the global address must be 4-byte aligned.
__device__ __forceinline__ void copy_to_lds4(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
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

// ---- activations -------------------------------------------------------------
// GELU in its tanh form, 0.5 x (1 + tanh(u)) with u = sqrt(2/pi)(x + 0.044715 x^3).
// Since 0.5 (1 + tanh u) = 1 / (1 + e^{-2u}), this is x / (1 + 2^{-2u log2 e}),
// evaluated with the hardware base-2 exponential and reciprocal (v_exp_f32,
// v_rcp_f32).  Large |u| saturates correctly: e^{-2u} -> inf gives -0/+0,
// e^{-2u} -> 0 gives x.
__device__ __forceinline__ float gelu_tanh(float x) {
    const float k0 = 0.7978845608028654f;          // sqrt(2/pi)
    const float k1 = 0.044715f;
    const float m2log2e = -2.0f * 1.4426950408889634f;
    float u = k0 * (x + k1 * x * x * x);
    float e = __builtin_amdgcn_exp2f(m2log2e * u);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// GELU'(x) of the same tanh form.  With g = 0.5 (1 + tanh u) = 1 / (1 + e^{-2u})
// and 1 - tanh^2 u = 4 g (1 - g), the product and chain rules give
// GELU'(x) = g + 2 x g (1 - g) u'(x), u'(x) = sqrt(2/pi) (1 + 3 * 0.044715 x^2).
// Saturates like gelu_tanh: g -> 0 gives 0, g -> 1 gives 1.
__device__ __forceinline__ float gelu_tanh_deriv(float x) {
    const float k0 = 0.7978845608028654f;          // sqrt(2/pi)
    const float k1 = 0.044715f;
    const float m2log2e = -2.0f * 1.4426950408889634f;
    const float x2 = x * x;
    const float u = k0 * (x + k1 * x2 * x);
    const float g = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(m2log2e * u));
    const float du = k0 * (1.0f + 3.0f * k1 * x2);
    return g + 2.0f * x * g * (1.0f - g) * du;
}

// Epilogues that add a bias to the product (DRELU and DGELU take none).
__host__ __device__ __forceinline__ bool epilog_has_bias(int epilog) {
    return epilog == GE_EPILOG_BIAS || epilog == GE_EPILOG_RELU_BIAS || epilog == GE_EPILOG_RELU_AUX_BIAS ||
           epilog == GE_EPILOG_GELU_BIAS || epilog == GE_EPILOG_GELU_AUX_BIAS || epilog == GE_EPILOG_TANH_BIAS;
}

// Backward epilogues (the product scaled by an activation derivative read
// from aux), and those of them that also return the bias gradient.
__host__ __device__ __forceinline__ bool epilog_is_grad(int epilog) {
    return epilog == GE_EPILOG_DRELU || epilog == GE_EPILOG_DGELU || epilog == GE_EPILOG_DRELU_BGRAD ||
           epilog == GE_EPILOG_DGELU_BGRAD;
}
__host__ __device__ __forceinline__ bool epilog_is_bgrad(int epilog) {
    return epilog == GE_EPILOG_DRELU_BGRAD || epilog == GE_EPILOG_DGELU_BGRAD;
}
__host__ __device__ __forceinline__ bool epilog_reads_mask(int epilog) {
    return epilog == GE_EPILOG_DRELU || epilog == GE_EPILOG_DRELU_BGRAD;
}

// Apply the activation of an epilogue to a pre-activation value.  The
// backward epilogues pass the product through; their factor comes from
// grad_factor8.
__device__ __forceinline__ float activate(int epilog, float x) {
    if (epilog == GE_EPILOG_RELU_BIAS || epilog == GE_EPILOG_RELU_AUX_BIAS) return x > 0.0f ? x : 0.0f;
    if (epilog == GE_EPILOG_GELU_BIAS || epilog == GE_EPILOG_GELU_AUX_BIAS) return gelu_tanh(x);
    if (epilog == GE_EPILOG_TANH_BIAS) return tanhf(x);   // the device library's tanh: once per output
    return x;
}

// The backward factor of DRELU (the mask bit RELU_AUX_BIAS wrote) or DGELU
// (GELU' of the pre-activation GELU_AUX_BIAS wrote) for the 8 columns
// nc .. nc+7 of row m (nc a multiple of 8, m < m of the problem).  Columns at
// or beyond n get 0 and are never read: the aux rows are only padded to 128
// columns, while a tile may reach further.
template <int DOUT>
__device__ __forceinline__ void grad_factor8(const KernelArgs& p, int epilog, int64_t m, int nc, float* f) {
    if (nc >= p.n) {
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = 0.0f;
        return;
    }
    if (epilog_reads_mask(epilog)) {
        const uint32_t w = p.aux[m * p.ldaux + (nc >> 5)] >> (nc & 31);
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = ((w >> j) & 1u) ? 1.0f : 0.0f;
        return;
    }
    float pre[8];
    const int64_t idx = m * p.ldaux + nc;
    if (nc + 8 <= p.n) {
        load8<DOUT>(p.aux, idx, pre);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) pre[j] = (nc + j < p.n) ? load_scalar<DOUT>(p.aux, idx + j) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = gelu_tanh_deriv(pre[j]);
}

// Apply the backward factor: DGELU multiplies; DRELU selects (C or +0), so
// that a masked entry is exactly zero whatever C holds (-0, inf, NaN).
__device__ __forceinline__ float grad_apply(int epilog, float x, float f) {
    return epilog_reads_mask(epilog) ? (f != 0.0f ? x : 0.0f) : x * f;
}

// ---- bias gradient (DRELU_BGRAD, DGELU_BGRAD) --------------------------------
// The tile kernels sum their fp32 outputs along the bias-gradient axis: COL
// (the bias was added to every row: g[j] = sum_i D[i][j]) gives per-column
// sums over the tile's rows, ROW (g[i] = sum_j D[i][j]) per-row sums over its
// columns.  Each lane adds what it computed; the lanes sharing a column (COL)
// or row (ROW) and then the waves sharing it are summed in a fixed order, and
// the tile writes its partial to partial[t * len + idx] (t the tile's row
// index for COL, column index for ROW; len = n or m).  A second kernel sums
// the partials over t in order, so the result is deterministic.
template <int FM, int FN>
struct BgradAcc {
    float col[FN][2][8];   // COL: columns nb + 16g + 8h + j of fragment column fn
    float row[FM];         // ROW: the lane's row of fragment row fm
    __device__ __forceinline__ void clear() {
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int j = 0; j < 8; ++j) col[f][g][j] = 0.0f;
#pragma unroll
        for (int f = 0; f < FM; ++f) row[f] = 0.0f;
    }
};

// Reduce a tile's sums and write its partial.  smem holds at least
// max(WM*BN, WN*BM) floats and is free once every wave passed the first
// barrier here; every thread of the workgroup must call this.
template <int BM, int BN, int WM, int WN, int FM, int FN>
__device__ __forceinline__ void bgrad_tile(const KernelArgs& p, BgradAcc<FM, FN>& acc, float* red, int tm, int tn,
                                           int wm, int wn, int lane, int tid, int nthreads) {
    constexpr int TM = BM / WM, TN = BN / WN;
    const int r32 = lane & 31, h = lane >> 5;
    const bool col_axis = p.axis == GE_BIAS_COL;
    __syncthreads();   // every wave is done with the LDS stages
    if (col_axis) {
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float v = acc.col[f][g][j];
#pragma unroll
                    for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o);   // the 32 rows of a half
                    if (r32 == 0) red[wm * BN + wn * TN + f * 32 + 16 * g + 8 * h + j] = v;
                }
    } else {
#pragma unroll
        for (int f = 0; f < FM; ++f) {
            const float v = acc.row[f] + __shfl_xor(acc.row[f], 32);   // both column halves
            if (h == 0) red[wn * BM + wm * TM + f * 32 + r32] = v;
        }
    }
    __syncthreads();
    if (col_axis) {
        for (int c = tid; c < BN; c += nthreads) {
            const int n = tn * BN + c;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < WM; ++w) v += red[w * BN + c];
            if (n < p.n) p.partial[(int64_t)tm * p.n + n] = v;
        }
    } else {
        for (int r = tid; r < BM; r += nthreads) {
            const int m = tm * BM + r;
            float v = 0.0f;
#pragma unroll
            for (int w = 0; w < WN; ++w) v += red[w * BM + r];
            if (m < p.m) p.partial[(int64_t)tn * p.m + m] = v;
        }
    }
}

// The added input term beta * C for the 8 columns nc .. nc+7 of row m
// (nc a multiple of 8, m within the problem); columns at or beyond n get 0.
template <int DOUT>
__device__ __forceinline__ void beta_c8(const KernelArgs& p, float beta, int64_t m, int nc, float* cb) {
    const int64_t idx = m * p.ldc + nc;
    if (nc + 8 <= p.n) {
        load8<DOUT>(p.cin, idx, cb);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) cb[j] = (nc + j < p.n) ? load_scalar<DOUT>(p.cin, idx + j) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) cb[j] *= beta;
}

// GELU_AUX_BIAS: store the pre-activation of the 8 columns nc .. nc+7 of
// row m into the aux matrix (D's dtype, row stride ldaux elements).
template <int DOUT>
__device__ __forceinline__ void store_pre8(const KernelArgs& p, int64_t m, int nc, const float* x) {
    const int64_t idx = m * p.ldaux + nc;
    if (nc + 8 <= p.n) {
        store8<DOUT>(p.aux, idx, x);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (nc + j < p.n) store_one<DOUT>(p.aux, idx + j, x[j]);
    }
}

}  // namespace ge
