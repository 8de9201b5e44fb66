/*
 * oracle.c -- plain CPU reference for D = epilogue(A*B + bias).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or
 * constant with the HIP library: it defines its own dtype codes, epilogue
 * codes and number-format codecs, written from the format definitions.
 *
 * Pages cited (titles as printed, or as given by the page address):
 *   [cuBLASLt page]  "PyTorch inference: cuBLASLt bias fusion optimization"
 *                    (blog.hotdry.top, 2025-09-22)
 *   [nvmath page]    "nvmath-python cuBLASLt bias fusion for PyTorch inference"
 *                    (blog.hotdry.top, 2025-09-22)
 *   [epilog page]    "Explaining how nvmath-python's epilog mechanism configures
 *                    parameters to fuse the bias add into the cuBLASLt matmul
 *                    kernel" (blog.hotdry.top, 2025-09-22)
 *   [NVGEMM page]    "PyTorch 2.14 NVGEMM epilogue fusion" (zdabc.icu)
 *
 * The method fuses into one kernel what is, by definition, a sequence of
 * separate passes: a matrix product, a bias add, an activation and (for the
 * ReLU-with-aux epilogue) a sign mask ([NVGEMM page], section "NVGEMM
 * changes"; [epilog page], first body paragraph).  The fused result equals
 * that sequence up to floating-point rounding order, so this oracle is the
 * plain sequence, each pass on its own, in double precision:
 *
 *   O1  C[i][j] = sa*sb * sum_{p=0..k-1} A[i][p] * B[p][j]   (p ascending)
 *   O2  P = C + bias   (ROW: bias[i] added to every column of row i;
 *                       COL: bias[j] added to every row of column j)
 *   O3  Y = act(P), act in {identity, ReLU, GELU}
 *   O4  M[i][j] = (P[i][j] > 0), packed into a row-major bit matrix
 *
 * Inputs arrive as raw codes (fp32 words, fp16/bf16 half-words, e4m3 bytes)
 * and are decoded exactly to double by this file's own decoders.
 *
 * Built with gcc -O2 -fno-fast-math -ffp-contract=off (no FMA contraction,
 * IEEE semantics).  OpenMP only splits independent output rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- codes private to the oracle ---------------------------------------- */
enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_E4M3 = 3 };
enum { ORC_NONE = 0, ORC_BIAS = 1, ORC_RELU_BIAS = 2, ORC_RELU_AUX_BIAS = 3,
       ORC_GELU_BIAS = 4, ORC_GELU_ERF = 5 /* report-only erf form */,
       ORC_TANH_BIAS = 6 };
enum { ORC_ROW = 0, ORC_COL = 1 };

/* ---- number formats ------------------------------------------------------
 * A binary floating-point format with E exponent bits, M fraction bits and
 * exponent bias B encodes, for exponent field e and fraction field f:
 *   e == 0            : (-1)^s * f * 2^(1-B-M)            (subnormal)
 *   0 < e < 2^E-1     : (-1)^s * (2^M + f) * 2^(e-B-M)    (normal)
 *   e == 2^E-1        : IEEE formats: inf (f == 0) or NaN;
 *                       OCP E4M3: normal, except f == 2^M-1 which is NaN
 *                       (the format has no infinities; max finite 448).
 * fp16 = IEEE binary16 (E5 M10 B15); bf16 = top half of binary32 (E8 M7
 * B127); e4m3 = OCP 8-bit floating point E4M3 (E4 M3 B7).
 */
static double dec_bits(uint32_t bits, int E, int M, int B, int ieee_special)
{
    uint32_t s = (bits >> (E + M)) & 1u;
    uint32_t e = (bits >> M) & ((1u << E) - 1u);
    uint32_t f = bits & ((1u << M) - 1u);
    uint32_t emax = (1u << E) - 1u;
    double mag;
    if (e == emax && ieee_special) {
        mag = (f == 0) ? INFINITY : NAN;
    } else if (e == emax && !ieee_special && f == (1u << M) - 1u) {
        mag = NAN;
    } else if (e == 0) {
        mag = ldexp((double)f, 1 - B - M);
    } else {
        mag = ldexp((double)((1u << M) + f), (int)e - B - M);
    }
    return s ? -mag : mag;
}

double orc_dec_f16(uint16_t h)  { return dec_bits(h, 5, 10, 15, 1); }
double orc_dec_bf16(uint16_t h) { return dec_bits(h, 8, 7, 127, 1); }
double orc_dec_e4m3(uint8_t v)  { return dec_bits(v, 4, 3, 7, 0); }
double orc_dec_f32(uint32_t w)  { return dec_bits(w, 8, 23, 127, 1); }

/* Round-to-nearest-even encode of a double into the format above.
 * Overflow: IEEE formats -> inf; e4m3 saturates to +-448 when sat != 0,
 * else returns NaN.  NaN -> canonical NaN. */
static uint32_t enc_bits(double x, int E, int M, int B, int ieee_special, int sat)
{
    uint32_t s = signbit(x) ? 1u : 0u;
    uint32_t emax = (1u << E) - 1u;
    uint32_t sign = s << (E + M);
    double a = fabs(x);
    if (isnan(x)) {
        return ieee_special ? (sign | (emax << M) | (1u << (M - 1)))
                            : (sign | (emax << M) | ((1u << M) - 1u));
    }
    /* largest finite magnitude */
    double maxfin = ieee_special
        ? ldexp((double)((2u << M) - 1u), (int)emax - 1 - B - M)
        : ldexp((double)((2u << M) - 2u), (int)emax - B - M);
    if (isinf(x)) {
        if (ieee_special) return sign | (emax << M);
        return sat ? (sign | (emax << M) | ((1u << M) - 2u))
                   : (sign | (emax << M) | ((1u << M) - 1u));
    }
    if (a == 0.0) return sign;
    /* unbiased exponent of a, clamped to the minimum normal exponent so that
     * the quantum below is the subnormal quantum for tiny values */
    int ex;
    (void)frexp(a, &ex);          /* a = fr * 2^ex, fr in [0.5, 1) */
    int e_unb = ex - 1;           /* a in [2^e_unb, 2^(e_unb+1)) */
    if (e_unb < 1 - B) e_unb = 1 - B;
    double q = ldexp(1.0, e_unb - M); /* spacing of representable values */
    double r = a / q;                 /* exact: power-of-two scaling */
    double fl = floor(r);
    double diff = r - fl;
    double n;
    if (diff > 0.5) n = fl + 1.0;
    else if (diff < 0.5) n = fl;
    else n = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0; /* tie: to even */
    double v = n * q;                 /* rounded magnitude (exact) */
    if (v > maxfin) {
        if (ieee_special) return sign | (emax << M);      /* inf */
        return sat ? (sign | (emax << M) | ((1u << M) - 2u))
                   : (sign | (emax << M) | ((1u << M) - 1u));
    }
    /* assemble: n in [2^M, 2^(M+1)] for normals, [0, 2^M] for subnormals */
    if (n >= (double)(2u << M)) { n /= 2.0; e_unb += 1; }  /* carried into next binade */
    uint32_t mant = (uint32_t)n;
    uint32_t efield;
    if (mant < (1u << M)) {
        efield = 0;                                 /* subnormal */
    } else {
        efield = (uint32_t)(e_unb + B);
        mant -= (1u << M);
    }
    return sign | (efield << M) | mant;
}

uint16_t orc_enc_f16(double x)  { return (uint16_t)enc_bits(x, 5, 10, 15, 1, 0); }
uint16_t orc_enc_bf16(double x) { return (uint16_t)enc_bits(x, 8, 7, 127, 1, 0); }
uint8_t  orc_enc_e4m3_sat(double x) { return (uint8_t)enc_bits(x, 4, 3, 7, 0, 1); }

/* decode one element of a raw buffer */
static double dec_at(int dtype, const void* p, int64_t idx)
{
    switch (dtype) {
    case ORC_F32: { uint32_t w; memcpy(&w, (const uint8_t*)p + 4 * idx, 4); return orc_dec_f32(w); }
    case ORC_F16: return orc_dec_f16(((const uint16_t*)p)[idx]);
    case ORC_BF16: return orc_dec_bf16(((const uint16_t*)p)[idx]);
    case ORC_E4M3: return orc_dec_e4m3(((const uint8_t*)p)[idx]);
    }
    return NAN;
}

/* O0: exact decode of n raw elements to double. */
int orc_decode(int dtype, const void* src, int64_t n, double* dst)
{
    if (dtype < ORC_F32 || dtype > ORC_E4M3) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) dst[i] = dec_at(dtype, src, i);
    return 0;
}

/* ---- O1: the matrix product ---------------------------------------------
 * Row-major A (m x k, leading dimension lda).  B is k x n row-major (op_b=0,
 * leading dimension ldb >= n) or, for a Linear layer's weight, n x k
 * row-major with B[p][j] = W[j][p] (op_b=1, ldb >= k).  Operand layouts
 * follow the nvmath page's code example (a is m x k, b is k x n).
 * Accumulates in double with p ascending, then scales by sa*sb (per-tensor
 * dequantisation factors of fp8 inputs; 1 otherwise). */
static double b_at(int tb, const void* B, int64_t ldb, int op_b, int64_t p, int64_t j)
{
    return op_b ? dec_at(tb, B, j * ldb + p) : dec_at(tb, B, p * ldb + j);
}

/* absval = 0: the product itself.  absval = 1: the same sums over the
 * absolute values of the operands, |sa*sb| * sum_p |A[i][p]| * |B[p][j]| --
 * the magnitude term of the standard forward error bound of a dot product
 * computed in floating point (Higham, "Accuracy and Stability of Numerical
 * Algorithms", section 3.1: |fl(x.y) - x.y| <= gamma_n * |x|.|y|), which the
 * parity tests use to bound each output element's rounding error. */
static double opnd(double v, int absval) { return absval ? fabs(v) : v; }

static int gemm_impl(int64_t m, int64_t n, int64_t k,
                     int ta, const void* A, int64_t lda,
                     int tb, const void* B, int64_t ldb, int op_b,
                     double sa, double sb, int absval, double* C)
{
    if (m < 0 || n < 0 || k < 0) return -1;
    const double s = absval ? fabs(sa * sb) : sa * sb;
    /* decode B once (column access pattern), A per row */
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(k * n > 0 ? k * n : 1));
    if (!Bd) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < k; ++p)
        for (int64_t j = 0; j < n; ++j) Bd[p * n + j] = opnd(b_at(tb, B, ldb, op_b, p, j), absval);
    int err = 0;
#pragma omp parallel
    {
        double* arow = (double*)malloc(sizeof(double) * (size_t)(k > 0 ? k : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (!arow || !acc) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < m; ++i) {
                for (int64_t p = 0; p < k; ++p) arow[p] = opnd(dec_at(ta, A, i * lda + p), absval);
                for (int64_t j = 0; j < n; ++j) acc[j] = 0.0;
                for (int64_t p = 0; p < k; ++p) {         /* p ascending */
                    const double a = arow[p];
                    const double* brow = Bd + p * n;
                    for (int64_t j = 0; j < n; ++j) acc[j] += a * brow[j];
                }
                for (int64_t j = 0; j < n; ++j) C[i * n + j] = s * acc[j];
            }
        }
        free(arow);
        free(acc);
    }
    free(Bd);
    return err;
}

int orc_gemm(int64_t m, int64_t n, int64_t k,
             int ta, const void* A, int64_t lda,
             int tb, const void* B, int64_t ldb, int op_b,
             double sa, double sb, double* C /* m x n, dense */)
{
    return gemm_impl(m, n, k, ta, A, lda, tb, B, ldb, op_b, sa, sb, 0, C);
}

/* |sa*sb| * |A|.|B| (see gemm_impl). */
int orc_gemm_abs(int64_t m, int64_t n, int64_t k,
                 int ta, const void* A, int64_t lda,
                 int tb, const void* B, int64_t ldb, int op_b,
                 double sa, double sb, double* G /* m x n, dense */)
{
    return gemm_impl(m, n, k, ta, A, lda, tb, B, ldb, op_b, sa, sb, 1, G);
}

/* O1 on selected entries only, for problems too large to compute whole.
 * A_rows holds some rows of A (leading dimension lda); entry t is
 * C[row of A_rows[slot[t]]][col[t]].  Same arithmetic as orc_gemm (absval 0)
 * or orc_gemm_abs (absval 1). */
static int entries_impl(int64_t k, int ta, const void* A_rows, int64_t lda,
                        int tb, const void* B, int64_t ldb, int op_b,
                        double sa, double sb, int absval, int64_t cnt,
                        const int64_t* slot, const int64_t* col, double* out)
{
    if (k < 0 || cnt < 0) return -1;
    const double s = absval ? fabs(sa * sb) : sa * sb;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < cnt; ++t) {
        double acc = 0.0;
        for (int64_t p = 0; p < k; ++p)              /* p ascending */
            acc += opnd(dec_at(ta, A_rows, slot[t] * lda + p), absval) *
                   opnd(b_at(tb, B, ldb, op_b, p, col[t]), absval);
        out[t] = s * acc;
    }
    return 0;
}

int orc_gemm_entries(int64_t k, int ta, const void* A_rows, int64_t lda,
                     int tb, const void* B, int64_t ldb, int op_b,
                     double sa, double sb, int64_t cnt,
                     const int64_t* slot, const int64_t* col, double* out)
{
    return entries_impl(k, ta, A_rows, lda, tb, B, ldb, op_b, sa, sb, 0, cnt, slot, col, out);
}

int orc_gemm_abs_entries(int64_t k, int ta, const void* A_rows, int64_t lda,
                         int tb, const void* B, int64_t ldb, int op_b,
                         double sa, double sb, int64_t cnt,
                         const int64_t* slot, const int64_t* col, double* out)
{
    return entries_impl(k, ta, A_rows, lda, tb, B, ldb, op_b, sa, sb, 1, cnt, slot, col, out);
}

/* ---- O1x: the product with per-block scales (block-scaled fp8) ------------
 * The nvmath page names FP8 among the supported input types and, in its
 * closing paragraph, low-precision formats as where the fused epilogue is
 * going.  Beyond one scale per tensor, the OCP Microscaling (MX) format
 * gives every run of 32 consecutive elements along K its own scale: an E8M0
 * value, an 8-bit biased exponent with no sign and no mantissa, scale =
 * 2^(e - 127), the code 0xFF being NaN.  With SA one scale per (row i of A,
 * block b = p / 32) and SB one per (column j of B, block b):
 *
 *   C[i][j] = sa*sb * sum_p  (dec(A[i][p]) * 2^(SA[i][p/32] - 127))
 *                          * (dec(B[p][j]) * 2^(SB[j][p/32] - 127))
 *
 * SA is m x ceil(k/32) bytes with row stride ldsa; SB is n x ceil(k/32)
 * bytes (the blocks of column j contiguous, whichever layout B has) with
 * row stride ldsb.  absval = 1 gives the same sum over absolute values (the
 * magnitude term of the error bound, see gemm_impl). */
double orc_dec_e8m0(uint8_t e)
{
    if (e == 0xFFu) return NAN;
    return ldexp(1.0, (int)e - 127);
}

static int gemm_mx_impl(int64_t m, int64_t n, int64_t k,
                        int ta, const void* A, int64_t lda, const uint8_t* SA, int64_t ldsa,
                        int tb, const void* B, int64_t ldb, int op_b, const uint8_t* SB, int64_t ldsb,
                        double sa, double sb, int absval, double* C)
{
    if (m < 0 || n < 0 || k < 0) return -1;
    const int64_t kb = (k + 31) / 32;
    if (ldsa < kb || ldsb < kb) return -1;
    const double s = absval ? fabs(sa * sb) : sa * sb;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t p = 0; p < k; ++p) {           /* p ascending */
                const double a = dec_at(ta, A, i * lda + p) * orc_dec_e8m0(SA[i * ldsa + p / 32]);
                const double b = b_at(tb, B, ldb, op_b, p, j) * orc_dec_e8m0(SB[j * ldsb + p / 32]);
                acc += opnd(a, absval) * opnd(b, absval);
            }
            C[i * n + j] = s * acc;
        }
    }
    return err;
}

int orc_gemm_mx(int64_t m, int64_t n, int64_t k, int ta, const void* A, int64_t lda, const uint8_t* SA,
                int64_t ldsa, int tb, const void* B, int64_t ldb, int op_b, const uint8_t* SB, int64_t ldsb,
                double sa, double sb, double* C)
{
    return gemm_mx_impl(m, n, k, ta, A, lda, SA, ldsa, tb, B, ldb, op_b, SB, ldsb, sa, sb, 0, C);
}

int orc_gemm_mx_abs(int64_t m, int64_t n, int64_t k, int ta, const void* A, int64_t lda, const uint8_t* SA,
                    int64_t ldsa, int tb, const void* B, int64_t ldb, int op_b, const uint8_t* SB, int64_t ldsb,
                    double sa, double sb, double* G)
{
    return gemm_mx_impl(m, n, k, ta, A, lda, SA, ldsa, tb, B, ldb, op_b, SB, ldsb, sa, sb, 1, G);
}

/* O1x at selected entries (problems too large to compute whole): A_rows
 * holds some rows of A with their scale rows in SA_rows; entry t is
 * C[row slot[t] of A_rows][col[t]].  Same arithmetic as gemm_mx_impl. */
static int mx_entries_impl(int64_t k, int ta, const void* A_rows, int64_t lda, const uint8_t* SA_rows,
                           int64_t ldsa, int tb, const void* B, int64_t ldb, int op_b, const uint8_t* SB,
                           int64_t ldsb, double sa, double sb, int absval, int64_t cnt, const int64_t* slot,
                           const int64_t* col, double* out)
{
    if (k < 0 || cnt < 0) return -1;
    const double s = absval ? fabs(sa * sb) : sa * sb;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < cnt; ++t) {
        double acc = 0.0;
        for (int64_t p = 0; p < k; ++p) {               /* p ascending */
            const double a = dec_at(ta, A_rows, slot[t] * lda + p) * orc_dec_e8m0(SA_rows[slot[t] * ldsa + p / 32]);
            const double b = b_at(tb, B, ldb, op_b, p, col[t]) * orc_dec_e8m0(SB[col[t] * ldsb + p / 32]);
            acc += opnd(a, absval) * opnd(b, absval);
        }
        out[t] = s * acc;
    }
    return 0;
}

int orc_gemm_mx_entries(int64_t k, int ta, const void* A_rows, int64_t lda, const uint8_t* SA_rows, int64_t ldsa,
                        int tb, const void* B, int64_t ldb, int op_b, const uint8_t* SB, int64_t ldsb, double sa,
                        double sb, int64_t cnt, const int64_t* slot, const int64_t* col, double* out)
{
    return mx_entries_impl(k, ta, A_rows, lda, SA_rows, ldsa, tb, B, ldb, op_b, SB, ldsb, sa, sb, 0, cnt, slot,
                           col, out);
}

int orc_gemm_mx_abs_entries(int64_t k, int ta, const void* A_rows, int64_t lda, const uint8_t* SA_rows,
                            int64_t ldsa, int tb, const void* B, int64_t ldb, int op_b, const uint8_t* SB,
                            int64_t ldsb, double sa, double sb, int64_t cnt, const int64_t* slot,
                            const int64_t* col, double* out)
{
    return mx_entries_impl(k, ta, A_rows, lda, SA_rows, ldsa, tb, B, ldb, op_b, SB, ldsb, sa, sb, 1, cnt, slot,
                           col, out);
}

/* ---- O2: bias broadcast ---------------------------------------------------
 * ROW: the bias has one value per output row (shape (m,) or (m,1)) and is
 * added to every column ([epilog page], paragraph on epilog_inputs: the bias
 * matches the output's row count and is added to each column).
 * COL: one value per output column (shape (1,n)), added to every row
 * ([nvmath page], paragraph on shape constraints, which allows (m,1) or
 * (1,n)); this is a Linear layer's bias.
 * rows/cols give each entry's output coordinates. */
int orc_bias_entries(int64_t cnt, const double* C, const int64_t* rows,
                     const int64_t* cols, int axis, int tbias,
                     const void* bias, double* P)
{
    if (axis != ORC_ROW && axis != ORC_COL) return -1;
    for (int64_t t = 0; t < cnt; ++t) {
        int64_t idx = (axis == ORC_ROW) ? rows[t] : cols[t];
        P[t] = C[t] + dec_at(tbias, bias, idx);
    }
    return 0;
}

int orc_bias(int64_t m, int64_t n, const double* C, int axis, int tbias,
             const void* bias, double* P)
{
    if (axis != ORC_ROW && axis != ORC_COL) return -1;
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            P[i * n + j] = C[i * n + j] + dec_at(tbias, bias, axis == ORC_ROW ? i : j);
    return 0;
}

/* ---- O3: activation --------------------------------------------------------
 * ReLU(x) = max(x, 0) ([epilog page], paragraph on the epilog enum: ReLU is
 * applied right after the bias).
 * GELU(x) = x * Phi(x) with Phi the standard normal CDF.  The pages name
 * GELU as a fused activation ([cuBLASLt page], paragraph 2; NVGEMM page,
 * section on epilogue fusion) but print no formula.  The tanh form
 *   GELU(x) ~= 0.5 x (1 + tanh( sqrt(2/pi) (x + 0.044715 x^3) ))
 * is the one computed here; the exact erf form 0.5 x (1 + erf(x/sqrt 2)) is
 * provided for reporting only (ORC_GELU_ERF). */
static double gelu_tanh(double x)
{
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}
static double gelu_erf(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

double orc_act1(int epilog, double x)
{
    switch (epilog) {
    case ORC_NONE:
    case ORC_BIAS: return x;
    case ORC_RELU_BIAS:
    case ORC_RELU_AUX_BIAS: return x > 0.0 ? x : 0.0; /* max(x,0); NaN -> 0 */
    case ORC_GELU_BIAS: return gelu_tanh(x);
    case ORC_GELU_ERF: return gelu_erf(x);
    /* Tanh is among the predefined epilogues the [nvmath page] names
     * (limitations paragraph: Bias, ReLU, Tanh, ...): Y = tanh(P). */
    case ORC_TANH_BIAS: return tanh(x);
    }
    return NAN;
}

int orc_act(int64_t cnt, int epilog, const double* P, double* Y)
{
    if (epilog < ORC_NONE || epilog > ORC_TANH_BIAS) return -1;
    for (int64_t t = 0; t < cnt; ++t) Y[t] = orc_act1(epilog, P[t]);
    return 0;
}

/* ---- O4: ReLU sign mask ----------------------------------------------------
 * The ReLU-with-aux epilogue also returns a mask of the ReLU input's sign for
 * the backward pass ([epilog page], paragraph on the epilog enum; [nvmath
 * page], paragraph on limitations).  Bit (i,j) = 1 iff the pre-activation
 * P[i][j] > 0 (so P == 0 and NaN give 0, matching ReLU'(0) = 0).
 * Layout: row-major bit matrix, row i starts at 32-bit word i*ldw; bit j of
 * the row is bit (j % 32) of little-endian word i*ldw + j/32.  ldw is the row
 * stride in words (the library uses round_up(n,128)/32).  Padding bits are 0. */
int orc_mask(int64_t m, int64_t n, const double* P, int64_t ldw, uint32_t* words)
{
    if (ldw * 32 < n) return -1;
    memset(words, 0, sizeof(uint32_t) * (size_t)(m * ldw));
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            if (P[i * n + j] > 0.0) words[i * ldw + j / 32] |= (1u << (j % 32));
    return 0;
}

/* ---- training-side epilogues ---------------------------------------------
 * The pages tie the aux output to the backward pass: in training the backward
 * pass needs the intermediate activation, and a ReLU epilogue with aux output
 * returns the mask it needs ([nvmath page], paragraph on limitations); fusing
 * GELU and the bias gradient into the epilogue is where they see the method
 * going next ([nvmath page], closing paragraph).  Their plainest reading, as
 * separate passes after O1 (O2 and O3 as above where a bias is involved):
 *
 *   O5  GELU with aux:  Y = GELU(P) (O3) and the aux output is P itself,
 *                       the value GELU's backward needs (stored in D's dtype);
 *   O6  DRELU:          D = C * ReLU'(P), ReLU'(P) = (P > 0) read from the O4
 *                       bit matrix of a forward pass (no bias);
 *   O7  DGELU:          D = C * GELU'(P), P read from an O5 aux output.
 *
 * GELU' is the derivative of the tanh form, by the product and chain rules:
 *   d/dx [0.5 x (1 + tanh u(x))] = 0.5 (1 + tanh u) + 0.5 x (1 - tanh(u)^2) u'(x)
 *   with u = sqrt(2/pi) (x + 0.044715 x^3), u' = sqrt(2/pi) (1 + 3 * 0.044715 x^2). */
double orc_gelu_deriv(double x)
{
    const double c = sqrt(2.0 / M_PI);
    const double u = c * (x + 0.044715 * x * x * x);
    const double du = c * (1.0 + 3.0 * 0.044715 * x * x);
    const double t = tanh(u);
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * du;
}

/* O6: D[i][j] = C[i][j] if bit (i,j) of the O4 layout (row stride ldw words)
 * is set, else 0. */
int orc_drelu(int64_t m, int64_t n, const double* C, int64_t ldw, const uint32_t* words, double* D)
{
    if (ldw * 32 < n) return -1;
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            const uint32_t bit = (words[i * ldw + j / 32] >> (j % 32)) & 1u;
            D[i * n + j] = bit ? C[i * n + j] : 0.0;
        }
    return 0;
}

/* O7: D[i][j] = C[i][j] * GELU'(P[i][j]), P given as codes of dtype tp with
 * row stride ldp elements, decoded exactly. */
int orc_dgelu(int64_t m, int64_t n, const double* C, int tp, const void* P, int64_t ldp, double* D)
{
    if (ldp < n || tp < ORC_F32 || tp > ORC_E4M3) return -1;
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            D[i * n + j] = C[i * n + j] * orc_gelu_deriv(dec_at(tp, P, i * ldp + j));
    return 0;
}

/* O8: the bias gradient of the backward epilogues (the dBias fusion the
 * [nvmath page] closing paragraph looks ahead to).  The forward added the
 * bias along one axis, so its gradient sums the backward result Y (O6 or O7,
 * unrounded) along the other:
 *   ROW (bias[i] was added to row i):    g[i] = sum_j Y[i][j]   (j ascending)
 *   COL (bias[j] was added to column j): g[j] = sum_i Y[i][j]   (i ascending) */
int orc_bgrad(int64_t m, int64_t n, const double* Y, int axis, double* g)
{
    if (axis == ORC_ROW) {
        for (int64_t i = 0; i < m; ++i) {
            double s = 0.0;
            for (int64_t j = 0; j < n; ++j) s += Y[i * n + j];
            g[i] = s;
        }
        return 0;
    }
    if (axis == ORC_COL) {
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int64_t i = 0; i < m; ++i) s += Y[i * n + j];
            g[j] = s;
        }
        return 0;
    }
    return -1;
}

/* O1b: an added input term, P0 = C + beta * Cin, before the bias (the general
 * epilogue alpha*A*B + beta*C + bias of the [cuBLASLt page], paragraph on
 * compute and scale types; alpha is O1's sa*sb).  Cin is given as codes of
 * dtype tc with row stride ldc, decoded exactly. */
int orc_add_beta_c(int64_t m, int64_t n, const double* C, double beta, int tc, const void* Cin, int64_t ldc,
                   double* P0)
{
    if (ldc < n || tc < ORC_F32 || tc > ORC_E4M3) return -1;
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j)
            P0[i * n + j] = C[i * n + j] + beta * dec_at(tc, Cin, i * ldc + j);
    return 0;
}
