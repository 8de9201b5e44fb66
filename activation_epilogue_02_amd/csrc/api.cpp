// api.cpp -- the C-ABI front end: handle life cycle, validation, the
// planner (tile / small-m / unfused choice and launch shape) and execute.
//
// Every check runs on the host before any HIP runtime call, so that a call
// that fails launches nothing (nvmath page, paragraph on dtype and shape
// rules: mismatched dtypes or a wrongly shaped bias make the fusion fail;
// epilog page, paragraph on epilog_inputs: tensors must be 16-byte aligned).
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "ge_params.h"

using namespace ge;

// ---- the workspace the library holds itself (gemm_epilog_execute_static) -----
// One fixed array per GPU in the library's code object, held until the
// process ends, for callers that cannot allocate.  Host code never uses the
// array's name as a device address (it is a host-side stand-in): the first
// call on a device asks the runtime for that device's copy
// (hipGetSymbolAddress with the device current) and every call passes that
// address to the kernels.
static __device__ __align__(256) uint8_t scratch[GE_STATIC_WORKSPACE_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch` (looked up once per device).
int scratch_of_current_device(void** p) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return GE_ERR_HIP;
        g_scratch_ptr[dev] = q;
    }
    *p = g_scratch_ptr[dev];
    return GE_OK;
}
}  // namespace

struct ge_plan_s {
    ge_desc d;
    bool planned = false;
    int32_t epilog = 0, axis = 0;
    int32_t path = 0, tile_id = 0, unfused = 0;
    int32_t split_k = 1, k_per_split = 0;
    int32_t tiles_m = 0, tiles_n = 0, group_m = 1;
    int32_t k_stagger = 0;
    unsigned grid = 0;
    size_t ws_c = 0;         // unfused intermediate bytes
    size_t ws_partial = 0;   // split-K partial bytes
    size_t ws_counters = 0;  // split-K counter bytes
    int64_t n_counters = 0;  // split-K arrival counters per product
    int64_t part_bytes = 0;  // split-K partial bytes per product
    size_t ws_bgrad = 0;     // bias-gradient partial bytes
    int32_t bgrad_parts = 0; // bias-gradient partials per entry
    ge_pref pref = {0, 0, 0, 0, 0};   // the preferences the plan was made with
    int64_t ldaux = 0;       // mask row stride, 32-bit words
    bool bstr_set = false;   // per-product strides given (else packed)
    ge_batch_strides bstr = {0, 0, 0, 0, 0};
    const float* scale_d = nullptr;   // fp8 output: D's scale (NULL = 1)
    float* amax_d = nullptr;          // fp8 output: largest |y| per product, or NULL
};

namespace {

int elem_size(int t) {
    switch (t) {
    case GE_F32: return 4;
    case GE_F16: return 2;
    case GE_BF16: return 2;
    case GE_F8_E4M3: return 1;
    case GE_MXF8_E4M3: return 1;
    }
    return 0;
}

bool dtype_combo_ok(int a, int b, int d) {
    if (a != b) return false;
    switch (a) {
    case GE_F32: return d == GE_F32;
    case GE_F16: return d == GE_F16 || d == GE_F32 || d == GE_F8_E4M3;
    case GE_BF16: return d == GE_BF16 || d == GE_F32 || d == GE_F8_E4M3;
    case GE_F8_E4M3:
    case GE_MXF8_E4M3: return d == GE_BF16 || d == GE_F16 || d == GE_F32 || d == GE_F8_E4M3;
    }
    return false;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Epilogues that add a bias (DRELU and DGELU read none).
bool has_bias(int e) {
    return e == GE_EPILOG_BIAS || e == GE_EPILOG_RELU_BIAS || e == GE_EPILOG_RELU_AUX_BIAS ||
           e == GE_EPILOG_GELU_BIAS || e == GE_EPILOG_GELU_AUX_BIAS || e == GE_EPILOG_TANH_BIAS;
}
// Epilogues with an aux buffer: a bit mask (written by RELU_AUX_BIAS, read by
// DRELU) or a pre-activation matrix in D's dtype (written by GELU_AUX_BIAS,
// read by DGELU).
bool is_bgrad(int e) { return e == GE_EPILOG_DRELU_BGRAD || e == GE_EPILOG_DGELU_BGRAD; }
bool has_aux(int e) {
    return e == GE_EPILOG_RELU_AUX_BIAS || e == GE_EPILOG_DRELU || e == GE_EPILOG_GELU_AUX_BIAS ||
           e == GE_EPILOG_DGELU || is_bgrad(e);
}
bool aux_is_matrix(int e) {
    return e == GE_EPILOG_GELU_AUX_BIAS || e == GE_EPILOG_DGELU || e == GE_EPILOG_DGELU_BGRAD;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

const TileShape* find_tile(int id) {
    for (int i = 0; i < kNumTiles; ++i)
        if (kTiles[i].id == id) return &kTiles[i];
    return nullptr;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The register-staged tile kernel's tile for a problem (any dtype).
int choose_tile_plain(int64_t m, int64_t n) {
    const int64_t t256 = ceil_div(m, 256) * ceil_div(n, 256);
    const int64_t t128 = ceil_div(m, 128) * ceil_div(n, 128);
    if (t256 >= 512) return 3;
    if (t128 >= 512) return 2;
    if (t256 >= 256 && t128 < 256) return 3;
    if (t128 >= 256) return 2;
    return 1;
}

// Tile heuristic: the largest block tile that still gives every CU at least
// two tiles (256 CUs); below that, the shape with the most tiles.  Large
// tiles halve the L2 -> LDS traffic per flop; small problems need the
// parallelism more than the reuse.
int choose_tile(int64_t m, int64_t n, int a_type, int d_type) {
    const int64_t t256 = ceil_div(m, 256) * ceil_div(n, 256);
    const int64_t t128 = ceil_div(m, 128) * ceil_div(n, 128);
    // fp8 output: the tiles instantiated for it (the large one when it
    // gives every CU a tile, else 128 x 128)
    if (d_type == GE_F8_E4M3) {
        if (a_type == GE_MXF8_E4M3) return 8;
        if (a_type == GE_F8_E4M3) return t256 >= 512 ? 16 : ceil_div(m, 256) * ceil_div(n, 128) >= 512 ? 15 : 8;
        return t256 >= 256 ? 6 : 8;
    }
    // block-scaled fp8: the one tile the block-scaled MFMA compiles into
    // without register spills
    if (a_type == GE_MXF8_E4M3) return 8;
    if (a_type == GE_F8_E4M3) {
        // A CU takes about 0.2 128-byte lines per cycle into LDS, so tiles
        // with fewer bytes per flop keep the matrix cores busier: 256 x 256
        // with 8 waves and 64-byte K steps (four 32 KiB stages, spread
        // copies; tile 16) measures 8% faster than 256 x 128 (tile 15) on
        // 65536 x 8192 x 16384 (2379 against 2200 TFLOP/s).  With 128-byte
        // steps a 256 x 256 stage is 64 KiB and only two fit.  256 x 128 with
        // 8 waves (two per SIMD) beats 4 waves by 10% (1943 against 1765).
        const int64_t t2x1 = ceil_div(m, 256) * ceil_div(n, 128);
        if (t256 >= 512) return 16;
        if (t2x1 >= 512) return 15;
        if (t128 >= 256) return 8;
        return 1;
    }
    if (a_type == GE_F16 || a_type == GE_BF16) {
        // the pipelined direct-to-LDS kernel; at 256 x 256 the 8-wave
        // layout (two waves per SIMD fill each other's barrier gaps) with
        // four 64-byte K stages, whose copies are spread among the MFMAs,
        // measures fastest (65536 x 8192 x 16384: 1258 TFLOP/s against
        // 1164 for two 128-byte stages with the copies in one burst)
        if (t256 >= 512) return 6;
        if (t128 >= 512) return 8;
        if (t256 >= 256 && t128 < 256) return 6;
        if (t128 >= 256) return 8;
        return 13;   // small problems: 64 x 64 tiles, four deep stages
    }
    return choose_tile_plain(m, n);
}

// The pipelined kernels' direct copies address a tile's rows of A, and of B
// (either layout), as 32-bit offsets from the tile's first row or column:
// the span must stay below 4 GiB.  (A K step is at most 128 elements.)
bool tile_span_ok(const TileShape* t, const ge_desc& d) {
    if (t->kernel == 1 || t->kernel == 3) return true;   // per-lane 64-bit addresses
    const int64_t es = elem_size(d.a_type), lim = (int64_t)1 << 32;
    if ((int64_t)t->bm * d.lda * es > lim) return false;
    if (d.op_b == GE_OP_T) return (int64_t)t->bn * d.ldb * es <= lim;
    return ((int64_t)128 * d.ldb + t->bn) * es <= lim;
}

// Tile rows per group of the launch order (see tile_coords).  The 32 tiles
// an XCD runs at once then cover g tile rows and 32 / g columns.  Fewer rows
// than the 8 that minimise the panels in flight measure faster: with eight,
// every B line is wanted by eight CUs at the same moment and A lines by
// four, and the requests queue behind the one that misses (65536 x 8192 x
// 16384 bf16, 256 x 256 tiles: 1207 / 1258 / 1236 TFLOP/s at 8 / 4 / 2 rows;
// the block-scaled 128 x 128 tile: 1150 / 1198 / 1278).
int32_t auto_group_m(const TileShape* t, int64_t tm, int a_type) {
    const int64_t g = a_type == GE_MXF8_E4M3 ? 2 : (t->kernel == 1 ? 8 : 4);
    return (int32_t)(tm < g ? (tm > 0 ? tm : 1) : g);
}

// Full K steps of rotation per tile row and column of a group (the
// pipelined kernel's K order).  The tiles that share a panel of A or B run in
// lock-step, so their requests for the same lines arrive together and queue
// behind the one that misses; rotating each tile's K order spreads them, at
// the cost of a longer stretch of each panel held in L2.  Measured on 65536 x
// 8192 x 16384 (TFLOP/s at 0 / 1 / 2 / 4 / 8 steps): the block-scaled 128 x
// 128 tile, 16 tiles on each A panel at once, 1290 / 1335 / 1356 / 1347 /
// 1290; the fp8 256 x 256 tile 2332-2367 unrotated against 2358-2392 at one
// step; the bf16 256 x 256 tile 1273-1276 / 1273 / 1262 / 1247 (none there).
// GE_K_STAGGER=<steps> in the environment overrides the choice.
int32_t auto_k_stagger(const TileShape* t, int a_type) {
    if (const char* e = getenv("GE_K_STAGGER")) {
        const int v = atoi(e);
        return v > 0 ? v : 0;
    }
    if (a_type == GE_MXF8_E4M3 && t->id == 8) return 2;
    if (a_type == GE_F8_E4M3 && t->id == 16) return 1;
    return 0;
}

// The pipelined kernel takes 16-bit and fp8 inputs (its 64 x 64 tile only
// 16-bit ones); block-scaled fp8 runs on its 128 x 128 tile only.
bool tile_supports(const TileShape* t, int a_type, int d_type) {
    if (d_type == GE_F8_E4M3) {   // fp8 output: the instantiated tiles only
        if (a_type == GE_MXF8_E4M3) return t->id == 8;
        if (a_type == GE_F8_E4M3) return t->id == 16 || t->id == 15 || t->id == 8;
        return t->id == 6 || t->id == 8;
    }
    if (a_type == GE_MXF8_E4M3) return t->id == 8;
    if (t->kernel == 1) return true;
    if (t->id == 13 || t->id == 14) return a_type == GE_F16 || a_type == GE_BF16;
    if (t->kernel == 6) return a_type == GE_F8_E4M3;
    return a_type == GE_F16 || a_type == GE_BF16 || a_type == GE_F8_E4M3;
}

bool smallm_supported(const ge_desc& d) {
    return d.m <= 16 && d.op_b == GE_OP_T && (d.a_type == GE_F16 || d.a_type == GE_BF16) &&
           (d.d_type == d.a_type || d.d_type == GE_F32);
}

// Automatic K split of the small-m path.  The kernel's register use leaves
// room for one workgroup per CU (256 CUs), so a grid beyond 256 runs in a
// second round that pays the whole load-latency chain again, and the
// split's serial device-scope round trips (partial store, arrival count,
// reload) only pay off when the column blocks alone leave CUs idle.  Hence:
// the largest power of two that keeps the grid within one round and each of
// the 8 waves at two or more 64-wide K spans.
int smallm_auto_split(int64_t tiles_n, int64_t spans) {
    constexpr int64_t kCUs = 256, kWaves = 8, kMinSpansPerWave = 2;
    int split = 1;
    while (tiles_n * split * 2 <= kCUs && spans >= split * 2 * kWaves * kMinSpansPerWave) split *= 2;
    return split;
}

// GE_LOG=1 in the environment: every successful plan prints its
// description (path, tile, grid, split, workspace) to stderr.
bool plan_log() {
    const char* e = getenv("GE_LOG");
    return e && e[0] == '1';
}

bool test_fail_launch() {
    const char* e = getenv("GE_TEST_FAIL_LAUNCH");
    return e && e[0] == '1';
}

}  // namespace

extern "C" {

int gemm_epilog_create(ge_handle* h, const ge_desc* desc) {
    if (!h || !desc) return GE_ERR_NULL;
    *h = nullptr;
    const ge_desc& d = *desc;
    if (d.m < 0 || d.n < 0 || d.k < 0) return GE_ERR_SHAPE;
    if (d.m > INT32_MAX || d.n > INT32_MAX || d.k > INT32_MAX) return GE_ERR_SHAPE;
    if (d.batch < 0 || d.batch > 65535 || (d.op_b != GE_OP_N && d.op_b != GE_OP_T)) return GE_ERR_SHAPE;
    if (!dtype_combo_ok(d.a_type, d.b_type, d.d_type)) return GE_ERR_DTYPE;
    // the bias follows D's dtype; for fp8 D it is bf16
    if (d.bias_type != (d.d_type == GE_F8_E4M3 ? GE_BF16 : d.d_type)) return GE_ERR_DTYPE;
    if (d.lda < d.k || d.ldd < d.n) return GE_ERR_SHAPE;
    if (d.ldb < (d.op_b == GE_OP_N ? d.n : d.k)) return GE_ERR_SHAPE;
    if ((d.lda * elem_size(d.a_type)) % 16 || (d.ldb * elem_size(d.b_type)) % 16 ||
        (d.ldd * elem_size(d.d_type)) % 16)
        return GE_ERR_ALIGN;
    ge_plan_s* p = new (std::nothrow) ge_plan_s();
    if (!p) return GE_ERR_ALLOC;
    p->d = d;
    *h = p;
    return GE_OK;
}

int gemm_epilog_plan(ge_handle h, int32_t epilog, int32_t bias_axis, const ge_pref* pref) {
    if (!h) return GE_ERR_NULL;
    if (epilog < GE_EPILOG_NONE || epilog > GE_EPILOG_TANH_BIAS) return GE_ERR_EPILOG;
    if (bias_axis != GE_BIAS_ROW && bias_axis != GE_BIAS_COL) return GE_ERR_EPILOG;
    ge_pref pr = {0, 0, 0, 0, 0};
    if (pref) pr = *pref;
    if (pr.path < 0 || pr.path > PATH_SMALLM || pr.unfused < 0 || pr.unfused > 1 || pr.split_k < 0 ||
        pr.group_m < 0)
        return GE_ERR_SHAPE;
    if (pr.tile != 0 && !find_tile(pr.tile)) return GE_ERR_SHAPE;
    const ge_desc& d = h->d;

    ge_plan_s q = *h;
    q.planned = false;
    q.k_stagger = 0;
    q.epilog = epilog;
    q.axis = bias_axis;
    q.unfused = (pr.unfused && epilog != GE_EPILOG_NONE) ? 1 : 0;
    // fp8 output serves the inference epilogues in the fused kernel (no aux
    // matrix in D's dtype, no backward epilogue, no fp8 intermediate)
    if (d.d_type == GE_F8_E4M3) {
        const bool inference = epilog <= GE_EPILOG_GELU_BIAS || epilog == GE_EPILOG_TANH_BIAS;
        if (!inference || q.unfused) return GE_ERR_DTYPE;
    }
    // aux row stride: round_up(n, 128) bits (mask, in 32-bit words) or
    // elements (pre-activation matrix)
    q.ldaux = !has_aux(epilog) ? 0
              : aux_is_matrix(epilog) ? (int64_t)round_up((size_t)d.n, 128)
                                      : (int64_t)round_up((size_t)d.n, 128) / 32;
    if (q.ldaux > INT32_MAX) return GE_ERR_SHAPE;

    // a batch takes product z's bias at z * len values: with a column bias
    // whose n values are not a whole number of 16-byte chunks, every other
    // product's bias would start misaligned for the kernels' 16-byte loads
    if (d.batch > 1 && bias_axis == GE_BIAS_COL && has_bias(epilog) && (d.n * elem_size(d.bias_type)) % 16 != 0)
        return GE_ERR_ALIGN;

    // the small-m kernel serves the inference epilogues only
    const bool smallm_epilog = epilog <= GE_EPILOG_GELU_BIAS || epilog == GE_EPILOG_TANH_BIAS;
    int path = pr.path;
    if (path == 0) path = (smallm_supported(d) && smallm_epilog) ? PATH_SMALLM : PATH_TILE;
    if (path == PATH_SMALLM && !smallm_supported(d)) return GE_ERR_SHAPE;
    if (path == PATH_SMALLM && !smallm_epilog) return GE_ERR_EPILOG;
    q.path = path;
    q.split_k = 1;
    q.ws_partial = q.ws_counters = 0;
    q.n_counters = q.part_bytes = 0;
    if (path == PATH_SMALLM) {
        q.tile_id = 0;
        q.tiles_m = 1;
        // column blocks of 16 * rg rows of W (rg row groups per wave, which
        // share each x fragment).  Every workgroup reads all of x, as many
        // load instructions per CU as its W slab needs, so two groups cut a
        // CU's loads by a quarter; they pay when the 32-column blocks alone
        // still fill the chip (measured at k = 4096: n = 8192 19.0 against
        // 21.0 us, 16384 33.2 against 39.8 us; four groups no better).  A K
        // split to make up the blocks does not: its partial exchange costs
        // about 6 us (n = 4096: 14.5 us with two groups in two slices,
        // 11.1 us with one group unsplit).
        if (pr.group_m != 0 && pr.group_m != 1 && pr.group_m != 2 && pr.group_m != 4) return GE_ERR_SHAPE;
        const int rg = pr.group_m > 0 ? pr.group_m : (ceil_div(d.n, 32) >= 256 ? 2 : 1);
        q.tiles_n = (int32_t)ceil_div(d.n, 16 * rg);
        // K slices of whole 64-element spans (the kernel's load unit)
        const int64_t spans = ceil_div(d.k, 64);
        int split = pr.split_k > 0 ? pr.split_k : smallm_auto_split(q.tiles_n, spans);
        if (split > spans) split = spans > 0 ? (int)spans : 1;
        q.k_per_split = (int32_t)(ceil_div(spans, split) * 64);
        split = q.k_per_split > 0 ? (int)ceil_div(d.k, q.k_per_split) : 1;
        q.split_k = split;
        q.group_m = rg;
        const int64_t grid = (int64_t)q.tiles_n * split;
        if (grid > INT32_MAX) return GE_ERR_SHAPE;
        q.grid = (unsigned)grid;
        if (split > 1) {
            const size_t nbs = d.batch > 1 ? (size_t)d.batch : 1;
            q.n_counters = q.tiles_n;
            q.part_bytes = (int64_t)split * q.tiles_n * 256 * rg * (int64_t)sizeof(float);
            q.ws_partial = round_up(nbs * (size_t)q.part_bytes, 256);
            q.ws_counters = round_up(nbs * (size_t)q.n_counters * sizeof(uint32_t), 256);
        }
    } else {
        q.tile_id = pr.tile ? pr.tile : choose_tile(d.m, d.n, d.a_type, d.d_type);
        // the automatic split-K 64 x 64 tile serves problems with so few tiles
        // and so long a K that the slices' parallelism outweighs their
        // partial exchange: at most 64 tiles with k >= 4096, or at most 128
        // with k >= 8192 (measured: 1024 x 512 x 8192 takes 29.2 us unsplit
        // and 22.6 us in 2 slices; 1024 x 512 x 2048 10.8 us unsplit and
        // 12.9 / 13.9 us in 2 / 4); the bias-gradient partials would share
        // its partial buffer
        const int64_t t64 = ceil_div(d.m, 64) * ceil_div(d.n, 64);
        if (!pr.tile && q.tile_id == 13 && !is_bgrad(epilog) &&
            ((t64 <= 64 && d.k >= 4096) || (t64 <= 128 && d.k >= 8192)))
            q.tile_id = 14;
        const TileShape* t = find_tile(q.tile_id);
        if (!tile_supports(t, d.a_type, d.d_type)) return GE_ERR_SHAPE;
        if (!tile_span_ok(t, d)) {
            if (pr.tile || d.a_type == GE_MXF8_E4M3 || d.d_type == GE_F8_E4M3) return GE_ERR_SHAPE;
            q.tile_id = choose_tile_plain(d.m, d.n);
            t = find_tile(q.tile_id);
        }
        if (pr.split_k > 1 && t->kernel != 5) return GE_ERR_SHAPE;   // only the split-K tile splits K
        if (t->kernel == 5 && is_bgrad(epilog)) return GE_ERR_EPILOG;
        const int64_t tm = ceil_div(d.m, t->bm), tn = ceil_div(d.n, t->bn);
        if (tm * tn > INT32_MAX) return GE_ERR_SHAPE;
        q.tiles_m = (int32_t)tm;
        q.tiles_n = (int32_t)tn;
        q.group_m = pr.group_m > 0 ? (int32_t)(pr.group_m < tm ? pr.group_m : (tm > 0 ? tm : 1))
                                   : auto_group_m(t, tm, d.a_type);
        q.grid = (unsigned)(tm * tn);
        q.k_per_split = (int32_t)d.k;
        q.k_stagger = auto_k_stagger(t, d.a_type);
        if (t->kernel == 5) {
            // K slices of whole 64-element steps: the largest power of two
            // that keeps the grid within 256 workgroups, every slice at 16 or
            // more steps (32 beyond 128 workgroups) and the split at most 8
            // (16 for at most 4 tiles), unless forced.  The last slice of a tile reads every partial, so
            // beyond that more slices cost more than they gain.  Measured
            // (bf16, the best split and its time): 128 x 128 x 65536 16,
            // 25.9 us (30.0 at 32); 256 x 256 x 4096 4, 12.4; 256 x 256 x
            // 8192 4-8, 14.6; 256 x 256 x 65536 8, 38.4 (41.4 at 16, 180 us
            // unsplit); 256 x 512 x 32768 8, 33.7; 512 x 512 x 8192 4, 17.5;
            // 512 x 512 x 16384 4, 23.5; 1024 x 512 x 16384 2, 37.8;
            // 1024 x 512 x 2048 1, 10.8 (12.9 in 2 slices of 16 steps)
            const int64_t steps = ceil_div(d.k, 64);
            int split = pr.split_k;
            if (split <= 0) {
                const int cap = tm * tn <= 4 ? 16 : 8;
                split = 1;
                while (split * 2 <= cap && tm * tn * split * 2 <= 256 &&
                       steps >= split * 2 * (tm * tn * split * 2 > 128 ? 32 : 16))
                    split *= 2;
            }
            if (split > steps) split = steps > 0 ? (int)steps : 1;
            if (split > 65535) return GE_ERR_SHAPE;
            q.k_per_split = (int32_t)(ceil_div(steps, split) * 64);
            split = q.k_per_split > 0 ? (int)ceil_div(d.k, q.k_per_split) : 1;
            q.split_k = split;
            if (split > 1) {
                const size_t nbs = d.batch > 1 ? (size_t)d.batch : 1;
                q.n_counters = tm * tn;
                q.part_bytes = tm * tn * split * (int64_t)t->bm * t->bn * (int64_t)sizeof(float);
                q.ws_partial = round_up(nbs * (size_t)q.part_bytes, 256);
                q.ws_counters = round_up(nbs * (size_t)q.n_counters * sizeof(uint32_t), 256);
            }
        }
    }
    const size_t nb = d.batch > 1 ? (size_t)d.batch : 1;   // products per launch
    q.ws_c = q.unfused ? round_up(nb * (size_t)d.m * (size_t)d.ldd * elem_size(d.d_type), 256) : 0;
    // bias gradient: one fp32 partial per tile row (COL) or column (ROW) and
    // gradient entry; the unfused pair sums its stored D in blocks of 256
    q.ws_bgrad = 0;
    q.bgrad_parts = 0;
    if (is_bgrad(epilog)) {
        const bool col = bias_axis == GE_BIAS_COL;
        const int64_t parts = q.unfused ? ceil_div(col ? d.m : d.n, 256) : (col ? q.tiles_m : q.tiles_n);
        if (parts > 65535) return GE_ERR_SHAPE;
        q.bgrad_parts = (int32_t)parts;
        q.ws_bgrad = round_up(nb * (size_t)parts * (size_t)(col ? d.n : d.m) * sizeof(float), 256);
    }
    q.planned = true;
    q.pref = pr;
    *h = q;
    if (plan_log()) {
        char line[512];
        gemm_epilog_describe(h, line, sizeof line);
        fprintf(stderr, "gemm_epilog: plan %s\n", line);
    }
    return GE_OK;
}

int gemm_epilog_workspace_size(ge_handle h, size_t* bytes) {
    if (!h || !bytes) return GE_ERR_NULL;
    if (!h->planned) return GE_ERR_STATE;
    *bytes = h->ws_c + h->ws_partial + h->ws_counters + h->ws_bgrad;
    return GE_OK;
}

int gemm_epilog_aux_ld(ge_handle h, int64_t* ld_bits) {
    if (!h || !ld_bits) return GE_ERR_NULL;
    const int64_t ld = (int64_t)round_up((size_t)h->d.n, 128);
    *ld_bits = (h->planned && aux_is_matrix(h->epilog)) ? ld * 8 * elem_size(h->d.d_type) : ld;
    return GE_OK;
}

// execute and execute_c: cin (NULL = no added term) is C in D's dtype with
// row stride ldc, scaled by the device scalar *beta.  static_ws: the
// workspace is the library's own array (execute_static), not the caller's.
// Per-product byte strides of a launch (the packed layout unless the caller
// set strides), validated: GE_OK or an error status.
struct ProductStrides {
    int64_t a, b, bias, d, aux, c, sa, sb;
};

static int product_strides(const ge_plan_s& h, int64_t ldc, ProductStrides* out) {
    const ge_desc& d = h.d;
    const int64_t ea = elem_size(d.a_type), ed = elem_size(d.d_type), eb = elem_size(d.bias_type);
    const bool aux_matrix = aux_is_matrix(h.epilog);
    const int64_t aux_es = aux_matrix ? ed : 4;
    const int64_t len = h.axis == GE_BIAS_ROW ? d.m : d.n;
    const int64_t mx_ld = GE_MX_SCALE_LD(d.k);
    ge_batch_strides s = {d.m * d.lda, (d.op_b == GE_OP_N ? d.k : d.n) * d.ldb, len, d.m * d.ldd,
                          d.m * h.ldaux};
    if (h.bstr_set && d.batch > 1) {
        s = h.bstr;
        // inputs: any stride (0 shares one operand); rows stay 16-byte aligned
        if ((s.a * ea) % 16 || (s.b * ea) % 16 || (s.d * ed) % 16 || (s.aux * aux_es) % 16) return GE_ERR_ALIGN;
        if (h.axis == GE_BIAS_COL && has_bias(h.epilog) && (s.bias * eb) % 16) return GE_ERR_ALIGN;
        // outputs: no two products may write the same element
        if (s.d < (d.m - 1) * d.ldd + d.n) return GE_ERR_SHAPE;
        const bool aux_out = h.epilog == GE_EPILOG_RELU_AUX_BIAS || h.epilog == GE_EPILOG_GELU_AUX_BIAS;
        if (aux_out && s.aux < d.m * h.ldaux) return GE_ERR_SHAPE;
        if (is_bgrad(h.epilog) && s.bias < len) return GE_ERR_SHAPE;
    }
    out->a = s.a * ea;
    out->b = s.b * ea;
    out->bias = s.bias * eb;
    out->d = s.d * ed;
    out->aux = s.aux * aux_es;
    out->c = d.m * ldc * ed;
    out->sa = d.m * mx_ld;
    out->sb = d.n * mx_ld;
    return GE_OK;
}

// m_run < 0: the planned m; else the rows of this call (0 .. planned m).
static int execute_impl(ge_handle h, const void* A, const void* B, const void* cin, int64_t ldc, const float* beta,
                        const void* bias, void* D, void* aux, const float* scale_a, const float* scale_b,
                        void* workspace, size_t workspace_bytes, void* stream, bool static_ws = false,
                        const void* mx_a = nullptr, const void* mx_b = nullptr, int64_t m_run = -1) {
    if (!h) return GE_ERR_NULL;
    if (!h->planned) return GE_ERR_STATE;
    const ge_desc& d = h->d;
    if (m_run > d.m) return GE_ERR_SHAPE;
    const int64_t M = m_run >= 0 ? m_run : d.m;   // rows of this call
    // block-scaled fp8: the scales come with execute_mx, and only with it
    const bool mx = d.a_type == GE_MXF8_E4M3;
    if (!mx && (mx_a || mx_b)) return GE_ERR_DTYPE;
    if (mx && ((!mx_a && M * d.k > 0) || (!mx_b && d.n * d.k > 0))) return GE_ERR_NULL;
    if (!aligned(mx_a, 16) || !aligned(mx_b, 16)) return GE_ERR_ALIGN;
    // a pointer may be NULL only when its buffer holds no elements
    if ((!A && M * d.k > 0) || (!B && d.k * d.n > 0) || (!D && M * d.n > 0)) return GE_ERR_NULL;
    const int64_t bias_len = h->axis == GE_BIAS_ROW ? M : d.n;
    if ((has_bias(h->epilog) || is_bgrad(h->epilog)) && !bias && bias_len > 0) return GE_ERR_NULL;
    const bool want_aux = has_aux(h->epilog) && M > 0 && d.n > 0;   // else aux holds nothing
    if (aux && !has_aux(h->epilog)) return GE_ERR_EPILOG;
    if (want_aux && !aux) return GE_ERR_EPILOG;
    if (cin) {
        if (h->d.d_type == GE_F8_E4M3) return GE_ERR_DTYPE;
        if (ldc < h->d.n) return GE_ERR_SHAPE;
        if ((ldc * elem_size(h->d.d_type)) % 16 || !aligned(cin, 16) || !aligned(beta, 4)) return GE_ERR_ALIGN;
    }
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || !aligned(bias, 16) || !aligned(aux, 16) ||
        !aligned(workspace, 16) || !aligned(scale_a, 4) || !aligned(scale_b, 4))
        return GE_ERR_ALIGN;
    ProductStrides ps;
    {
        const int st = product_strides(*h, cin ? ldc : 0, &ps);
        if (st != GE_OK) return st;
    }
    const size_t need = h->ws_c + h->ws_partial + h->ws_counters + h->ws_bgrad;
    if (static_ws) {
        if (need > (size_t)GE_STATIC_WORKSPACE_BYTES) return GE_ERR_STATIC_LIMIT;
    } else if (need > 0 && (!workspace || workspace_bytes < need)) {
        return GE_ERR_WORKSPACE;
    }
    if (test_fail_launch()) return GE_ERR_HIP;
    if (static_ws && need > 0) {
        // validation is done: only now the first HIP call
        const int st = scratch_of_current_device(&workspace);
        if (st != GE_OK) return st;
        workspace_bytes = (size_t)GE_STATIC_WORKSPACE_BYTES;
    }
    // fp8 output: amax starts from 0 at every call (a kernel, so that the
    // call can be captured in a HIP graph)
    if (h->amax_d && launch_clear_counters((uint32_t*)h->amax_d, d.batch > 1 ? d.batch : 1, stream) != 0)
        return GE_ERR_HIP;
    if (M == 0 || d.n == 0) {
        // empty output; a bias gradient over no rows (or columns) is zero
        if (is_bgrad(h->epilog) && bias_len > 0) {
            KernelArgs z;
            memset(&z, 0, sizeof(z));
            z.bias = bias;
            z.m = (int32_t)M;
            z.n = (int32_t)d.n;
            z.axis = h->axis;
            z.batch = d.batch > 1 ? d.batch : 1;
            z.bs_bias = ps.bias;
            if (launch_bgrad_reduce(d.d_type, z, 0, stream) != 0) return GE_ERR_HIP;
        }
        return GE_OK;
    }

    KernelArgs a;
    memset(&a, 0, sizeof(a));
    a.A = A;
    a.B = B;
    a.bias = bias;
    a.D = D;
    a.aux = (uint32_t*)aux;
    a.scale_a = scale_a;
    a.scale_b = scale_b;
    a.m = (int32_t)M;
    a.n = (int32_t)d.n;
    a.k = (int32_t)d.k;
    a.epilog = h->epilog;
    a.axis = h->axis;
    a.ldaux = (int32_t)h->ldaux;
    a.lda = d.lda;
    a.ldb = d.ldb;
    a.ldd = d.ldd;
    a.tiles_m = h->tiles_m;
    a.tiles_n = h->tiles_n;
    a.group_m = h->group_m;
    a.split_k = h->split_k;
    a.k_per_split = h->k_per_split;
    a.k_stagger = h->k_stagger;
    unsigned grid = h->grid;
    int32_t bgrad_parts = h->bgrad_parts;
    if (h->path != PATH_SMALLM && M != d.m) {
        // fewer rows than planned: the same kernel over the tile rows there are
        const TileShape* t = find_tile(h->tile_id);
        a.tiles_m = (int32_t)ceil_div(M, t->bm);
        grid = (unsigned)(a.tiles_m * (int64_t)a.tiles_n);
        if (is_bgrad(h->epilog) && h->axis == GE_BIAS_COL)
            bgrad_parts = (int32_t)(h->unfused ? ceil_div(M, 256) : a.tiles_m);
    }
    // batched: per-product strides in bytes (counters: elements); the
    // workspace parts keep their planned (largest) size
    const int64_t len = h->axis == GE_BIAS_COL ? d.n : d.m;
    a.batch = d.batch > 1 ? d.batch : 1;
    a.bs_part = h->split_k > 1 ? h->part_bytes : (int64_t)h->bgrad_parts * len * (int64_t)sizeof(float);
    a.bs_cnt = h->n_counters;
    a.bs_a = ps.a;
    a.bs_b = ps.b;
    a.bs_bias = ps.bias;
    a.bs_d = ps.d;
    a.bs_aux = ps.aux;
    a.bs_c = ps.c;
    a.cin = cin;
    a.beta = beta;
    a.ldc = ldc;
    a.scale_d = h->scale_d;
    a.amax = h->amax_d;
    uint8_t* ws = (uint8_t*)workspace;
    if (h->split_k > 1) {
        a.partial = (float*)(ws + h->ws_c);
        a.counters = (uint32_t*)(ws + h->ws_c + h->ws_partial);
        if (launch_clear_counters(a.counters, (int)(h->n_counters * a.batch), stream) != 0) return GE_ERR_HIP;
    }

    if (is_bgrad(h->epilog)) a.partial = (float*)(ws + h->ws_c + h->ws_partial + h->ws_counters);

    KernelArgs k1 = a;
    if (h->unfused) {
        // kernel 1: the plain product, rounded to d_type, into the workspace
        k1.epilog = GE_EPILOG_NONE;
        k1.cin = nullptr;   // the second kernel adds beta * C
        k1.bias = nullptr;
        k1.aux = nullptr;
        k1.ldaux = 0;
        k1.D = ws;
        k1.bs_d = M * d.ldd * elem_size(d.d_type);   // packed, as the second kernel reads it
    }
    int err;
    if (h->path == PATH_SMALLM) {
        err = launch_smallm(d.a_type, d.d_type, d.op_b, h->group_m, k1, grid, stream);
    } else if (mx) {
        const MxArgs mxa = {(const uint8_t*)mx_a, (const uint8_t*)mx_b, (int32_t)GE_MX_SCALE_LD(d.k),
                            (int32_t)ceil_div(d.k, 32), ps.sa, ps.sb};
        err = launch_tile_mx(h->tile_id, d.d_type, d.op_b, k1, mxa, grid, stream);
    } else {
        err = launch_tile(h->tile_id, d.a_type, d.d_type, d.op_b, k1, grid, stream);
    }
    if (err != 0) return GE_ERR_HIP;
    if (h->unfused) {
        // kernel 2: D = act(C + bias) (+ mask)
        err = launch_elementwise(d.d_type, a, ws, stream);
        if (err != 0) return GE_ERR_HIP;
        // the bias gradient of the stored D
        if (is_bgrad(h->epilog) && launch_bgrad_sum(d.d_type, a, bgrad_parts, stream) != 0)
            return GE_ERR_HIP;
    }
    if (is_bgrad(h->epilog) && launch_bgrad_reduce(d.d_type, a, bgrad_parts, stream) != 0) return GE_ERR_HIP;
    return GE_OK;
}

int gemm_epilog_execute(ge_handle h, const void* A, const void* B, const void* bias, void* D, void* aux,
                        const float* scale_a, const float* scale_b, void* workspace, size_t workspace_bytes,
                        void* stream) {
    return execute_impl(h, A, B, nullptr, 0, nullptr, bias, D, aux, scale_a, scale_b, workspace, workspace_bytes,
                        stream);
}

int gemm_epilog_execute_c(ge_handle h, const void* A, const void* B, const void* C, int64_t ldc,
                          const float* beta, const void* bias, void* D, void* aux, const float* scale_a,
                          const float* scale_b, void* workspace, size_t workspace_bytes, void* stream) {
    if (!h) return GE_ERR_NULL;
    if (!beta || (!C && h->d.m * h->d.n > 0)) return GE_ERR_NULL;
    return execute_impl(h, A, B, C, ldc, beta, bias, D, aux, scale_a, scale_b, workspace, workspace_bytes, stream);
}

int gemm_epilog_execute_mx(ge_handle h, const void* A, const void* B, const void* a_scales, const void* b_scales,
                           const void* bias, void* D, void* aux, const float* scale_a, const float* scale_b,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (!h) return GE_ERR_NULL;
    if (h->d.a_type != GE_MXF8_E4M3) return GE_ERR_DTYPE;
    return execute_impl(h, A, B, nullptr, 0, nullptr, bias, D, aux, scale_a, scale_b, workspace, workspace_bytes,
                        stream, false, a_scales, b_scales);
}

int gemm_epilog_execute_m(ge_handle h, int64_t m, const void* A, const void* B, const void* bias, void* D,
                          void* aux, const float* scale_a, const float* scale_b, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (!h) return GE_ERR_NULL;
    if (m < 0 || m > h->d.m) return GE_ERR_SHAPE;
    if (h->d.a_type == GE_MXF8_E4M3) return GE_ERR_DTYPE;   // block scales come with execute_mx
    return execute_impl(h, A, B, nullptr, 0, nullptr, bias, D, aux, scale_a, scale_b, workspace, workspace_bytes,
                        stream, false, nullptr, nullptr, m);
}

int gemm_epilog_set_fp8_output(ge_handle h, const float* scale_d, float* amax_d) {
    if (!h) return GE_ERR_NULL;
    if (h->d.d_type != GE_F8_E4M3) return GE_ERR_DTYPE;
    if (!aligned(scale_d, 4) || !aligned(amax_d, 4)) return GE_ERR_ALIGN;
    h->scale_d = scale_d;
    h->amax_d = amax_d;
    return GE_OK;
}

int gemm_epilog_set_batch_strides(ge_handle h, const ge_batch_strides* s) {
    if (!h) return GE_ERR_NULL;
    if (!s) {
        h->bstr_set = false;
        return GE_OK;
    }
    if (s->a < 0 || s->b < 0 || s->bias < 0 || s->d < 0 || s->aux < 0) return GE_ERR_SHAPE;
    h->bstr = *s;
    h->bstr_set = true;
    return GE_OK;
}

int gemm_epilog_execute_static(ge_handle h, const void* A, const void* B, const void* bias, void* D, void* aux,
                               const float* scale_a, const float* scale_b, void* stream) {
    return execute_impl(h, A, B, nullptr, 0, nullptr, bias, D, aux, scale_a, scale_b, nullptr, 0, stream, true);
}

int gemm_epilog_free(ge_handle h) {
    delete h;
    return GE_OK;
}

const char* gemm_epilog_status_string(int s) {
    switch (s) {
    case GE_OK: return "GE_OK: success";
    case GE_ERR_NULL: return "GE_ERR_NULL: a required pointer is NULL";
    case GE_ERR_SHAPE: return "GE_ERR_SHAPE: invalid dimension, leading dimension or plan option";
    case GE_ERR_DTYPE: return "GE_ERR_DTYPE: unsupported or mismatched dtypes";
    case GE_ERR_EPILOG: return "GE_ERR_EPILOG: invalid epilogue, bias axis or aux buffer";
    case GE_ERR_ALIGN: return "GE_ERR_ALIGN: pointer or row stride not 16-byte aligned";
    case GE_ERR_STATE: return "GE_ERR_STATE: handle not planned";
    case GE_ERR_WORKSPACE: return "GE_ERR_WORKSPACE: workspace missing or too small";
    case GE_ERR_HIP: return "GE_ERR_HIP: kernel launch failed";
    case GE_ERR_ALLOC: return "GE_ERR_ALLOC: host allocation failed";
    case GE_ERR_STATIC_LIMIT:
        return "GE_ERR_STATIC_LIMIT: the plan needs more workspace than the library's fixed array "
               "(GE_STATIC_WORKSPACE_BYTES)";
    }
    return "unknown status";
}

int gemm_epilog_autotune(ge_handle h, const void* A, const void* B, const void* bias, void* D, void* aux,
                         const float* scale_a, const float* scale_b, void* workspace, size_t workspace_bytes,
                         int32_t iters, void* stream, float* best_ms) {
    if (!h) return GE_ERR_NULL;
    if (!h->planned) return GE_ERR_STATE;
    if (iters < 1) return GE_ERR_SHAPE;
    const ge_plan_s orig = *h;
    // candidates: tile ids (tile path) or row groups x K splits (small-m
    // path, encoded as 256 * row groups + split)
    int cand[kNumTiles + 24];
    int nc = 0;
    if (orig.path == PATH_SMALLM) {
        const int64_t spans = ceil_div(orig.d.k, 64);
        for (int rg = 1; rg <= 4; rg *= 2)
            for (int s = 1; s <= 64 && s <= (spans > 0 ? spans : 1); s *= 2) cand[nc++] = 256 * rg + s;
    } else {
        for (int i = 0; i < kNumTiles; ++i) cand[nc++] = kTiles[i].id;
    }
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return GE_ERR_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return GE_ERR_HIP;
    }
    ge_plan_s best = orig;
    float best_t = -1.0f;
    int status = GE_OK;
    for (int c = 0; c < nc && status == GE_OK; ++c) {
        ge_pref pr = orig.pref;
        if (orig.path == PATH_SMALLM) {
            pr.path = PATH_SMALLM;
            pr.group_m = cand[c] / 256;
            pr.split_k = cand[c] % 256;
        } else {
            pr.path = PATH_TILE;
            pr.tile = cand[c];
        }
        ge_plan_s trial = orig;
        if (gemm_epilog_plan(&trial, orig.epilog, orig.axis, &pr) != GE_OK) continue;   // not for this dtype
        size_t need = 0;
        gemm_epilog_workspace_size(&trial, &need);
        if (need > workspace_bytes) continue;
        // one untimed call (also validates the arguments), then the timed ones
        int r = gemm_epilog_execute(&trial, A, B, bias, D, aux, scale_a, scale_b, workspace, workspace_bytes,
                                    stream);
        if (r != GE_OK) {
            status = r;
            break;
        }
        if (hipEventRecord(e0, (hipStream_t)stream) != hipSuccess) { status = GE_ERR_HIP; break; }
        for (int i = 0; i < iters && r == GE_OK; ++i)
            r = gemm_epilog_execute(&trial, A, B, bias, D, aux, scale_a, scale_b, workspace, workspace_bytes,
                                    stream);
        if (r != GE_OK) { status = r; break; }
        float ms = 0.0f;
        if (hipEventRecord(e1, (hipStream_t)stream) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
            status = GE_ERR_HIP;
            break;
        }
        ms /= (float)iters;
        if (best_t < 0.0f || ms < best_t) {
            best_t = ms;
            best = trial;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (status != GE_OK) return status;
    if (best_t < 0.0f) return GE_ERR_WORKSPACE;   // no candidate fits the workspace
    best.pref = orig.pref;
    *h = best;
    if (best_ms) *best_ms = best_t;
    return GE_OK;
}

int gemm_epilog_describe(ge_handle h, char* buf, size_t cap) {
    if (!h || !buf) return GE_ERR_NULL;
    if (cap == 0) return GE_OK;
    const ge_desc& d = h->d;
    if (!h->planned) {
        snprintf(buf, cap, "m=%lld n=%lld k=%lld unplanned", (long long)d.m, (long long)d.n, (long long)d.k);
        return GE_OK;
    }
    const TileShape* t = find_tile(h->tile_id);
    snprintf(buf, cap,
             "m=%lld n=%lld k=%lld a=%d d=%d op_b=%d epilog=%d axis=%d path=%s tile=%dx%d waves=%dx%d "
             "tile_id=%d kernel=%d stages=%d grid=%u group_m=%d split_k=%d unfused=%d workspace=%zu "
             "ldaux_words=%lld k_stagger=%d",
             (long long)d.m, (long long)d.n, (long long)d.k, d.a_type, d.d_type, d.op_b, h->epilog, h->axis,
             h->path == PATH_SMALLM ? "smallm" : "tile", t ? t->bm : 16, t ? t->bn : 16 * h->group_m, t ? t->wm : 1,
             t ? t->wn : 8, h->tile_id, t ? t->kernel : 0,
             t ? (t->kernel >= 2 && t->kernel != 3 ? tile2_stages(*t, elem_size(d.a_type)) : t->stages) : 0, h->grid, h->group_m,
             h->split_k,
             h->unfused,
             h->ws_c + h->ws_partial + h->ws_counters + h->ws_bgrad, (long long)h->ldaux,
             h->k_stagger);
    return GE_OK;
}

}  // extern "C"
