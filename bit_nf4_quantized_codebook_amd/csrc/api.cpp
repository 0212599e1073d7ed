// C ABI of the NF4 quantized-codebook linear layer: argument validation, workspace planning and
// launch sequencing on the caller's stream.  Declarations and contracts: include/nf4.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/nf4.h"
#include "launch.h"

// ---------------------------------------------------------------------------------------------
// Static scratch of the forward entry point that allocates nothing (qlora_linear_fwd_static).
// Each GPU the library runs on holds its own copy from module load until the process ends.  In
// host code the name is a host-side stand-in, not a device address: host code uses only the
// address hipGetSymbolAddress returns for the current device (static_scratch below).  Every call
// on one GPU shares the array.
// ---------------------------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = QLORA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, const char *detail = nullptr) {
    if (detail) std::snprintf(g_last_error, sizeof g_last_error, fmt, detail);
    else std::snprintf(g_last_error, sizeof g_last_error, "%s", fmt);
    return status;
}

int hip_fail(hipError_t e, const char *where) {
    std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(e));
    return NF4_ERR_HIP;
}

#define NF4_CHECK_HIP(expr, where)                \
    do {                                          \
        hipError_t e_ = (expr);                   \
        if (e_ != hipSuccess) return hip_fail(e_, where); \
    } while (0)

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------------------------------------
// Standard normal quantile: Halley iteration on the CDF (via erfc, tail-aware form), started from
// the rational approximation of Abramowitz & Stegun 26.2.23.
// ---------------------------------------------------------------------------------------------
double upper_tail(double x) { return 0.5 * std::erfc(x / std::sqrt(2.0)); }   // Q(x) = 1 - Phi(x)

double normal_quantile(double p) {
    const double q = (p < 0.5) ? p : 1.0 - p;      // exact for p >= 0.5 (Sterbenz)
    const double t = std::sqrt(-2.0 * std::log(q));
    double z = t - (2.515517 + 0.802853 * t + 0.010328 * t * t) /
                       (1.0 + 1.432788 * t + 0.189269 * t * t + 0.001308 * t * t * t);
    // z approximates the upper-tail point: Q(z) = q, z >= 0
    if (q == 0.5) return 0.0;
    const double inv_sqrt_2pi = 0.39894228040143267794;
    for (int it = 0; it < 100; ++it) {
        const double f = upper_tail(z) - q;             // decreasing in z
        const double dens = inv_sqrt_2pi * std::exp(-0.5 * z * z);
        const double u = -f / dens;                      // Newton step for Q(z) = q
        const double step = u / (1.0 + 0.5 * z * u);     // Halley correction (Q'' = z * dens)
        const double zn = z - step;
        if (zn == z || std::fabs(step) <= 1e-17 * std::fabs(z)) { z = zn; break; }
        z = zn;
    }
    return (p < 0.5) ? -z : z;
}

// Largest float f with f <= (a + b) / 2, computed exactly (TwoSum keeps the rounding error).
float threshold_below_midpoint(float a, float b) {
    const double s = (double)a + (double)b;
    const double bv = s - (double)a;
    const double err = ((double)a - (s - bv)) + ((double)b - bv);
    const double hs = s * 0.5, he = err * 0.5;
    auto above = [&](float f) { return ((double)f - hs) > he; };   // f > midpoint
    float t = (float)hs;
    while (above(t)) t = std::nextafterf(t, -INFINITY);
    for (;;) {
        const float u = std::nextafterf(t, INFINITY);
        if (!above(u)) t = u; else break;
    }
    return t;
}

// Ascending (equal neighbours allowed), finite, containing 0; the zero code is the first 0 entry.
int check_codebook(const float cb[16], int *zero_code) {
    int z = -1;
    for (int j = 0; j < 16; ++j) {
        if (!std::isfinite(cb[j])) return fail(NF4_ERR_ARG, "codebook entries must be finite");
        if (j > 0 && !(cb[j - 1] <= cb[j])) return fail(NF4_ERR_ARG, "codebook must be ascending");
        if (cb[j] == 0.0f && z < 0) z = j;
    }
    if (z < 0) return fail(NF4_ERR_ARG, "codebook must contain 0.0f");
    *zero_code = z;
    return NF4_OK;
}

// Decision thresholds of the nearest-codeword search: the code is the number of thresholds
// strictly below n.  thr[j] separates codes j and j + 1; for equal neighbours code j + 1 must never
// win (ties go to the lower index), so its threshold is the next one up (+inf past the end).
void code_thresholds(const float cb[16], float thr[15]) {
    for (int j = 14; j >= 0; --j) {
        if (cb[j] == cb[j + 1]) thr[j] = (j == 14) ? INFINITY : thr[j + 1];
        else thr[j] = threshold_below_midpoint(cb[j], cb[j + 1]);
    }
}

int check_weight(const nf4_weight *w) {
    if (!w) return fail(NF4_ERR_NULL, "weight descriptor is NULL");
    if (!w->packed || !w->absmax_q || !w->absmax_scale || !w->absmax_mean)
        return fail(NF4_ERR_NULL, "weight descriptor has a NULL pointer");
    if (w->rows <= 0 || w->cols <= 0) return fail(NF4_ERR_SHAPE, "weight rows and cols must be > 0");
    if (w->block != 64) return fail(NF4_ERR_UNSUPPORTED, "block must be 64");
    if (w->dq_block != 256) return fail(NF4_ERR_UNSUPPORTED, "dq_block must be 256");
    if (w->dq_format != NF4_DQ_E4M3 && w->dq_format != NF4_DQ_INT8)
        return fail(NF4_ERR_ARG, "dq_format must be NF4_DQ_E4M3 or NF4_DQ_INT8");
    if (!aligned16(w->packed)) return fail(NF4_ERR_ALIGN, "packed weight must be 16-byte aligned");
    int zc;
    return check_codebook(w->codebook, &zc);
}

nf4k::WeightView view_of(const nf4_weight *w) {
    nf4k::WeightView v;
    v.packed = w->packed;
    v.c2 = w->absmax_q;
    v.c1 = w->absmax_scale;
    v.mean = w->absmax_mean;
    v.rows = w->rows;
    v.cols = w->cols;
    for (int j = 0; j < 16; ++j) v.cb[j] = w->codebook[j];
    v.dq_int8 = w->dq_format == NF4_DQ_INT8 ? 1u : 0u;
    return v;
}

// ---------------------------------------------------------------------------------------------
// Workspace plan of the linear layer (identical for the size query and the calls)
// ---------------------------------------------------------------------------------------------
constexpr int64_t kTile = 64;
constexpr int64_t kGemvMaxM = 64;     // token counts whose forward is a weight-streaming GEMV
// Up to this many bytes of T's float32 partials, each wide-GEMV workgroup that needs s T sums them
// itself (no reduction launch); beyond, their reading costs the GEMV more than the launch
constexpr size_t kGemvTSumBytes = 128 << 10;
// From this many tokens on, the weight is expanded to bf16 once per call and multiplied by a plain
// bf16 GEMM: the expansion pass costs about 2.5 bytes of HBM traffic per weight, while dequantizing
// inside the GEMM repeats the work once per 256-row tile of tokens and its VALU work does not hide
// under the MFMAs on gfx950.
constexpr int64_t kExpandMinM = 1024;
// The bf16 copy of the weight may exceed 2 GiB: the expansion kernels write it through 64-bit
// pointers, and each GEMM tile bases its buffer descriptor at its own first row and reads 256 rows
// of at most 2^20 elements from there (the 2 GiB operand limits on X and dY bound the reduction
// length once M >= kExpandMinM), so every offset stays far below 2^31.
bool use_expand(int64_t M, int64_t N, int64_t K) {
    (void)N;
    (void)K;
    return M >= kExpandMinM;
}

struct Plan {
    int ksT, ksdT, msL2, msL1;
    // split of the forward and backward products' reductions over workgroups (1: none)
    nf4k::SplitPlan kf, kb;
    size_t off_T, off_sT, off_dT, off_P, off_Yp, off_Tp, off_Wd, off_L2T, off_Pg, total;
};

constexpr int64_t kGemmTile = 256;   // output tile of the product kernels (both dims)
constexpr int kSplitQuantum = 4;     // reduction steps per split: a multiple of 4

// the products' splits: forward [M, N] over K (the wide GEMV's own rule up to kGemvMaxM tokens,
// none for the decode GEMV), backward [M, K] over N
void plan_splits(Plan &p, int64_t M, int64_t N, int64_t K, int32_t r) {
    const int64_t mt = (M + kGemmTile - 1) / kGemmTile;
    p.kf = p.kb = nf4k::SplitPlan{1, 0};
    if (M > kGemvMaxM)
        p.kf = nf4k::gemm_split(mt * ((N + kGemmTile - 1) / kGemmTile), (K + kTile - 1) / kTile, kSplitQuantum);
    else if (!nf4k::gemv_fits(M, N, K, r))
        p.kf = nf4k::gemv_wide_split(M, N, K);
    p.kb = nf4k::gemm_split(mt * ((K + kGemmTile - 1) / kGemmTile), (N + kTile - 1) / kTile, kSplitQuantum);
}
size_t split_floats(const Plan &p, int64_t M, int64_t N, int64_t K, bool fwd_only) {
    size_t f = p.kf.ksplit > 1 ? (size_t)p.kf.ksplit * M * N : 0;
    if (!fwd_only && p.kb.ksplit > 1) {
        const size_t b = (size_t)p.kb.ksplit * M * K;
        f = b > f ? b : f;
    }
    return f;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

Plan make_plan(int64_t M, int64_t N, int64_t K, int32_t r) {
    Plan p;
    const int64_t mt = (M + kTile - 1) / kTile, rt = (r + kTile - 1) / kTile;
    p.ksT = nf4k::choose_split(mt * rt, (K + kTile - 1) / kTile);
    if (M <= kGemvMaxM) {
        // one tile of T: four reduction steps per workgroup (one batch of loads), up to 64
        const int64_t ks4 = ((K + kTile - 1) / kTile + 3) / 4;
        if (ks4 > p.ksT) p.ksT = (int)(ks4 < 64 ? ks4 : 64);
    }
    p.ksdT = nf4k::choose_split(mt * rt, (N + kTile - 1) / kTile);
    p.msL2 = nf4k::choose_split(rt * ((N + kTile - 1) / kTile), mt);
    p.msL1 = nf4k::choose_split(((K + kTile - 1) / kTile) * rt, mt);
    size_t off = 0;
    p.off_T = off;   off += round256((size_t)M * r * 2);
    p.off_sT = off;  off += round256((size_t)M * r * 2);
    p.off_dT = off;  off += round256((size_t)M * r * 2);
    size_t pmax = (size_t)p.ksT * M * r;
    pmax = pmax > (size_t)p.ksdT * M * r ? pmax : (size_t)p.ksdT * M * r;
    // dL2 and dL1 run in one launch: their partials sit side by side
    const size_t ptn = (size_t)p.msL2 * r * N + (size_t)p.msL1 * K * r;
    pmax = pmax > ptn ? pmax : ptn;
    p.off_P = off;   off += round256(pmax * 4);
    p.off_Yp = p.off_Tp = p.off_Wd = p.off_L2T = off;
    if (use_expand(M, N, K)) {
        p.off_Wd = off;   off += round256((size_t)N * K * 2);
        p.off_L2T = off;  off += round256((size_t)N * r * 2);   // L2 transposed for the GEMM
    }
    if (nf4k::gemv_fits(M, N, K, r)) {
        const nf4k::GemvPlan g = nf4k::gemv_plan(M, N, K, r);
        p.off_Yp = off;  off += round256(g.yp_floats * 4);
        p.off_Tp = off;  off += round256(g.tp_floats * 4);
    }
    plan_splits(p, M, N, K, r);
    p.off_Pg = off;  off += round256(split_floats(p, M, N, K, false) * 4);
    p.total = off;
    return p;
}

// The forward's part of the workspace alone, packed from offset 0: s*T and T's partials (fused or
// expanded paths), the bf16 expansion and L2 transposed (from kExpandMinM tokens), or the decode
// GEMV's partials.  The split counts are make_plan's, so the kernels see the same launches.
Plan make_fwd_plan(int64_t M, int64_t N, int64_t K, int32_t r) {
    Plan p = make_plan(M, N, K, r);
    size_t off = 0;
    p.off_T = p.off_dT = 0;                      // backward only
    if (nf4k::gemv_fits(M, N, K, r)) {
        const nf4k::GemvPlan g = nf4k::gemv_plan(M, N, K, r);
        p.off_sT = p.off_P = p.off_Wd = p.off_L2T = p.off_Pg = 0;
        p.off_Yp = off;  off += round256(g.yp_floats * 4);
        p.off_Tp = off;  off += round256(g.tp_floats * 4);
        p.total = off;
        return p;
    }
    p.off_sT = off;  off += round256((size_t)M * r * 2);
    p.off_P = off;   off += round256((size_t)p.ksT * M * r * 4);
    p.off_Yp = p.off_Tp = p.off_Wd = p.off_L2T = off;
    if (use_expand(M, N, K)) {
        p.off_Wd = off;   off += round256((size_t)N * K * 2);
        p.off_L2T = off;  off += round256((size_t)N * r * 2);
    }
    p.off_Pg = off;  off += round256(split_floats(p, M, N, K, true) * 4);
    p.total = off;
    return p;
}

int check_linear_args(const nf4_weight *w, int64_t M, int32_t r, float scale) {
    int rc = check_weight(w);
    if (rc) return rc;
    if (M <= 0) return fail(NF4_ERR_SHAPE, "M must be >= 1");
    if (r < 1 || r > 128) return fail(NF4_ERR_UNSUPPORTED, "r must be in [1, 128]");
    if (r % 8) return fail(NF4_ERR_UNSUPPORTED, "r must be a multiple of 8");
    if (w->cols % 64) return fail(NF4_ERR_UNSUPPORTED, "weight cols (K) must be a multiple of 64");
    if (w->rows % 8) return fail(NF4_ERR_UNSUPPORTED, "weight rows (N) must be a multiple of 8");
    if (!std::isfinite(scale)) return fail(NF4_ERR_ARG, "scale must be finite");
    // kernels address each operand with 32-bit byte offsets
    const int64_t lim = (int64_t)1 << 31;
    if (w->rows * (w->cols / 2) >= lim || M * w->cols * 2 >= lim || M * w->rows * 2 >= lim)
        return fail(NF4_ERR_UNSUPPORTED, "an operand exceeds 2 GiB");
    return NF4_OK;
}

template <typename T>
T *ws_at(void *ws, size_t off) {
    return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off);
}

// T (unscaled) and/or s*T, both bf16 [M, r], from X [M, K] and L1 [K, r]: the split-K partials
// (launched here), and the reduction that sums them (launched by the caller, on its own or with
// the weight expansion)
nf4k::Reduction T_partials(const uint16_t *X, const uint16_t *L1, int64_t M, int64_t K, int32_t r, float scale,
                           uint16_t *T_out, uint16_t *sT_out, const Plan &p, void *ws, hipStream_t s,
                           hipError_t *err) {
    float *P = ws_at<float>(ws, p.off_P);
    *err = nf4k::launch_skinny_nt(X, L1, /*b_rows_k=*/true, P, M, r, K, p.ksT, s);
    return nf4k::Reduction{P, p.ksT, M * r, 1.0f, T_out, scale, sT_out};
}
int compute_T(const uint16_t *X, const uint16_t *L1, int64_t M, int64_t K, int32_t r, float scale,
              uint16_t *T_out, uint16_t *sT_out, const Plan &p, void *ws, hipStream_t s) {
    hipError_t e;
    const nf4k::Reduction red = T_partials(X, L1, M, K, r, scale, T_out, sT_out, p, ws, s, &e);
    NF4_CHECK_HIP(e, "T = X L1");
    NF4_CHECK_HIP(nf4k::launch_reduce_partials(red, nullptr, s), "T reduce");
    return NF4_OK;
}

struct TimingState {
    hipEvent_t *begin = nullptr, *end = nullptr;
    int32_t *kinds = nullptr;
    int32_t n = 0, count = 0;
};
thread_local TimingState g_timing;

}  // namespace

namespace nf4k {
void timing_before(hipStream_t stream, int kind) {
    if (g_timing.count < g_timing.n) {
        (void)hipEventRecord(g_timing.begin[g_timing.count], stream);
        if (g_timing.kinds) g_timing.kinds[g_timing.count] = kind;
    }
}
void timing_after(hipStream_t stream) {
    if (g_timing.count < g_timing.n) {
        (void)hipEventRecord(g_timing.end[g_timing.count], stream);
        ++g_timing.count;
    }
}
}  // namespace nf4k

// Entry points: their declarations in nf4.h give them C linkage.

int nf4_set_gemm_timing_events(void **begin, void **end, int32_t *kinds, int32_t n) {
    if (n < 0) return fail(NF4_ERR_ARG, "n must be >= 0");
    if (n > 0 && (!begin || !end)) return fail(NF4_ERR_NULL, "event arrays must be non-NULL");
    g_timing.begin = reinterpret_cast<hipEvent_t *>(begin);
    g_timing.end = reinterpret_cast<hipEvent_t *>(end);
    g_timing.kinds = kinds;
    g_timing.n = n;
    g_timing.count = 0;
    return NF4_OK;
}

int32_t nf4_gemm_timing_count(void) { return g_timing.count; }


const char *nf4_status_string(int status) {
    switch (status) {
        case NF4_OK: return "ok";
        case NF4_ERR_NULL: return "null pointer";
        case NF4_ERR_SHAPE: return "invalid shape";
        case NF4_ERR_ALIGN: return "misaligned pointer";
        case NF4_ERR_UNSUPPORTED: return "unsupported parameter";
        case NF4_ERR_WORKSPACE: return "workspace too small";
        case NF4_ERR_HIP: return "HIP runtime error";
        case NF4_ERR_ARG: return "invalid argument";
        default: return "unknown status";
    }
}

const char *nf4_last_error(void) { return g_last_error; }

const char *nf4_version(void) { return "0.1.0"; }

int nf4_build_codebook(float out_codebook[16], double delta) {
    if (!out_codebook) return fail(NF4_ERR_NULL, "out_codebook is NULL");
    if (delta == 0.0) delta = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
    if (!(delta > 0.5 && delta < 1.0)) return fail(NF4_ERR_ARG, "delta must be in (0.5, 1)");
    const double zmax = normal_quantile(delta);
    double v[16];
    int n = 0;
    for (int j = 7; j >= 1; --j) v[n++] = -(normal_quantile(0.5 + (delta - 0.5) * ((double)j / 7.0)) / zmax);
    v[n++] = 0.0;
    for (int j = 1; j <= 8; ++j) v[n++] = normal_quantile(0.5 + (delta - 0.5) * ((double)j / 8.0)) / zmax;
    for (int j = 0; j < 16; ++j) out_codebook[j] = (float)v[j];
    return NF4_OK;
}

int nf4_build_int4_codebook(float out_codebook[16]) {
    if (!out_codebook) return fail(NF4_ERR_NULL, "out_codebook is NULL");
    // two's complement k = -8 .. 7 over 7 (eq. (1) at 4 bits maps absmax to 7)
    for (int c = 0; c < 16; ++c) out_codebook[c] = (float)((double)(c - 8) / 7.0);
    return NF4_OK;
}

int nf4_build_fp4_codebook(float out_codebook[16]) {
    if (!out_codebook) return fail(NF4_ERR_NULL, "out_codebook is NULL");
    // E2M1 magnitudes: exponent field 0 is subnormal (m / 2), else 2^(e - 1) (1 + m / 2)
    double mag[8];
    for (int e = 0; e < 4; ++e)
        for (int m = 0; m < 2; ++m) mag[2 * e + m] = e == 0 ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, e - 1);
    for (int i = 0; i < 8; ++i) {
        out_codebook[7 - i] = (float)(-mag[i] / 6.0) + 0.0f;   // + 0.0f: the negative zero stored as +0
        out_codebook[8 + i] = (float)(mag[i] / 6.0);
    }
    return NF4_OK;
}

int nf4_quantize(const float *W, int64_t numel, int32_t block, const float codebook[16],
                 uint8_t *packed, float *absmax, void *stream) {
    if (!codebook) return fail(NF4_ERR_NULL, "codebook is NULL");
    if (numel < 0) return fail(NF4_ERR_SHAPE, "numel must be >= 0");
    if (block != 64) return fail(NF4_ERR_UNSUPPORTED, "block must be 64");
    int zc;
    int rc = check_codebook(codebook, &zc);
    if (rc) return rc;
    if (numel == 0) return NF4_OK;
    if (!W || !packed || !absmax) return fail(NF4_ERR_NULL, "W, packed and absmax must be non-NULL");
    if (!aligned16(W) || !aligned16(packed)) return fail(NF4_ERR_ALIGN, "W and packed must be 16-byte aligned");
    float thr[15];
    code_thresholds(codebook, thr);
    NF4_CHECK_HIP(nf4k::launch_quantize(W, numel, thr, (uint32_t)zc, packed, absmax,
                                        reinterpret_cast<hipStream_t>(stream)),
                  "quantize");
    return NF4_OK;
}

size_t nf4_double_quant_workspace_size(int64_t nblocks, int32_t dq_block) {
    (void)dq_block;
    if (nblocks <= 0) return 0;
    return nf4k::double_quant_ws(nblocks);
}

namespace {
int double_quant_impl(const float *absmax, int64_t nblocks, int32_t dq_block, uint8_t *absmax_q,
                      float *absmax_scale, float *absmax_mean, void *workspace, size_t workspace_bytes,
                      bool int8, void *stream) {
    if (nblocks <= 0) return fail(NF4_ERR_SHAPE, "nblocks must be >= 1");
    if (dq_block != 256) return fail(NF4_ERR_UNSUPPORTED, "dq_block must be 256");
    if (!absmax || !absmax_q || !absmax_scale || !absmax_mean || !workspace)
        return fail(NF4_ERR_NULL, "double quant pointers must be non-NULL");
    if (!aligned16(absmax) || !aligned16(absmax_q) || !aligned16(workspace))
        return fail(NF4_ERR_ALIGN, "absmax, absmax_q and workspace must be 16-byte aligned");
    if (workspace_bytes < nf4k::double_quant_ws(nblocks))
        return fail(NF4_ERR_WORKSPACE, "double quant workspace too small");
    NF4_CHECK_HIP(nf4k::launch_double_quant(absmax, nblocks, absmax_q, absmax_scale, absmax_mean,
                                            workspace, int8, reinterpret_cast<hipStream_t>(stream)),
                  "double quant");
    return NF4_OK;
}
}  // namespace

int nf4_double_quant(const float *absmax, int64_t nblocks, int32_t dq_block, uint8_t *absmax_q,
                     float *absmax_scale, float *absmax_mean, void *workspace,
                     size_t workspace_bytes, void *stream) {
    return double_quant_impl(absmax, nblocks, dq_block, absmax_q, absmax_scale, absmax_mean, workspace,
                             workspace_bytes, false, stream);
}

int nf4_double_quant_int8(const float *absmax, int64_t nblocks, int32_t dq_block, uint8_t *absmax_q,
                          float *absmax_scale, float *absmax_mean, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return double_quant_impl(absmax, nblocks, dq_block, absmax_q, absmax_scale, absmax_mean, workspace,
                             workspace_bytes, true, stream);
}

int nf4_dequant(const nf4_weight *w, uint16_t *out_bf16, void *stream) {
    int rc = check_weight(w);
    if (rc) return rc;
    if (!out_bf16) return fail(NF4_ERR_NULL, "out_bf16 is NULL");
    if (!aligned16(out_bf16)) return fail(NF4_ERR_ALIGN, "out_bf16 must be 16-byte aligned");
    const int64_t numel = w->rows * w->cols;
    if (numel % 2) return fail(NF4_ERR_SHAPE, "rows*cols must be even");
    if (numel % 64 == 0)   // whole blocks: the table-lookup expansion
        NF4_CHECK_HIP(nf4k::launch_expand_weight(view_of(w), /*transposed=*/false, out_bf16, nullptr,
                                                 reinterpret_cast<hipStream_t>(stream)),
                      "dequant");
    else
        NF4_CHECK_HIP(nf4k::launch_dequant(w->packed, w->absmax_q, w->absmax_scale, w->absmax_mean, nullptr,
                                           (uint32_t)w->dq_format, numel, w->codebook, out_bf16, reinterpret_cast<hipStream_t>(stream)),
                      "dequant");
    return NF4_OK;
}

int nf4_dequant_single(const uint8_t *packed, const float *absmax, int64_t numel, int32_t block,
                       const float codebook[16], uint16_t *out_bf16, void *stream) {
    if (!codebook) return fail(NF4_ERR_NULL, "codebook is NULL");
    if (numel < 0) return fail(NF4_ERR_SHAPE, "numel must be >= 0");
    if (block != 64) return fail(NF4_ERR_UNSUPPORTED, "block must be 64");
    int zc;
    int rc = check_codebook(codebook, &zc);
    if (rc) return rc;
    if (numel == 0) return NF4_OK;
    if (!packed || !absmax || !out_bf16) return fail(NF4_ERR_NULL, "packed, absmax and out_bf16 must be non-NULL");
    if (!aligned16(packed) || !aligned16(out_bf16))
        return fail(NF4_ERR_ALIGN, "packed and out_bf16 must be 16-byte aligned");
    NF4_CHECK_HIP(nf4k::launch_dequant(packed, nullptr, nullptr, nullptr, absmax, 0u, numel, codebook, out_bf16,
                                       reinterpret_cast<hipStream_t>(stream)),
                  "single-level dequant");
    return NF4_OK;
}

size_t qlora_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (M <= 0 || N <= 0 || K <= 0 || r <= 0) return 0;
    return make_plan(M, N, K, r).total;
}

int qlora_linear_route(int64_t M, int64_t N, int64_t K, int32_t r, int32_t info[4]) {
    if (!info) return fail(NF4_ERR_NULL, "info is NULL");
    if (M <= 0 || N <= 0 || K <= 0 || r <= 0) return fail(NF4_ERR_SHAPE, "M, N, K and r must be >= 1");
    const Plan p = make_plan(M, N, K, r);
    const bool gemv = nf4k::gemv_fits(M, N, K, r);
    info[0] = gemv ? 1 : (M <= kGemvMaxM ? 2 : (use_expand(M, N, K) ? 4 : 3));
    info[1] = p.kf.ksplit;
    info[2] = p.kb.ksplit;
    info[3] = use_expand(M, N, K) ? 4 : 3;
    return NF4_OK;
}

namespace {
int check_fwd_args(const nf4_weight *w, const uint16_t *X, const uint16_t *L1, const uint16_t *L2, float scale,
                   int64_t M, int32_t r, uint16_t *Y, uint16_t *T_out) {
    int rc = check_linear_args(w, M, r, scale);
    if (rc) return rc;
    if (!X || !L1 || !L2 || !Y) return fail(NF4_ERR_NULL, "X, L1, L2 and Y must be non-NULL");
    if (!aligned16(X) || !aligned16(L1) || !aligned16(L2) || !aligned16(Y) ||
        (T_out && !aligned16(T_out)))
        return fail(NF4_ERR_ALIGN, "activations and adapters must be 16-byte aligned");
    return NF4_OK;
}

nf4k::SplitK split_of(const nf4k::SplitPlan &sp, const Plan &p, void *ws) {
    return nf4k::SplitK{sp.ksplit, sp.per, ws_at<float>(ws, p.off_Pg)};
}
// the fixed-order sum of a split product's partials into out (n elements), added to what out
// holds when accumulating; nothing when the product was not split
int reduce_split(const nf4k::SplitPlan &sp, const Plan &p, void *ws, int64_t n, uint16_t *out, bool accumulate,
                 hipStream_t s) {
    if (sp.ksplit <= 1) return NF4_OK;
    nf4k::Reduction red{ws_at<float>(ws, p.off_Pg), sp.ksplit, n, 1.0f, out, 0.0f, nullptr};
    red.accum = accumulate;
    NF4_CHECK_HIP(nf4k::launch_reduce_partials(red, nullptr, s), "split product reduce");
    return NF4_OK;
}

// The forward's launches on a workspace laid out by plan p (make_plan or make_fwd_plan).
int linear_fwd_run(const nf4_weight *w, const uint16_t *X, const uint16_t *L1, const uint16_t *L2, float scale,
                   int64_t M, int32_t r, uint16_t *Y, uint16_t *T_out, const Plan &p, void *workspace,
                   hipStream_t s) {
    const int64_t N = w->rows, K = w->cols;
    if (nf4k::gemv_fits(M, N, K, r)) {
        NF4_CHECK_HIP(nf4k::launch_gemv_fwd(view_of(w), X, L1, L2, scale, r, M, Y, T_out,
                                            ws_at<float>(workspace, p.off_Yp), ws_at<float>(workspace, p.off_Tp), s),
                      "dequant GEMV (fwd)");
        return NF4_OK;
    }
    uint16_t *sT = ws_at<uint16_t>(workspace, p.off_sT);
    if (M > kGemvMaxM && use_expand(M, N, K)) {
        // T's partials; one launch expands the weight, sums them and transposes L2; the GEMM
        uint16_t *Wd = ws_at<uint16_t>(workspace, p.off_Wd);
        uint16_t *L2T = ws_at<uint16_t>(workspace, p.off_L2T);
        hipError_t e;
        const nf4k::Reduction red = T_partials(X, L1, M, K, r, scale, T_out, sT, p, workspace, s, &e);
        NF4_CHECK_HIP(e, "T = X L1");
        NF4_CHECK_HIP(nf4k::launch_expand_weight(view_of(w), /*transposed=*/false, Wd, &red, s, L2, L2T, r, N),
                      "weight expansion + T reduce + L2 transpose");
        NF4_CHECK_HIP(nf4k::launch_gemm_bf16_fwd(X, Wd, sT, L2T, r, M, N, K, Y, split_of(p.kf, p, workspace), s),
                      "bf16 GEMM (fwd)");
        return reduce_split(p.kf, p, workspace, M * N, Y, false, s);
    }
    if (M <= kGemvMaxM && (size_t)p.ksT * M * r * 4 <= kGemvTSumBytes) {
        // T's partials; the GEMV sums them itself (s T in its LDS, T_out from its first workgroup)
        hipError_t e;
        const nf4k::Reduction red = T_partials(X, L1, M, K, r, scale, T_out, nullptr, p, workspace, s, &e);
        NF4_CHECK_HIP(e, "T = X L1");
        NF4_CHECK_HIP(nf4k::launch_gemv_wide_fwd(view_of(w), X, &red, nullptr, L2, r, M, Y,
                                                 split_of(p.kf, p, workspace), s),
                      "dequant GEMV (fwd)");
        return reduce_split(p.kf, p, workspace, M * N, Y, false, s);
    }
    int rc = compute_T(X, L1, M, K, r, scale, T_out, sT, p, workspace, s);
    if (rc) return rc;
    if (M <= kGemvMaxM) {
        NF4_CHECK_HIP(nf4k::launch_gemv_wide_fwd(view_of(w), X, nullptr, sT, L2, r, M, Y,
                                                 split_of(p.kf, p, workspace), s),
                      "dequant GEMV (fwd)");
        return reduce_split(p.kf, p, workspace, M * N, Y, false, s);
    }
    NF4_CHECK_HIP(nf4k::launch_dqgemm_fwd(view_of(w), X, sT, L2, r, M, Y, split_of(p.kf, p, workspace), s),
                  "fused dequant GEMM (fwd)");
    return reduce_split(p.kf, p, workspace, M * N, Y, false, s);
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void **out) {
    int dev = -1;
    NF4_CHECK_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(NF4_ERR_UNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        NF4_CHECK_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!ptr) return fail(NF4_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return NF4_OK;
}
}  // namespace

int qlora_linear_fwd(const nf4_weight *w, const uint16_t *X, const uint16_t *L1, const uint16_t *L2,
                     float scale, int64_t M, int32_t r, uint16_t *Y, uint16_t *T_out, void *workspace,
                     size_t workspace_bytes, void *stream) {
    int rc = check_fwd_args(w, X, L1, L2, scale, M, r, Y, T_out);
    if (rc) return rc;
    const Plan p = make_plan(M, w->rows, w->cols, r);
    if (!workspace || workspace_bytes < p.total) return fail(NF4_ERR_WORKSPACE, "linear workspace too small");
    if (!aligned16(workspace)) return fail(NF4_ERR_ALIGN, "workspace must be 16-byte aligned");
    return linear_fwd_run(w, X, L1, L2, scale, M, r, Y, T_out, p, workspace, reinterpret_cast<hipStream_t>(stream));
}

int qlora_linear_fwd_static(const nf4_weight *w, const uint16_t *X, const uint16_t *L1, const uint16_t *L2,
                            float scale, int64_t M, int32_t r, uint16_t *Y, uint16_t *T_out, void *stream) {
    int rc = check_fwd_args(w, X, L1, L2, scale, M, r, Y, T_out);
    if (rc) return rc;
    const Plan p = make_fwd_plan(M, w->rows, w->cols, r);
    if (p.total > kStaticScratchBytes) {
        std::snprintf(g_last_error, sizeof g_last_error,
                      "this shape needs %zu bytes of scratch; the static scratch holds %zu bytes "
                      "(use qlora_linear_fwd with a workspace)", p.total, kStaticScratchBytes);
        return NF4_ERR_WORKSPACE;
    }
    void *ws = nullptr;
    rc = static_scratch(&ws);
    if (rc) return rc;
    return linear_fwd_run(w, X, L1, L2, scale, M, r, Y, T_out, p, ws, reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------------------------------------
// Up to three linears sharing their input (the q, k and v projections of an attention block),
// forward as one product over their weights concatenated along N
// ---------------------------------------------------------------------------------------------
namespace {
constexpr int kMultiMax = 3;
constexpr int64_t kGemmTileN = 256;

struct MultiPlan {
    bool fused;
    Plan lin;                    // the linear layer's plan for [sum N, K] (fused) or the largest N
    size_t off_sT[kMultiMax];    // s T of each adapter (fused)
    size_t total;
};

bool multi_fusable(int32_t n, const int64_t *N, int64_t K, int64_t M) {
    if (n < 2 || M < kExpandMinM) return false;
    int64_t tot = 0;
    for (int i = 0; i < n; ++i) {
        if (i + 1 < n && N[i] % kGemmTileN) return false;   // no product tile spans two weights
        tot += N[i];
    }
    return use_expand(M, tot, K);
}

MultiPlan make_multi_plan(int32_t n, const int64_t *N, int64_t K, int64_t M, int32_t r) {
    MultiPlan p{};
    p.fused = multi_fusable(n, N, K, M);
    int64_t tot = 0, nmax = 0;
    for (int i = 0; i < n; ++i) {
        tot += N[i];
        nmax = N[i] > nmax ? N[i] : nmax;
    }
    size_t total = 0;
    for (int i = 0; i < n; ++i) {   // the separate calls run on the front of the workspace
        const size_t t = make_plan(M, N[i], K, r).total;
        total = t > total ? t : total;
    }
    if (p.fused) {
        p.lin = make_plan(M, tot, K, r);
        size_t off = p.lin.total;
        p.off_sT[0] = p.lin.off_sT;
        for (int i = 1; i < n; ++i) {
            p.off_sT[i] = off;
            off += round256((size_t)M * r * 2);
        }
        total = off > total ? off : total;
    } else {
        p.lin = make_plan(M, nmax, K, r);
    }
    p.total = total;
    return p;
}
}  // namespace

size_t qlora_multi_workspace_size(int32_t n, const int64_t *N, int64_t K, int64_t M, int32_t r) {
    if (n < 1 || n > kMultiMax || !N || K <= 0 || M <= 0 || r <= 0) return 0;
    for (int i = 0; i < n; ++i)
        if (N[i] <= 0) return 0;
    return make_multi_plan(n, N, K, M, r).total;
}

int qlora_multi_fwd(int32_t n, const nf4_weight *const *w, const uint16_t *X, const uint16_t *const *L1,
                    const uint16_t *const *L2, float scale, int64_t M, int32_t r, uint16_t *const *Y,
                    uint16_t *const *T_out, void *workspace, size_t workspace_bytes, void *stream) {
    if (n < 1 || n > kMultiMax) return fail(NF4_ERR_ARG, "n must be 1, 2 or 3");
    if (!w || !L1 || !L2 || !Y) return fail(NF4_ERR_NULL, "w, L1, L2 and Y must be non-NULL arrays");
    int64_t N[kMultiMax];
    for (int i = 0; i < n; ++i) {
        int rc = check_fwd_args(w[i], X, L1[i], L2[i], scale, M, r, Y[i], T_out ? T_out[i] : nullptr);
        if (rc) return rc;
        if (w[i]->cols != w[0]->cols) return fail(NF4_ERR_SHAPE, "the weights must have the same cols (K)");
        N[i] = w[i]->rows;
    }
    const int64_t K = w[0]->cols;
    const MultiPlan p = make_multi_plan(n, N, K, M, r);
    if (!workspace || workspace_bytes < p.total) return fail(NF4_ERR_WORKSPACE, "multi workspace too small");
    if (!aligned16(workspace)) return fail(NF4_ERR_ALIGN, "workspace must be 16-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (!p.fused) {
        for (int i = 0; i < n; ++i) {
            const Plan pi = make_plan(M, N[i], K, r);
            int rc = linear_fwd_run(w[i], X, L1[i], L2[i], scale, M, r, Y[i], T_out ? T_out[i] : nullptr, pi,
                                    workspace, s);
            if (rc) return rc;
        }
        return NF4_OK;
    }
    // each adapter's T partials, then the expansion of its weight into its rows of the combined
    // weight (the same launch sums the partials and transposes its L2 into its rows of L2^T);
    // then one product for all
    uint16_t *Wd = ws_at<uint16_t>(workspace, p.lin.off_Wd);
    uint16_t *L2T = ws_at<uint16_t>(workspace, p.lin.off_L2T);
    nf4k::FwdSegment seg[kMultiMax];
    int64_t row0 = 0;
    for (int i = 0; i < n; ++i) {
        uint16_t *sT = ws_at<uint16_t>(workspace, p.off_sT[i]);
        hipError_t e;
        const nf4k::Reduction red =
            T_partials(X, L1[i], M, K, r, scale, T_out ? T_out[i] : nullptr, sT, p.lin, workspace, s, &e);
        NF4_CHECK_HIP(e, "T = X L1");
        NF4_CHECK_HIP(nf4k::launch_expand_weight(view_of(w[i]), /*transposed=*/false, Wd + row0 * K, &red, s, L2[i],
                                                 L2T + row0 * r, r, N[i]),
                      "weight expansion + T reduce + L2 transpose");
        seg[i] = nf4k::FwdSegment{N[i], sT, L2T + row0 * r, Y[i]};
        row0 += N[i];
    }
    const Plan &pl = p.lin;
    NF4_CHECK_HIP(nf4k::launch_gemm_bf16_fwd_seg(X, Wd, seg, n, r, M, K, split_of(pl.kf, pl, workspace), s),
                  "bf16 GEMM (fwd, concatenated weights)");
    if (pl.kf.ksplit > 1) {
        // each linear's partials: [M, N_i] blocks at M * (its first column), split k of all of them
        // at k M sum(N)
        const float *Pg = ws_at<float>(workspace, pl.off_Pg);
        nf4k::Reduction red[kMultiMax];
        int64_t c0 = 0;
        for (int i = 0; i < n; ++i) {
            red[i] = nf4k::Reduction{Pg + M * c0, pl.kf.ksplit, M * N[i], 1.0f, Y[i], 0.0f, nullptr};
            red[i].stride = M * row0;
            c0 += N[i];
        }
        NF4_CHECK_HIP(nf4k::launch_reduce_partials(red[0], n > 1 ? &red[1] : nullptr, s, n > 2 ? &red[2] : nullptr),
                      "split product reduce");
    }
    return NF4_OK;
}

int qlora_linear_bwd(const nf4_weight *w, const uint16_t *dY, const uint16_t *X, const uint16_t *L1,
                     const uint16_t *L2, const uint16_t *T, float scale, int64_t M, int32_t r,
                     uint16_t *dX, uint16_t *dL1, uint16_t *dL2, uint32_t flags, void *workspace,
                     size_t workspace_bytes, void *stream) {
    int rc = check_linear_args(w, M, r, scale);
    if (rc) return rc;
    if (flags & ~QLORA_DX_ACCUMULATE) return fail(NF4_ERR_ARG, "unknown flags");
    if (!dY || !X || !L1 || !L2 || !dL1 || !dL2)
        return fail(NF4_ERR_NULL, "dY, X, L1, L2, dL1 and dL2 must be non-NULL");
    if (!aligned16(dY) || !aligned16(X) || !aligned16(L1) || !aligned16(L2) || !aligned16(dL1) ||
        !aligned16(dL2) || (T && !aligned16(T)) || (dX && !aligned16(dX)))
        return fail(NF4_ERR_ALIGN, "activations, adapters and gradients must be 16-byte aligned");
    const int64_t N = w->rows, K = w->cols;
    const Plan p = make_plan(M, N, K, r);
    if (!workspace || workspace_bytes < p.total) return fail(NF4_ERR_WORKSPACE, "linear workspace too small");
    if (!aligned16(workspace)) return fail(NF4_ERR_ALIGN, "workspace must be 16-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float *P = ws_at<float>(workspace, p.off_P);
    uint16_t *dT = ws_at<uint16_t>(workspace, p.off_dT);
    const uint16_t *Tuse = T;
    if (!Tuse) {
        uint16_t *Tb = ws_at<uint16_t>(workspace, p.off_T);
        if (nf4k::gemv_fits(M, N, K, r)) {
            // the decode-size forward's partials and summation order: T has the forward's bits
            NF4_CHECK_HIP(nf4k::launch_gemv_T(X, L1, r, M, K, ws_at<float>(workspace, p.off_Tp), Tb, s), "T = X L1");
        } else {
            rc = compute_T(X, L1, M, K, r, 1.0f, Tb, nullptr, p, workspace, s);
            if (rc) return rc;
        }
        Tuse = Tb;
    }
    // dT = s dY L2^T  (L2 [r, N] is already the row-major transpose the product needs)
    NF4_CHECK_HIP(nf4k::launch_skinny_nt(dY, L2, /*b_rows_k=*/false, P, M, r, N, p.ksdT, s), "dT = dY L2^T");
    const nf4k::Reduction red_dT{P, p.ksdT, M * r, scale, dT, 0.0f, nullptr};
    // at large M, one launch expands the weight (transposed) and sums dT's partials
    const bool expand = dX && use_expand(M, N, K);
    uint16_t *WdT = ws_at<uint16_t>(workspace, p.off_Wd);
    if (expand)
        NF4_CHECK_HIP(nf4k::launch_expand_weight(view_of(w), /*transposed=*/true, WdT, &red_dT, s),
                      "weight expansion + dT reduce");
    else
        NF4_CHECK_HIP(nf4k::launch_reduce_partials(red_dT, nullptr, s), "dT reduce");
    // dL2 = s T^T dY and dL1 = X^T dT, independent: one launch for both products, one for both
    // reductions (the partials side by side)
    float *P1 = P + (size_t)p.msL2 * r * N;
    // unsplit (below 1024 tokens): the products write dL2 and dL1 themselves, no reduction launch
    const bool tn_direct = p.msL2 == 1 && p.msL1 == 1;
    nf4k::TnProduct tn_dL2{Tuse, dY, P, r, N, p.msL2};
    nf4k::TnProduct tn_dL1{X, dT, P1, K, r, p.msL1};
    if (tn_direct) {
        tn_dL2.out = dL2; tn_dL2.scale = scale;
        tn_dL1.out = dL1; tn_dL1.scale = 1.0f;
    }
    NF4_CHECK_HIP(nf4k::launch_skinny_tn(tn_dL2, &tn_dL1, M, s), "dL2 = T^T dY, dL1 = X^T dT");
    if (!tn_direct) {
        const nf4k::Reduction red_dL2{P, p.msL2, (int64_t)r * N, scale, dL2, 0.0f, nullptr};
        const nf4k::Reduction red_dL1{P1, p.msL1, K * (int64_t)r, 1.0f, dL1, 0.0f, nullptr};
        NF4_CHECK_HIP(nf4k::launch_reduce_partials(red_dL2, &red_dL1, s), "dL2, dL1 reduce");
    }
    // dX = dY deq(W) + dT L1^T
    const bool acc = (flags & QLORA_DX_ACCUMULATE) != 0;
    if (expand) {
        NF4_CHECK_HIP(nf4k::launch_gemm_bf16_bwd(dY, WdT, dT, L1, r, M, N, K, dX, acc, split_of(p.kb, p, workspace), s),
                      "bf16 GEMM (bwd)");
    } else if (dX) {
        NF4_CHECK_HIP(nf4k::launch_dqgemm_bwd(view_of(w), dY, dT, L1, r, M, dX, acc, split_of(p.kb, p, workspace), s),
                      "fused dequant GEMM (bwd)");
    }
    if (dX) return reduce_split(p.kb, p, workspace, M * K, dX, acc, s);
    return NF4_OK;
}

int qlora_swiglu_fwd(const uint16_t *g, const uint16_t *u, uint16_t *h, int64_t n, void *stream) {
    if (n < 0) return fail(NF4_ERR_SHAPE, "n must be >= 0");
    if (n == 0) return NF4_OK;
    if (!g || !u || !h) return fail(NF4_ERR_NULL, "g, u and h must be non-NULL");
    if (!aligned16(g) || !aligned16(u) || !aligned16(h)) return fail(NF4_ERR_ALIGN, "swiglu buffers must be 16-byte aligned");
    NF4_CHECK_HIP(nf4k::launch_swiglu_fwd(g, u, h, n, reinterpret_cast<hipStream_t>(stream)), "swiglu fwd");
    return NF4_OK;
}

// ---------------------------------------------------------------------------------------------
// Gated MLP forward: gate and up in one product, the glue in its epilogue
// ---------------------------------------------------------------------------------------------
namespace {
// backward: dG and dU after the linear layer's own plan (which the composed path hands to
// qlora_linear_bwd); the fused path also keeps the up weight's transposed expansion, dT and T
struct GatedBwdPlan {
    bool fused;
    Plan lin;
    size_t off_dG, off_dU, off_WdTu, off_dTu, off_Tu, total;
};
GatedBwdPlan make_gated_bwd_plan(int64_t M, int64_t F, int64_t K, int32_t r) {
    GatedBwdPlan g;
    g.fused = use_expand(M, F, K);
    g.lin = make_plan(M, F, K, r);
    size_t off = g.lin.total;
    g.off_dG = off;   off += round256((size_t)M * F * 2);
    g.off_dU = off;   off += round256((size_t)M * F * 2);
    g.off_WdTu = g.off_dTu = g.off_Tu = off;
    if (g.fused) {
        g.off_WdTu = off;  off += round256((size_t)F * K * 2);
        g.off_dTu = off;   off += round256((size_t)M * r * 2);
        g.off_Tu = off;    off += round256((size_t)M * r * 2);
    }
    g.total = off;
    return g;
}
}  // namespace

size_t qlora_gated_workspace_size(int64_t M, int64_t F, int64_t K, int32_t r) {
    if (M <= 0 || F <= 0 || K <= 0 || r <= 0) return 0;
    const int64_t N2[2] = {F, F};
    const size_t f = make_multi_plan(2, N2, K, M, r).total, b = make_gated_bwd_plan(M, F, K, r).total;
    return f > b ? f : b;
}

int qlora_gated_fwd(const nf4_weight *w_gate, const nf4_weight *w_up, const uint16_t *X, const uint16_t *L1_gate,
                    const uint16_t *L2_gate, const uint16_t *L1_up, const uint16_t *L2_up, float scale, int64_t M,
                    int32_t r, uint16_t *G, uint16_t *U, uint16_t *H, uint16_t *T_gate_out, uint16_t *T_up_out,
                    uint32_t flags, void *workspace, size_t workspace_bytes, void *stream) {
    if (flags & ~QLORA_GATED_FUSE) return fail(NF4_ERR_ARG, "unknown flags");
    int rc = check_linear_args(w_gate, M, r, scale);
    if (rc) return rc;
    rc = check_linear_args(w_up, M, r, scale);
    if (rc) return rc;
    if (w_gate->rows != w_up->rows || w_gate->cols != w_up->cols)
        return fail(NF4_ERR_SHAPE, "gate and up weights must have the same shape");
    if (!X || !L1_gate || !L2_gate || !L1_up || !L2_up || !G || !U || !H)
        return fail(NF4_ERR_NULL, "X, the adapters, G, U and H must be non-NULL");
    if (!aligned16(X) || !aligned16(L1_gate) || !aligned16(L2_gate) || !aligned16(L1_up) || !aligned16(L2_up) ||
        !aligned16(G) || !aligned16(U) || !aligned16(H) || (T_gate_out && !aligned16(T_gate_out)) ||
        (T_up_out && !aligned16(T_up_out)))
        return fail(NF4_ERR_ALIGN, "activations and adapters must be 16-byte aligned");
    const int64_t F = w_gate->rows, K = w_gate->cols;
    const int64_t N2[2] = {F, F};
    const MultiPlan p = make_multi_plan(2, N2, K, M, r);
    if (!workspace || workspace_bytes < p.total) return fail(NF4_ERR_WORKSPACE, "gated workspace too small");
    if (!aligned16(workspace)) return fail(NF4_ERR_ALIGN, "workspace must be 16-byte aligned");
    // gate and up as the linears sharing X (one product over both weights from 1024 tokens), then
    // the glue
    const nf4_weight *w2[2] = {w_gate, w_up};
    const uint16_t *l1[2] = {L1_gate, L1_up}, *l2[2] = {L2_gate, L2_up};
    uint16_t *y[2] = {G, U}, *t[2] = {T_gate_out, T_up_out};
    rc = qlora_multi_fwd(2, w2, X, l1, l2, scale, M, r, y, t, workspace, workspace_bytes, stream);
    if (rc) return rc;
    return qlora_swiglu_fwd(G, U, H, M * F, stream);
}

int qlora_gated_bwd(const nf4_weight *w_gate, const nf4_weight *w_up, const uint16_t *dH, const uint16_t *X,
                    const uint16_t *G, const uint16_t *U, const uint16_t *L1_gate, const uint16_t *L2_gate,
                    const uint16_t *L1_up, const uint16_t *L2_up, const uint16_t *T_gate, const uint16_t *T_up,
                    float scale, int64_t M, int32_t r, uint16_t *dX, uint16_t *dL1_gate, uint16_t *dL2_gate,
                    uint16_t *dL1_up, uint16_t *dL2_up, uint32_t flags, void *workspace, size_t workspace_bytes,
                    void *stream) {
    if (flags & ~(QLORA_GATED_FUSE | QLORA_DX_ACCUMULATE)) return fail(NF4_ERR_ARG, "unknown flags");
    int rc = check_linear_args(w_gate, M, r, scale);
    if (rc) return rc;
    rc = check_linear_args(w_up, M, r, scale);
    if (rc) return rc;
    if (w_gate->rows != w_up->rows || w_gate->cols != w_up->cols)
        return fail(NF4_ERR_SHAPE, "gate and up weights must have the same shape");
    if (!dH || !X || !G || !U || !L1_gate || !L2_gate || !L1_up || !L2_up || !dL1_gate || !dL2_gate || !dL1_up ||
        !dL2_up)
        return fail(NF4_ERR_NULL, "dH, X, G, U, the adapters and their gradients must be non-NULL");
    for (const void *q : {(const void *)dH, (const void *)X, (const void *)G, (const void *)U, (const void *)L1_gate,
                          (const void *)L2_gate, (const void *)L1_up, (const void *)L2_up, (const void *)T_gate,
                          (const void *)T_up, (const void *)dX, (const void *)dL1_gate, (const void *)dL2_gate,
                          (const void *)dL1_up, (const void *)dL2_up})
        if (q && !aligned16(q)) return fail(NF4_ERR_ALIGN, "activations, adapters and gradients must be 16-byte aligned");
    const int64_t F = w_gate->rows, K = w_gate->cols;
    const GatedBwdPlan p = make_gated_bwd_plan(M, F, K, r);
    if (!workspace || workspace_bytes < p.total) return fail(NF4_ERR_WORKSPACE, "gated workspace too small");
    if (!aligned16(workspace)) return fail(NF4_ERR_ALIGN, "workspace must be 16-byte aligned");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    uint16_t *dG = ws_at<uint16_t>(workspace, p.off_dG), *dU = ws_at<uint16_t>(workspace, p.off_dU);
    rc = qlora_swiglu_bwd(dH, G, U, dG, dU, M * F, stream);
    if (rc) return rc;
    const uint32_t acc = flags & QLORA_DX_ACCUMULATE;
    if (!p.fused || !(flags & QLORA_GATED_FUSE) || !dX) {
        // the two linears' backward as their own calls, the second adding into dX
        rc = qlora_linear_bwd(w_gate, dG, X, L1_gate, L2_gate, T_gate, scale, M, r, dX, dL1_gate, dL2_gate, acc,
                              workspace, p.lin.total, stream);
        if (rc) return rc;
        return qlora_linear_bwd(w_up, dU, X, L1_up, L2_up, T_up, scale, M, r, dX, dL1_up, dL2_up,
                                dX ? QLORA_DX_ACCUMULATE : 0u, workspace, p.lin.total, stream);
    }
    // per adapter: dT (summed by the weight's transposed expansion), then dL2 and dL1; then one
    // product for dX over both
    const Plan &lp = p.lin;
    float *P = ws_at<float>(workspace, lp.off_P);
    struct Side {
        const nf4_weight *w;
        const uint16_t *dA, *L1, *L2, *T;
        uint16_t *Tb, *dT, *WdT, *dL1, *dL2;
    } sides[2] = {
        {w_gate, dG, L1_gate, L2_gate, T_gate, ws_at<uint16_t>(workspace, lp.off_T), ws_at<uint16_t>(workspace, lp.off_dT),
         ws_at<uint16_t>(workspace, lp.off_Wd), dL1_gate, dL2_gate},
        {w_up, dU, L1_up, L2_up, T_up, ws_at<uint16_t>(workspace, p.off_Tu), ws_at<uint16_t>(workspace, p.off_dTu),
         ws_at<uint16_t>(workspace, p.off_WdTu), dL1_up, dL2_up},
    };
    for (const Side &sd : sides) {
        const uint16_t *Tuse = sd.T;
        if (!Tuse) {
            rc = compute_T(X, sd.L1, M, K, r, 1.0f, sd.Tb, nullptr, lp, workspace, s);
            if (rc) return rc;
            Tuse = sd.Tb;
        }
        NF4_CHECK_HIP(nf4k::launch_skinny_nt(sd.dA, sd.L2, /*b_rows_k=*/false, P, M, r, F, lp.ksdT, s), "dT = dA L2^T");
        const nf4k::Reduction red_dT{P, lp.ksdT, M * r, scale, sd.dT, 0.0f, nullptr};
        NF4_CHECK_HIP(nf4k::launch_expand_weight(view_of(sd.w), /*transposed=*/true, sd.WdT, &red_dT, s),
                      "weight expansion + dT reduce");
        float *P1 = P + (size_t)lp.msL2 * r * F;
        const bool tn_direct = lp.msL2 == 1 && lp.msL1 == 1;
        nf4k::TnProduct tn_dL2{Tuse, sd.dA, P, r, F, lp.msL2};
        nf4k::TnProduct tn_dL1{X, sd.dT, P1, K, r, lp.msL1};
        if (tn_direct) {
            tn_dL2.out = sd.dL2; tn_dL2.scale = scale;
            tn_dL1.out = sd.dL1; tn_dL1.scale = 1.0f;
        }
        NF4_CHECK_HIP(nf4k::launch_skinny_tn(tn_dL2, &tn_dL1, M, s), "dL2 = T^T dA, dL1 = X^T dT");
        if (!tn_direct) {
            const nf4k::Reduction red_dL2{P, lp.msL2, (int64_t)r * F, scale, sd.dL2, 0.0f, nullptr};
            const nf4k::Reduction red_dL1{P1, lp.msL1, K * (int64_t)r, 1.0f, sd.dL1, 0.0f, nullptr};
            NF4_CHECK_HIP(nf4k::launch_reduce_partials(red_dL2, &red_dL1, s), "dL2, dL1 reduce");
        }
    }
    NF4_CHECK_HIP(nf4k::launch_gemm_bf16_bwd_dual(dG, sides[0].WdT, sides[0].dT, L1_gate, dU, sides[1].WdT, sides[1].dT,
                                                  L1_up, r, M, F, K, dX, acc != 0, s),
                  "two-segment bf16 GEMM (bwd)");
    return NF4_OK;
}

int qlora_swiglu_bwd(const uint16_t *dh, const uint16_t *g, const uint16_t *u, uint16_t *dg,
                     uint16_t *du, int64_t n, void *stream) {
    if (n < 0) return fail(NF4_ERR_SHAPE, "n must be >= 0");
    if (n == 0) return NF4_OK;
    if (!dh || !g || !u || !dg || !du) return fail(NF4_ERR_NULL, "swiglu pointers must be non-NULL");
    if (!aligned16(dh) || !aligned16(g) || !aligned16(u) || !aligned16(dg) || !aligned16(du))
        return fail(NF4_ERR_ALIGN, "swiglu buffers must be 16-byte aligned");
    NF4_CHECK_HIP(nf4k::launch_swiglu_bwd(dh, g, u, dg, du, n, reinterpret_cast<hipStream_t>(stream)),
                  "swiglu bwd");
    return NF4_OK;
}

