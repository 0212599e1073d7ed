/*
 * NF4 / double-quantization oracle: plain, slow, obviously correct host C.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline leg of
 * the benchmark may load this code.  It shares no source with the HIP library.
 *
 * Built with  gcc -O2 -ffp-contract=off -fno-fast-math  so that every float operation below is
 * one IEEE operation in the precision written (x86-64: FLT_EVAL_METHOD == 0, no FTZ/DAZ).
 *
 * Sources (all on the page "QLoRA: Efficient Finetuning of Quantized LLMs" study notes,
 * gitcode.csdn.net/6a0046f754b52172bc72e356):
 *   section 3.1  block-wise k-bit quantization, eq. (1) and eq. (2)
 *   section 3.2  4-bit NormalFloat, eq. (4) and the asymmetric exact-zero construction
 *   section 3.3  double quantization (8-bit float constants, block 256, mean removed)
 *   section 3.5  eq. (5) / eq. (6) double dequantization to BF16
 *   section 5.1.2, Fig. 7 text: one half of the normal holds 8 values, the other 7, plus 0.
 * Where those pages leave a step open, the reading taken is stated next to the code.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------
 * Standard normal quantile by bisection on the CDF Phi(x) = erfc(-x / sqrt 2) / 2.
 * The loop halves [lo, hi] until the midpoint no longer lies strictly inside, so the result
 * is the float64 x at which Phi crosses p, to the resolution of erfc.
 * ------------------------------------------------------------------------------------------ */
static double phi(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

double oracle_norm_ppf(double p) {
    double lo = -40.0, hi = 40.0;
    for (int it = 0; it < 4000; ++it) {
        double mid = 0.5 * (lo + hi);
        if (!(mid > lo && mid < hi)) break;
        if (phi(mid) < p) lo = mid; else hi = mid;
    }
    /* pick whichever end of the final bracket is closer in probability */
    return (fabs(phi(lo) - p) <= fabs(phi(hi) - p)) ? lo : hi;
}

/* ------------------------------------------------------------------------------------------
 * NF4 codebook (section 3.2, eq. 4; Fig. 7 text).
 * Reading: each half of the normal gets an evenly spaced probability grid that starts at 0.5
 * and ends at a shared tail probability delta; the positive half has 2^(k-1)+1 = 9 points and
 * the negative half 2^(k-1) = 8 points, both including 0.5 (the zero).  This gives equal
 * probability mass per code inside each half.  The quantiles are divided by Phi^-1(delta)
 * (normalise to [-1, 1] by the absolute maximum), the negative half is negated, the two halves
 * are merged with a single 0, and every value is rounded once from float64 to float32.
 * Output is ascending: out[0] = -1, out[7] = 0, out[15] = +1.
 * ------------------------------------------------------------------------------------------ */
int oracle_codebook(double delta, float out[16]) {
    if (!(delta > 0.5 && delta < 1.0)) return -1;
    const double zmax = oracle_norm_ppf(delta);
    double v[16];
    int n = 0;
    for (int j = 7; j >= 1; --j) {                 /* negative half: 7 non-zero values */
        double t = (double)j / 7.0;
        double p = 0.5 + (delta - 0.5) * t;
        v[n++] = -(oracle_norm_ppf(p) / zmax);
    }
    v[n++] = 0.0;                                  /* the shared exact zero */
    for (int j = 1; j <= 8; ++j) {                 /* positive half: 8 non-zero values */
        double t = (double)j / 8.0;
        double p = 0.5 + (delta - 0.5) * t;
        v[n++] = oracle_norm_ppf(p) / zmax;
    }
    for (int i = 0; i < 16; ++i) out[i] = (float)v[i];
    /* already ascending by construction; check rather than sort */
    for (int i = 1; i < 16; ++i) if (!(out[i - 1] < out[i])) return -2;
    return 0;
}

/* ------------------------------------------------------------------------------------------
 * bfloat16, round to nearest, ties to even (section 3.5: compute type BF16).
 * Defined by value: the two bf16 neighbours of x are compared by distance in float64 (exact,
 * they share the top 16 bits with x); on a tie the one with an even last bit wins.
 * Finite inputs only.
 * ------------------------------------------------------------------------------------------ */
static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

uint16_t oracle_bf16_rne(float x) {
    uint32_t u = bits_from_f32(x);
    uint32_t lo = u & 0xFFFF0000u;              /* toward zero */
    uint32_t hi = lo + 0x00010000u;             /* next magnitude up (may reach infinity) */
    double dx = (double)x;
    /* past the largest finite bf16 the next value up is 2^128 in magnitude (it encodes as inf) */
    double vhi = ((hi & 0x7F800000u) == 0x7F800000u) ? copysign(ldexp(1.0, 128), dx)
                                                      : (double)f32_from_bits(hi);
    double dlo = fabs(dx - (double)f32_from_bits(lo));
    double dhi = fabs(vhi - dx);
    uint32_t pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = ((lo >> 16) & 1u) ? hi : lo;
    return (uint16_t)(pick >> 16);
}

void oracle_bf16_rne_vec(const float *x, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(x[i]);
}

/* ------------------------------------------------------------------------------------------
 * 8-bit float for the second-level constants (section 3.3: "FP8").
 * Reading: OCP FP8 E4M3 -- 1 sign, 4 exponent (bias 7), 3 mantissa bits, subnormals, no
 * infinities, S.1111.111 is NaN, largest finite magnitude 448.
 * ------------------------------------------------------------------------------------------ */
float oracle_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (float)(s ? -mag : mag);
}

/* Nearest finite E4M3 value to t, ties to the even code, sign kept (so a negative value that
 * rounds to zero gives 0x80).  Inputs beyond +-448 saturate to +-448.  Plain linear search over
 * the 127 non-negative finite codes. */
uint8_t oracle_e4m3_encode(float t) {
    uint8_t sign = (bits_from_f32(t) >> 31) ? 0x80 : 0x00;
    double a = fabs((double)t);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(a - (double)oracle_e4m3_decode((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) { bestd = d; best = c; }
    }
    return (uint8_t)(sign | best);
}

void oracle_e4m3_encode_vec(const float *x, int64_t n, uint8_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}

void oracle_e4m3_decode_vec(const uint8_t *c, int64_t n, float *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}

/* ------------------------------------------------------------------------------------------
 * Level-1 block-wise quantization (section 3.1, section 3.2 step 3).
 * The tensor is flattened row-major and cut into consecutive blocks of `block` elements; the
 * last block may be short and its absmax covers only its valid elements.
 * Per block: a = max |x|; n = fp32(x / a) (one IEEE division, so |n| <= 1);
 * code = argmin_j |n - cb[j]|, ties to the lower index.  A block with a == 0 gets the code of
 * the exact zero for every element.
 * Distances are taken in float64.  Where two distances are close enough for rounding to
 * matter, n sits next to a midpoint of two codewords (magnitude >= 2^-5), so both n and the
 * codewords carry their last bit at or above 2^-29 and the float64 differences are exact.
 * Packing: element 2i goes to bits 0-3 of byte i, element 2i+1 to bits 4-7; an odd tail is
 * padded with the zero code.
 * ------------------------------------------------------------------------------------------ */
static int nearest_code(float nv, const float cb[16]) {
    int best = 0;
    double bestd = fabs((double)nv - (double)cb[0]);
    for (int j = 1; j < 16; ++j) {
        double d = fabs((double)nv - (double)cb[j]);
        if (d < bestd) { bestd = d; best = j; }
    }
    return best;
}

static int zero_code(const float cb[16]) {
    for (int j = 0; j < 16; ++j) if (cb[j] == 0.0f) return j;
    return -1;
}

int oracle_quantize(const float *W, int64_t numel, int32_t block, const float cb[16],
                    uint8_t *packed, float *absmax) {
    if (block <= 0 || numel < 0) return -1;
    const int zc = zero_code(cb);
    if (zc < 0) return -2;
    const int64_t nblocks = (numel + block - 1) / block;
    memset(packed, 0, (size_t)((numel + 1) / 2));
    for (int64_t b = 0; b < nblocks; ++b) {
        const int64_t i0 = b * block;
        const int64_t i1 = (i0 + block < numel) ? i0 + block : numel;
        float a = 0.0f;
        for (int64_t i = i0; i < i1; ++i) { float m = fabsf(W[i]); if (m > a) a = m; }
        absmax[b] = a;
        for (int64_t i = i0; i < i1; ++i) {
            int code = zc;
            if (a != 0.0f) {
                float nv = W[i] / a;
                code = nearest_code(nv, cb);
            }
            packed[i >> 1] |= (uint8_t)(code << ((i & 1) ? 4 : 0));
        }
    }
    if (numel & 1) packed[numel >> 1] |= (uint8_t)(zc << 4);
    return 0;
}

/* ------------------------------------------------------------------------------------------
 * Double quantization (section 3.3).
 * Reading of the mean: one float32 mean per weight tensor.  Its float64 sum is taken in groups
 * of 256 consecutive values, each group summed sequentially in ascending order; the group sums
 * are summed again the same way, level after level, until one value remains.
 * mu = fp32(S / n) (float64 division, then one rounding to float32).
 * Per 256-block j: y = fp32(a - mu); A_j = max |y|; s_j = fp32(A_j / 448);
 * code = E4M3(clamp(fp32(y / s_j), -448, 448)); if s_j == 0 every code is 0x00.
 * Stored: code per first-level block, s_j (the multiplier that undoes the scaling, i.e. the
 * inverse of the constant c in eq. 1) per 256-block, and mu.
 * ------------------------------------------------------------------------------------------ */
double oracle_grouped_sum(const double *v, int64_t n, int32_t group) {
    if (n <= 0) return 0.0;
    double *cur = (double *)malloc((size_t)n * sizeof(double));
    memcpy(cur, v, (size_t)n * sizeof(double));
    int64_t len = n;
    while (len > 1) {
        int64_t ng = (len + group - 1) / group;
        for (int64_t g = 0; g < ng; ++g) {
            double s = 0.0;
            int64_t e = (g + 1) * group < len ? (g + 1) * group : len;
            for (int64_t i = g * group; i < e; ++i) s += cur[i];
            cur[g] = s;                              /* g <= g*group: never overwrites unread data */
        }
        len = ng;
    }
    double r = cur[0];
    free(cur);
    return r;
}

int oracle_double_quant(const float *absmax, int64_t nb, int32_t dq_block,
                        uint8_t *codes, float *scales, float *mean_out) {
    if (nb <= 0 || dq_block <= 0) return -1;
    double *d = (double *)malloc((size_t)nb * sizeof(double));
    for (int64_t i = 0; i < nb; ++i) d[i] = (double)absmax[i];
    const double S = oracle_grouped_sum(d, nb, 256);
    free(d);
    const float mu = (float)(S / (double)nb);
    *mean_out = mu;
    const int64_t ng = (nb + dq_block - 1) / dq_block;
    for (int64_t g = 0; g < ng; ++g) {
        const int64_t i0 = g * dq_block;
        const int64_t i1 = (i0 + dq_block < nb) ? i0 + dq_block : nb;
        float A = 0.0f;
        for (int64_t i = i0; i < i1; ++i) { float y = absmax[i] - mu; float m = fabsf(y); if (m > A) A = m; }
        const float s = A / 448.0f;
        scales[g] = s;
        for (int64_t i = i0; i < i1; ++i) {
            if (s == 0.0f) { codes[i] = 0x00; continue; }
            float y = absmax[i] - mu;
            float t = y / s;
            if (t > 448.0f) t = 448.0f;
            if (t < -448.0f) t = -448.0f;
            codes[i] = oracle_e4m3_encode(t);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------------------------
 * Double dequantization, eq. (6): rebuild each block constant from the 8-bit code, its
 * 256-block multiplier and the mean, then dequantize the 4-bit codes with it, eq. (2).
 * a' = fmaf(dec(code_b), s_{b / dq_block}, mu)   (one rounding; C99 fmaf)
 * w  = bf16_RNE(fp32(cb[idx] * a'))
 * A negative a' (possible only for an all-zero block) turns the zero code into -0.0.
 * ------------------------------------------------------------------------------------------ */
static inline int nibble(const uint8_t *packed, int64_t i) {
    return (packed[i >> 1] >> ((i & 1) ? 4 : 0)) & 0xF;
}

/* ------------------------------------------------------------------------------------------
 * Double quantization with 8-bit integer codes: eq. (1) of section 3.1 applied to the centred
 * constants, in place of section 3.3's 8-bit float.  Same structure as above (mean, 256-blocks,
 * the stored multiplier s undoes the scaling): per block A = max |y|, s = fp32(A / 127),
 * code = rint(fp32(y / s)) (ties to even) clamped to [-127, 127], stored as its two's complement
 * byte; s == 0 gives code 0.  Decode: a' = fmaf((float)code, s, mu).
 * ------------------------------------------------------------------------------------------ */
int oracle_double_quant_int8(const float *absmax, int64_t nb, int32_t dq_block,
                             uint8_t *codes, float *scales, float *mean_out) {
    if (nb <= 0 || dq_block <= 0) return -1;
    double *d = (double *)malloc((size_t)nb * sizeof(double));
    for (int64_t i = 0; i < nb; ++i) d[i] = (double)absmax[i];
    const double S = oracle_grouped_sum(d, nb, 256);
    free(d);
    const float mu = (float)(S / (double)nb);
    *mean_out = mu;
    const int64_t ng = (nb + dq_block - 1) / dq_block;
    for (int64_t g = 0; g < ng; ++g) {
        const int64_t i0 = g * dq_block;
        const int64_t i1 = (i0 + dq_block < nb) ? i0 + dq_block : nb;
        float A = 0.0f;
        for (int64_t i = i0; i < i1; ++i) { float y = absmax[i] - mu; float m = fabsf(y); if (m > A) A = m; }
        const float s = A / 127.0f;
        scales[g] = s;
        for (int64_t i = i0; i < i1; ++i) {
            if (s == 0.0f) { codes[i] = 0x00; continue; }
            float y = absmax[i] - mu;
            float t = rintf(y / s);
            if (t > 127.0f) t = 127.0f;
            if (t < -127.0f) t = -127.0f;
            codes[i] = (uint8_t)(int8_t)t;
        }
    }
    return 0;
}

static float int8_decode(uint8_t c) { return (float)(int8_t)c; }

int oracle_block_scales_int8(const uint8_t *codes, const float *scales, float mu, int64_t nb,
                             int32_t dq_block, float *out) {
    if (dq_block <= 0) return -1;
    for (int64_t b = 0; b < nb; ++b)
        out[b] = fmaf(int8_decode(codes[b]), scales[b / dq_block], mu);
    return 0;
}

int oracle_dequant_int8dq(const uint8_t *packed, const uint8_t *codes, const float *scales, float mu,
                          int64_t numel, int32_t block, int32_t dq_block, const float cb[16],
                          uint16_t *out) {
    if (block <= 0 || dq_block <= 0) return -1;
    for (int64_t i = 0; i < numel; ++i) {
        const int64_t b = i / block;
        const float a = fmaf(int8_decode(codes[b]), scales[b / dq_block], mu);
        out[i] = oracle_bf16_rne(cb[nibble(packed, i)] * a);
    }
    return 0;
}

int oracle_block_scales(const uint8_t *codes, const float *scales, float mu, int64_t nb,
                        int32_t dq_block, float *out) {
    if (dq_block <= 0) return -1;
    for (int64_t b = 0; b < nb; ++b)
        out[b] = fmaf(oracle_e4m3_decode(codes[b]), scales[b / dq_block], mu);
    return 0;
}

int oracle_dequant(const uint8_t *packed, const uint8_t *codes, const float *scales, float mu,
                   int64_t numel, int32_t block, int32_t dq_block, const float cb[16],
                   uint16_t *out) {
    if (block <= 0 || dq_block <= 0) return -1;
    for (int64_t i = 0; i < numel; ++i) {
        const int64_t b = i / block;
        const float a = fmaf(oracle_e4m3_decode(codes[b]), scales[b / dq_block], mu);
        out[i] = oracle_bf16_rne(cb[nibble(packed, i)] * a);
    }
    return 0;
}

/* Single-level form (no double quantization): the block constant is the float32 absmax. */
int oracle_dequant_plain(const uint8_t *packed, const float *absmax, int64_t numel, int32_t block,
                         const float cb[16], uint16_t *out) {
    if (block <= 0) return -1;
    for (int64_t i = 0; i < numel; ++i)
        out[i] = oracle_bf16_rne(cb[nibble(packed, i)] * absmax[i / block]);
    return 0;
}

/* Unpack the 4-bit codes, one per byte (used by tests to inspect codes). */
void oracle_unpack(const uint8_t *packed, int64_t numel, uint8_t *codes) {
    for (int64_t i = 0; i < numel; ++i) codes[i] = (uint8_t)nibble(packed, i);
}
