/*
 * Runs every function of the CPU oracle (oracle/nf4_oracle.c) on ragged sizes and edge values, so
 * that a build with -fsanitize=address,undefined sees each of its loops and index computations.
 * Prints "ok" when every call returned success and the outputs pass basic invariants.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_norm_ppf(double p);
int oracle_codebook(double delta, float out[16]);
uint16_t oracle_bf16_rne(float x);
void oracle_bf16_rne_vec(const float *x, int64_t n, uint16_t *out);
float oracle_e4m3_decode(uint8_t c);
uint8_t oracle_e4m3_encode(float t);
void oracle_e4m3_encode_vec(const float *x, int64_t n, uint8_t *out);
void oracle_e4m3_decode_vec(const uint8_t *c, int64_t n, float *out);
int oracle_quantize(const float *W, int64_t numel, int32_t block, const float cb[16], uint8_t *packed,
                    float *absmax);
double oracle_grouped_sum(const double *v, int64_t n, int32_t group);
int oracle_double_quant(const float *absmax, int64_t nb, int32_t dq_block, uint8_t *codes, float *scales,
                        float *mean_out);
int oracle_double_quant_int8(const float *absmax, int64_t nb, int32_t dq_block, uint8_t *codes,
                             float *scales, float *mean_out);
int oracle_block_scales(const uint8_t *codes, const float *scales, float mu, int64_t nb, int32_t dq_block,
                        float *out);
int oracle_block_scales_int8(const uint8_t *codes, const float *scales, float mu, int64_t nb,
                             int32_t dq_block, float *out);
int oracle_dequant(const uint8_t *packed, const uint8_t *codes, const float *scales, float mu, int64_t numel,
                   int32_t block, int32_t dq_block, const float cb[16], uint16_t *out);
int oracle_dequant_int8dq(const uint8_t *packed, const uint8_t *codes, const float *scales, float mu,
                          int64_t numel, int32_t block, int32_t dq_block, const float cb[16], uint16_t *out);
int oracle_dequant_plain(const uint8_t *packed, const float *absmax, int64_t numel, int32_t block,
                         const float cb[16], uint16_t *out);
void oracle_unpack(const uint8_t *packed, int64_t numel, uint8_t *codes);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) {
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) * 0x1.0p-53;
}

#define CHECK(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); return 1; } } while (0)

static int one_size(int64_t n, const float cb[16]) {
    const int64_t nb = (n + 63) / 64, ng = (nb + 255) / 256;
    float *W = malloc(sizeof(float) * (size_t)(n ? n : 1));
    uint8_t *packed = malloc((size_t)((n + 1) / 2 + 1));
    float *absmax = malloc(sizeof(float) * (size_t)(nb ? nb : 1));
    uint8_t *codes = malloc((size_t)(nb ? nb : 1));
    float *scales = malloc(sizeof(float) * (size_t)(ng ? ng : 1));
    float *ap = malloc(sizeof(float) * (size_t)(nb ? nb : 1));
    uint16_t *deq = malloc(sizeof(uint16_t) * (size_t)(n ? n : 1));
    uint8_t *un = malloc((size_t)(n ? n : 1));
    for (int64_t i = 0; i < n; ++i) {
        double u = urand();
        W[i] = (float)((u - 0.5) * ((i % 97 == 0) ? 2.0 : 0.05));
        if (i % 640 < 64 && i >= 640) W[i] = 0.0f;           /* an all-zero block */
    }
    CHECK(oracle_quantize(W, n, 64, cb, packed, absmax) == 0);
    oracle_unpack(packed, n, un);
    for (int64_t i = 0; i < n; ++i) CHECK(un[i] < 16);
    for (int64_t b = 0; b < nb; ++b) CHECK(absmax[b] >= 0.0f);
    if (nb > 0) {
        float mu;
        CHECK(oracle_double_quant(absmax, nb, 256, codes, scales, &mu) == 0);
        CHECK(oracle_block_scales(codes, scales, mu, nb, 256, ap) == 0);
        CHECK(oracle_dequant(packed, codes, scales, mu, n, 64, 256, cb, deq) == 0);
        CHECK(oracle_double_quant_int8(absmax, nb, 256, codes, scales, &mu) == 0);
        CHECK(oracle_block_scales_int8(codes, scales, mu, nb, 256, ap) == 0);
        CHECK(oracle_dequant_int8dq(packed, codes, scales, mu, n, 64, 256, cb, deq) == 0);
    }
    CHECK(oracle_dequant_plain(packed, absmax, n, 64, cb, deq) == 0);
    for (int64_t i = 0; i < n; ++i) {            /* one level: |deq| <= absmax of the block */
        uint32_t bits = (uint32_t)deq[i] << 16;
        float v;
        memcpy(&v, &bits, 4);
        CHECK(fabsf(v) <= absmax[i / 64] * 1.01f + 1e-30f);
    }
    free(W); free(packed); free(absmax); free(codes); free(scales); free(ap); free(deq); free(un);
    return 0;
}

int main(void) {
    float cb[16];
    CHECK(oracle_codebook(1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0), cb) == 0);
    CHECK(cb[0] == -1.0f && cb[7] == 0.0f && cb[15] == 1.0f);
    CHECK(oracle_codebook(0.3, cb) != 0);
    CHECK(oracle_codebook(16.0 / 17.0, cb) == 0);
    CHECK(fabs(oracle_norm_ppf(0.975) - 1.959963984540054) < 1e-12);
    for (int c = 0; c < 256; ++c) {
        if ((c & 0x7F) == 0x7F) continue;
        CHECK(oracle_e4m3_encode(oracle_e4m3_decode((uint8_t)c)) == (uint8_t)c);
    }
    float xs[5] = {0.0f, -0.0f, 1e-40f, 3.3e38f, -448.5f};
    uint16_t hb[5];
    uint8_t eb[5];
    oracle_bf16_rne_vec(xs, 5, hb);
    oracle_e4m3_encode_vec(xs + 4, 1, eb);
    CHECK(eb[0] == 0xFE);
    float dv[1];
    oracle_e4m3_decode_vec(eb, 1, dv);
    CHECK(dv[0] == -448.0f);
    double g[1000];
    for (int i = 0; i < 1000; ++i) g[i] = urand();
    CHECK(oracle_grouped_sum(g, 1000, 256) > 0.0);
    CHECK(oracle_grouped_sum(g, 0, 256) == 0.0);
    const int64_t sizes[] = {0, 1, 2, 63, 64, 65, 127, 1000, 64 * 256, 64 * 256 + 1, 64 * 257 + 37, 70001};
    for (size_t k = 0; k < sizeof sizes / sizeof sizes[0]; ++k)
        if (one_size(sizes[k], cb)) return 1;
    CHECK(oracle_quantize(NULL, -1, 64, cb, NULL, NULL) != 0);
    CHECK(oracle_double_quant(NULL, 0, 256, NULL, NULL, NULL) != 0);
    printf("ok\n");
    return 0;
}
