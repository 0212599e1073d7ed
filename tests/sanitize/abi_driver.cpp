// Calls every entry point of include/nf4.h on its host-side paths only -- the codebook builders,
// the workspace size queries and the argument checks that return before any HIP call -- so that
// a build of the library with host-side -fsanitize=address,undefined sees that code.  Needs no
// GPU.  Prints "ok" when every call returned the expected status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "nf4.h"

#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::printf("FAIL %s:%d %s (%s)\n", __FILE__, __LINE__, #c, nf4_last_error()); \
            return 1;                                                         \
        }                                                                     \
    } while (0)

int main() {
    float cb[16];
    CHECK(nf4_build_codebook(cb, 0.0) == NF4_OK);
    CHECK(cb[0] == -1.0f && cb[7] == 0.0f && cb[15] == 1.0f);
    for (double d : {16.0 / 17.0, 0.99, 0.6, 0.999999}) CHECK(nf4_build_codebook(cb, d) == NF4_OK);
    CHECK(nf4_build_codebook(cb, 1.5) == NF4_ERR_ARG);
    CHECK(nf4_build_codebook(nullptr, 0.0) == NF4_ERR_NULL);
    float i4[16], f4[16];
    CHECK(nf4_build_int4_codebook(i4) == NF4_OK && nf4_build_fp4_codebook(f4) == NF4_OK);
    CHECK(nf4_build_codebook(cb, 0.0) == NF4_OK);
    for (int s = -8; s <= 1; ++s) CHECK(std::strlen(nf4_status_string(s)) > 0);
    CHECK(std::strlen(nf4_version()) > 0);

    // fake device pointers: the checks never dereference them
    alignas(16) static uint8_t arena[4096];
    void *a16 = arena + 16, *a8 = arena + 8;
    const float *W = (const float *)a16;
    uint8_t *packed = (uint8_t *)a16;
    float *absmax = (float *)a16;

    // quantize: empty is a no-op; every table (equal neighbours too) passes the codebook check and
    // threshold construction before the NULL and alignment checks
    for (const float *t : {(const float *)cb, (const float *)i4, (const float *)f4}) {
        CHECK(nf4_quantize(W, 0, 64, t, packed, absmax, nullptr) == NF4_OK);
        CHECK(nf4_quantize(nullptr, 64, 64, t, packed, absmax, nullptr) == NF4_ERR_NULL);
        CHECK(nf4_quantize((const float *)a8, 64, 64, t, packed, absmax, nullptr) == NF4_ERR_ALIGN);
    }
    CHECK(nf4_quantize(W, 64, 32, cb, packed, absmax, nullptr) == NF4_ERR_UNSUPPORTED);
    CHECK(nf4_quantize(W, -1, 64, cb, packed, absmax, nullptr) == NF4_ERR_SHAPE);
    float bad[16];
    std::memcpy(bad, cb, sizeof bad);
    bad[3] = bad[9];
    CHECK(nf4_quantize(W, 64, 64, bad, packed, absmax, nullptr) == NF4_ERR_ARG);
    bad[3] = NAN;
    CHECK(nf4_quantize(W, 64, 64, bad, packed, absmax, nullptr) == NF4_ERR_ARG);
    CHECK(nf4_dequant_single(packed, absmax, 64, 64, bad, (uint16_t *)a16, nullptr) == NF4_ERR_ARG);

    // double quant
    for (int64_t nb : {(int64_t)1, (int64_t)255, (int64_t)257, (int64_t)65537, (int64_t)3670016})
        CHECK(nf4_double_quant_workspace_size(nb, 256) > 0);
    const size_t wsq = nf4_double_quant_workspace_size(1000, 256);
    CHECK(nf4_double_quant(absmax, 0, 256, packed, absmax, absmax, a16, wsq, nullptr) == NF4_ERR_SHAPE);
    CHECK(nf4_double_quant(absmax, 1000, 128, packed, absmax, absmax, a16, wsq, nullptr) == NF4_ERR_UNSUPPORTED);
    CHECK(nf4_double_quant(absmax, 1000, 256, packed, absmax, absmax, nullptr, wsq, nullptr) == NF4_ERR_NULL);
    CHECK(nf4_double_quant(absmax, 1000, 256, packed, absmax, absmax, a16, wsq - 1, nullptr) == NF4_ERR_WORKSPACE);
    CHECK(nf4_double_quant_int8(absmax, 1000, 256, (uint8_t *)a8, absmax, absmax, a16, wsq, nullptr) ==
          NF4_ERR_ALIGN);

    // the weight descriptor
    nf4_weight w{};
    w.packed = packed; w.absmax_q = packed; w.absmax_scale = absmax; w.absmax_mean = absmax;
    w.rows = 4096; w.cols = 4096; w.block = 64; w.dq_block = 256; w.dq_format = NF4_DQ_E4M3;
    std::memcpy(w.codebook, cb, sizeof cb);
    uint16_t *out = (uint16_t *)a16;
    CHECK(nf4_dequant(nullptr, out, nullptr) == NF4_ERR_NULL);
    CHECK(nf4_dequant(&w, nullptr, nullptr) == NF4_ERR_NULL);
    CHECK(nf4_dequant(&w, (uint16_t *)a8, nullptr) == NF4_ERR_ALIGN);
    nf4_weight w2 = w;
    w2.block = 128;
    CHECK(nf4_dequant(&w2, out, nullptr) == NF4_ERR_UNSUPPORTED);
    w2 = w; w2.dq_format = 7;
    CHECK(nf4_dequant(&w2, out, nullptr) == NF4_ERR_ARG);
    w2 = w; w2.rows = 0;
    CHECK(nf4_dequant(&w2, out, nullptr) == NF4_ERR_SHAPE);

    // workspace plans over the routing boundaries and the workload shapes
    const int64_t Ms[] = {1, 2, 4, 8, 9, 16, 17, 300, 1023, 1024, 2048, 4096, 65536};
    const int64_t NKs[][2] = {{256, 256}, {4096, 4096}, {11008, 4096}, {4096, 11008}, {22016, 8192},
                              {8192, 22016}, {28672, 8192}, {3000, 11008}, {64, 26624}, {32768, 32768}};
    for (int64_t M : Ms)
        for (auto &nk : NKs)
            for (int32_t r : {8, 64, 128}) {
                CHECK(qlora_linear_workspace_size(M, nk[0], nk[1], r) > 0);
                CHECK(qlora_gated_workspace_size(M, nk[0], nk[1], r) > 0);
            }
    CHECK(qlora_linear_workspace_size(0, 64, 64, 8) == 0);

    // linear layer argument checks
    const uint16_t *X = (const uint16_t *)a16;
    uint16_t *Y = (uint16_t *)a16;
    const int64_t M = 64;
    const int32_t r = 16;
    const size_t wsl = qlora_linear_workspace_size(M, w.rows, w.cols, r);
    CHECK(qlora_linear_fwd(&w, X, X, X, 0.5f, 0, r, Y, nullptr, a16, wsl, nullptr) == NF4_ERR_SHAPE);
    CHECK(qlora_linear_fwd(&w, X, X, X, 0.5f, M, 12, Y, nullptr, a16, wsl, nullptr) == NF4_ERR_UNSUPPORTED);
    CHECK(qlora_linear_fwd(&w, X, X, X, 0.5f, M, 256, Y, nullptr, a16, wsl, nullptr) == NF4_ERR_UNSUPPORTED);
    CHECK(qlora_linear_fwd(&w, X, X, X, NAN, M, r, Y, nullptr, a16, wsl, nullptr) == NF4_ERR_ARG);
    CHECK(qlora_linear_fwd(&w, nullptr, X, X, 0.5f, M, r, Y, nullptr, a16, wsl, nullptr) == NF4_ERR_NULL);
    CHECK(qlora_linear_fwd(&w, X, X, X, 0.5f, M, r, (uint16_t *)a8, nullptr, a16, wsl, nullptr) == NF4_ERR_ALIGN);
    CHECK(qlora_linear_fwd(&w, X, X, X, 0.5f, M, r, Y, nullptr, a16, wsl - 1, nullptr) == NF4_ERR_WORKSPACE);
    CHECK(qlora_linear_fwd(&w, X, X, X, 0.5f, M, r, Y, nullptr, nullptr, wsl, nullptr) == NF4_ERR_WORKSPACE);
    w2 = w; w2.cols = 4000;
    CHECK(qlora_linear_fwd(&w2, X, X, X, 0.5f, M, r, Y, nullptr, a16, wsl, nullptr) == NF4_ERR_UNSUPPORTED);
    w2 = w; w2.rows = 1 << 20; w2.cols = 1 << 12;
    CHECK(qlora_linear_fwd(&w2, X, X, X, 0.5f, 1 << 20, r, Y, nullptr, a16, wsl, nullptr) == NF4_ERR_UNSUPPORTED);
    CHECK(qlora_linear_bwd(&w, X, X, X, X, nullptr, 0.5f, M, r, Y, Y, Y, 4u, a16, wsl, nullptr) == NF4_ERR_ARG);
    CHECK(qlora_linear_bwd(&w, X, X, X, X, nullptr, 0.5f, M, r, Y, nullptr, Y, 0u, a16, wsl, nullptr) == NF4_ERR_NULL);
    CHECK(qlora_linear_bwd(&w, X, X, X, X, (const uint16_t *)a8, 0.5f, M, r, Y, Y, Y, 0u, a16, wsl, nullptr) ==
          NF4_ERR_ALIGN);
    CHECK(qlora_linear_bwd(&w, X, X, X, X, nullptr, 0.5f, M, r, Y, Y, Y, 0u, a16, 0, nullptr) == NF4_ERR_WORKSPACE);

    // gated MLP and glue
    nf4_weight wu = w;
    wu.rows = 2048;
    const size_t wsg = qlora_gated_workspace_size(M, w.rows, w.cols, r);
    CHECK(qlora_gated_fwd(&w, &wu, X, X, X, X, X, 0.5f, M, r, Y, Y, Y, nullptr, nullptr, 0u, a16, wsg, nullptr) ==
          NF4_ERR_SHAPE);
    CHECK(qlora_gated_fwd(&w, &w, X, X, X, X, X, 0.5f, M, r, Y, Y, Y, nullptr, nullptr, 8u, a16, wsg, nullptr) ==
          NF4_ERR_ARG);
    CHECK(qlora_gated_bwd(&w, &w, X, X, X, X, X, X, X, X, nullptr, nullptr, 0.5f, M, r, Y, Y, Y, Y, nullptr, 0u, a16,
                          wsg, nullptr) == NF4_ERR_NULL);
    CHECK(qlora_swiglu_fwd(X, X, Y, -1, nullptr) == NF4_ERR_SHAPE);
    CHECK(qlora_swiglu_fwd(X, X, Y, 0, nullptr) == NF4_OK);
    CHECK(qlora_swiglu_bwd(X, X, X, Y, (uint16_t *)a8, 10, nullptr) == NF4_ERR_ALIGN);

    // timing hooks: set and clear without a stream
    CHECK(nf4_set_gemm_timing_events(nullptr, nullptr, nullptr, 0) == NF4_OK);
    CHECK(nf4_set_gemm_timing_events(nullptr, nullptr, nullptr, 2) == NF4_ERR_NULL);
    CHECK(nf4_set_gemm_timing_events(nullptr, nullptr, nullptr, -1) == NF4_ERR_ARG);
    CHECK(nf4_gemm_timing_count() == 0);
    std::printf("ok\n");
    return 0;
}
