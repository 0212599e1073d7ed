// Small-batch forward (9 to 16 tokens, and smaller token counts on shapes the row kernel of
// the decode GEMV does not take) of the QLoRA linear layer (gfx950):
//   Y = X deq(W)^T + s T L2,   T = X L1 computed beforehand (s T passed in, bf16 [M, r])
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (5) / eq. (6); section 4 eq. (3).
//
// This shape streams the 4-bit weight once from HBM; the cost to hide is the dequantization,
// not the arithmetic.  With up to 16 tokens the 16 rows of v_mfma_f32_16x16x32_bf16 are mostly
// used, so the products go there (rows past M are zero), and the VALU only turns codes into bf16
// -- exactly the dequantized weights of eq. (6), so this path matches the large-batch GEMM:
//   - a wave owns 16 W rows; per 256-column "macro step" lane (n = l % 16, g = l / 16) owns one
//     whole quantization block (row n, block 4 step + g): 32 packed bytes, one 16-entry bf16
//     table (v_perm byte planes), 8 dwords -> 8 MFMAs (one B fragment each)
//   - codes are expanded in planar order (elements 0,2,4,6 | 1,3,5,7 of each 8), so the X
//     fragments are stored in LDS in the same order (permuted once per window)
//   - W is fetched four macro steps ahead; X is staged through LDS in windows of 1024 columns,
//     double buffered (the next window travels through registers while the current one is
//     consumed), shared by the 4 waves of a block
// Epilogue: 2 more MFMAs add s T L2 (A = s T, B = a strided gather of L2), then bf16 stores.

#include "common.h"
#include "dqtile.h"
#include "launch.h"

namespace nf4k {

namespace {

constexpr int NWAVE = 4;
constexpr int ROWS_PER_WG = 16 * NWAVE;        // 64 W rows
constexpr int XWIN = 1024;                     // X window (columns)
constexpr int XROW = XWIN + 8;                 // padded LDS row (elements): rows start 4 banks apart
constexpr int MACRO = 256;                     // columns per macro step (4 blocks)

__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// natural 8 bf16 (4 dwords: pairs (0,1),(2,3),(4,5),(6,7)) -> planar order
__device__ __forceinline__ u32x4 to_planar(u32x4 v) {
    u32x4 o;
    o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);   // elements 0, 2
    o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);   // 4, 6
    o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);   // 1, 3
    o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);   // 5, 7
    return o;
}

struct GemvArgs {
    const uint16_t *X;       // [M, K]
    const uint8_t *packed;   // [N, K/2]
    const uint8_t *c2;
    const float *c1;
    const float *mean;
    uint32_t dq_int8;        // second-level codes are int8 (else E4M3)
    const uint16_t *sT;      // [M, r]  (s * X L1)
    const uint16_t *L2;      // [r, N]
    uint16_t *Y;             // [M, N]
    int64_t M, N, K;
    int32_t r;
    Codebook cb;
};

// I8: the second-level codes are int8 (else E4M3), fixed at compile time so that the E4M3
// kernel carries no per-block select.
template <int MROWS, bool I8>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs g) {
    // X window: [MROWS rows][XWIN cols], planar within each 8-column group, double buffered.
    // Lanes whose token row is >= MROWS feed zeros to the MFMA without touching LDS.
    __shared__ __align__(16) uint8_t Xs0[MROWS * XROW * 2];
    __shared__ __align__(16) uint8_t Xs1[MROWS * XROW * 2];
    constexpr int XCH = MROWS * (XWIN / 8) / 256;        // 16-byte X chunks per thread per window
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * ROWS_PER_WG + wave * 16;
    const int64_t n = n0 + ln;                      // this lane's W row
    const int64_t wrow_bytes = g.K >> 1, nblk = g.K >> 6;
    const float mean = g.mean[0];
    constexpr bool dq_i8 = I8;

    const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.packed + n0 * wrow_bytes, (g.N - n0) * wrow_bytes);
    const __amdgpu_buffer_rsrc_t rC2 = make_rsrc(g.c2, g.N * nblk);
    const __amdgpu_buffer_rsrc_t rC1 = make_rsrc(g.c1, ((g.N * nblk + 255) >> 8) * 4);
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(g.X, g.M * g.K * 2);

    const int nmacro = (int)((g.K + MACRO - 1) / MACRO);

    // ---- X windows: global -> registers early, registers -> LDS later ----
    u32x4 xr[XCH];
    auto fetch_x = [&](int win) {
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = tid + 256 * q;                 // chunk id: row = c / 128, col8 = c % 128
            const int row = c >> 7, col8 = c & 127;
            const int64_t k = (int64_t)win * XWIN + col8 * 8;
            const bool ok = row < g.M && k < g.K;
            xr[q] = bload16(rX, ok ? (uint32_t)((row * g.K + k) * 2) : 0xFFFFFFF0u);
        }
    };
    auto store_x = [&](uint8_t *dst) {
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = tid + 256 * q;
            const int row = c >> 7, col8 = c & 127;
            *reinterpret_cast<u32x4 *>(dst + (row * XROW + col8 * 8) * 2) = to_planar(xr[q]);
        }
    };

    struct WStage {
        u32x4 w[2];
        uint32_t c2, c1;
    };
    auto load_w = [&](int ms, WStage &st) {
        const int64_t blk = (int64_t)ms * 4 + lg;
        const bool live = ms < nmacro && blk < nblk;
        const uint32_t off = (uint32_t)(ln * wrow_bytes + blk * 32);
        st.w[0] = bload16(rW, live ? off : 0xFFFFFFF0u);
        st.w[1] = bload16(rW, live ? off + 16 : 0xFFFFFFF0u);
        const uint32_t b = (uint32_t)(n * nblk + blk);
        const bool okr = live && n < g.N;
        st.c2 = bload1(rC2, okr ? b : 0xFFFFFFF0u);
        st.c1 = bload4(rC1, okr ? (b >> 8) * 4 : 0xFFFFFFF0u);
    };

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto macro_step = [&](int ms, const WStage &st, const uint8_t *Xw) {
        const int kin = (ms * MACRO) % XWIN;             // column offset inside the window
        const int64_t blk = (int64_t)ms * 4 + lg;
        float a = block_scale(st.c2, __uint_as_float(st.c1), mean, dq_i8);
        if (ms >= nmacro || blk >= nblk) a = 0.0f;        // past K: contributes nothing
        const Lut t = make_lut(g.cb, a);
        const uint32_t wd[8] = {st.w[0].x, st.w[0].y, st.w[0].z, st.w[0].w,
                                st.w[1].x, st.w[1].y, st.w[1].z, st.w[1].w};
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const u32x4 b = dequant8_planar(t, wd[d]);
            // A: X row ln, columns kin + 64 lg + 8 d .. +7 (planar, same order as b)
            u32x4 av = {0u, 0u, 0u, 0u};
            if (ln < MROWS)
                av = *reinterpret_cast<const u32x4 *>(Xw + (ln * XROW + kin + lg * 64 + d * 8) * 2);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                          __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
        }
    };

    // Four macro steps per X window (XWIN / MACRO); W is fetched four macro steps ahead.
    // Window w+1 is fetched at the first macro step of window w, written to the other LDS buffer
    // at its third, and made visible by the barrier that closes window w.
    WStage S0, S1, S2, S3;
    fetch_x(0);
    store_x(Xs0);
    load_w(0, S0);
    load_w(1, S1);
    load_w(2, S2);
    load_w(3, S3);
    __syncthreads();
    for (int ms = 0; ms < nmacro; ms += 4) {
        const int win = ms / 4;
        uint8_t *Xcur = (win & 1) ? Xs1 : Xs0;
        uint8_t *Xnxt = (win & 1) ? Xs0 : Xs1;
        fetch_x(win + 1);                                // past the end: reads zeros
        macro_step(ms, S0, Xcur);
        load_w(ms + 4, S0);
        macro_step(ms + 1, S1, Xcur);
        load_w(ms + 5, S1);
        store_x(Xnxt);
        macro_step(ms + 2, S2, Xcur);
        load_w(ms + 6, S2);
        macro_step(ms + 3, S3, Xcur);
        load_w(ms + 7, S3);
        __syncthreads();
    }

    // ---- LoRA: acc += (s T) L2 over r in steps of 32 (two MFMAs for r = 64) ----
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(g.sT, g.M * (int64_t)g.r * 2);
    const __amdgpu_buffer_rsrc_t rL2 = make_rsrc(g.L2, (int64_t)g.r * g.N * 2);
    for (int j0 = 0; j0 < g.r; j0 += 32) {
        // A: sT row ln, j = j0 + 8 lg .. +7 (natural order); B: L2[j][n] for the same j
        const int jj = j0 + lg * 8;
        const bool oka = ln < g.M && jj < g.r;
        const u32x4 av = bload16(rT, oka ? (uint32_t)((ln * (int64_t)g.r + jj) * 2) : 0xFFFFFFF0u);
        uint32_t bw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ja = jj + 2 * i, jb = ja + 1;
            const uint32_t lo = bload2(rL2, (ja < g.r && n < g.N) ? (uint32_t)(((int64_t)ja * g.N + n) * 2) : 0xFFFFFFF0u);
            const uint32_t hi = bload2(rL2, (jb < g.r && n < g.N) ? (uint32_t)(((int64_t)jb * g.N + n) * 2) : 0xFFFFFFF0u);
            bw[i] = (lo & 0xFFFFu) | (hi << 16);
        }
        const u32x4 bv = {bw[0], bw[1], bw[2], bw[3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
    }

    // ---- store: lane holds rows 4 lg + i (tokens), column n ----
    if (n < g.N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = lg * 4 + i;
            if (m < g.M) g.Y[m * g.N + n] = (uint16_t)f32_to_bf16(acc[i]);
        }
    }
}

}  // namespace

hipError_t launch_gemv_wide_fwd(const WeightView &w, const uint16_t *X, const uint16_t *sT,
                                const uint16_t *L2, int32_t r, int64_t M, uint16_t *Y, hipStream_t stream) {
    GemvArgs a;
    a.X = X;
    a.packed = w.packed; a.c2 = w.c2; a.c1 = w.c1; a.mean = w.mean; a.dq_int8 = w.dq_int8;
    a.sT = sT; a.L2 = L2; a.Y = Y;
    a.M = M; a.N = w.rows; a.K = w.cols; a.r = r;
    for (int j = 0; j < 16; ++j) a.cb.v[j] = w.cb[j];
    const int grid = (int)((w.rows + ROWS_PER_WG - 1) / ROWS_PER_WG);
    timing_before(stream, 2);
    if (a.dq_int8)
        hipLaunchKernelGGL((gemv_kernel<16, true>), dim3(grid), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((gemv_kernel<16, false>), dim3(grid), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace nf4k
