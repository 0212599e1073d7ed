// Small-batch forward (9 to 64 tokens, and smaller token counts on shapes the row kernel of
// the decode GEMV does not take) of the QLoRA linear layer (gfx950):
//   Y = X deq(W)^T + s T L2,   T = X L1 computed beforehand (its float32 split partials, or
//   s T already reduced)
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (5) / eq. (6); section 4 eq. (3).
//
// This shape streams the 4-bit weight once from HBM; the cost to hide is the dequantization,
// not the arithmetic.  With up to 16 tokens the 16 rows of v_mfma_f32_16x16x32_bf16 are mostly
// used, so the products go there (rows past M are zero), and the VALU only turns codes into bf16
// -- exactly the dequantized weights of eq. (6), so this path matches the large-batch GEMM.
// 17 to 32 tokens take two groups of 16 and 33 to 64 four (with X windows of 512 columns, so
// that the two buffers fit in LDS): each decoded B fragment feeds one MFMA per group, so the
// decode, which bounds the kernel, is done once for all of them:
//   - a wave owns 16 W rows; per 256-column "macro step" lane (n = l % 16, g = l / 16) owns one
//     whole quantization block (row n, block 4 step + g): 32 packed bytes, one 16-entry bf16
//     table (v_perm byte planes), 8 dwords -> 8 MFMAs (one B fragment each)
//   - codes are expanded in planar order (elements 0,2,4,6 | 1,3,5,7 of each 8), so the X
//     fragments are stored in LDS in the same order (permuted once per window)
//   - W is fetched four macro steps ahead; X is staged through LDS in windows of 1024 columns
//     (512 for 64 tokens), double buffered (the next window travels through registers while the
//     current one is consumed), shared by the waves of a block
//   - a block has NW = ceil(N / 16 / 256) waves (4 to 8), so that the grid is about one block
//     per CU (28672 rows: 256 blocks of 7 waves, where 4-wave blocks made 448, two on most CUs);
//     where the rows give fewer blocks than CUs (4096 rows: 64) and each block has enough work,
//     the reduction is split over S = 256 / blocks workgroups of whole groups of 4 macro steps,
//     which write float32 partials that a fixed-order pass sums (the LoRA term rides in the last
//     split)
//   - the kernel is bound by the VALU work of the exact decode (about 250 VALU instructions per
//     wave per 4096 weights), not by HBM
// Prologue: s T into LDS.  Where T's float32 split partials are few (at most 128 KB), each
// workgroup that needs s T sums them itself in ascending split order (the order of the standalone
// reduction, so T has the same bits on every path), and workgroup 0 also writes T for the
// backward: this saves the reduction's own launch.  Otherwise s T comes reduced (bf16) and is
// copied in.
// Epilogue: 2 more MFMAs add s T L2 (A = s T, B = a strided gather of L2), then bf16 stores.

#include "common.h"
#include "dqtile.h"
#include "launch.h"

namespace nf4k {

namespace {

constexpr int NWAVE_MAX = 8;
constexpr int R_MAX = 128;                     // LoRA rank
constexpr int MACRO = 256;                     // columns per macro step (4 blocks)
// X window (columns) staged per buffer: 1024 for up to 32 token rows, 512 for 64 (so that the two
// buffers stay within LDS); padded LDS rows (+8 elements) start 4 banks apart
template <int MROWS> constexpr int xwin() { return MROWS >= 64 ? 512 : 1024; }

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
    const float *Tp;         // T's float32 partials [ksT][M, r], or null: sT given
    const uint16_t *sT;      // [M, r] s T (bf16), when Tp is null
    int32_t ksT;
    float tscale;            // s
    uint16_t *T_out;         // [M, r] T (optional)
    const uint16_t *L2;      // [r, N]
    uint16_t *Y;             // [M, N]
    float *P;                // [ksplit, M, N] partials (ksplit > 1)
    int64_t M, N, K;
    int32_t r;
    int32_t ksplit, kper;    // reduction split: macro steps per split (a multiple of 4)
    Codebook cb;
};

// I8: the second-level codes are int8 (else E4M3), fixed at compile time so that the E4M3
// kernel carries no per-block select.
template <int MROWS, bool I8, int NW>
__global__ __launch_bounds__(NW * 64) void gemv_kernel(GemvArgs g) {
    constexpr int XWIN = xwin<MROWS>();
    constexpr int XROW = XWIN + 8;
    constexpr int WPW = XWIN / MACRO;                     // macro steps per window: 4 or 2
    constexpr int C8 = XWIN / 8;                          // 16-byte chunks per window row
    // X window: [MROWS rows][XWIN cols], planar within each 8-column group, double buffered;
    // rows at or past the token count hold zeros.
    __shared__ __align__(16) uint8_t Xs0[MROWS * XROW * 2];
    __shared__ __align__(16) uint8_t Xs1[MROWS * XROW * 2];
    __shared__ __align__(16) uint16_t sTs[MROWS * R_MAX];  // s T, bf16 [M][r]
    constexpr int NT = NW * 64;
    constexpr int XCHUNKS = MROWS * C8;                   // 16-byte X chunks per window
    constexpr int XCH = (XCHUNKS + NT - 1) / NT;         // per thread (the last round part-filled)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ln = lane & 15, lg = lane >> 4;
    const int nrb = (int)(gridDim.x / g.ksplit);             // row blocks
    const int split = (int)blockIdx.x / nrb;
    const int64_t n0 = (int64_t)((int)blockIdx.x - split * nrb) * (16 * NW) + wave * 16;
    const int64_t n = n0 + ln;                      // this lane's W row
    const int64_t wrow_bytes = g.K >> 1, nblk = g.K >> 6;
    const float mean = g.mean[0];
    constexpr bool dq_i8 = I8;

    const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.packed + n0 * wrow_bytes, (g.N - n0) * wrow_bytes);
    const __amdgpu_buffer_rsrc_t rC2 = make_rsrc(g.c2, g.N * nblk);
    const __amdgpu_buffer_rsrc_t rC1 = make_rsrc(g.c1, ((g.N * nblk + 255) >> 8) * 4);
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(g.X, g.M * g.K * 2);
    constexpr int G = MROWS / 16;                     // 16-token groups

    const int nmacro = (int)((g.K + MACRO - 1) / MACRO);
    const int ms_begin = split * g.kper;                       // this workgroup's macro steps
    const int ms_end = min(nmacro, ms_begin + g.kper);
    const int64_t kend = min(g.K, (int64_t)ms_end * MACRO);

    // ---- X windows: global -> registers early, registers -> LDS later ----
    u32x4 xr[XCH];
    auto fetch_x = [&](int win) {
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = tid + NT * q;                  // chunk id: row = c / C8, col8 = c % C8
            const int row = c / C8, col8 = c % C8;
            const int64_t k = (int64_t)win * XWIN + col8 * 8;
            const bool ok = c < XCHUNKS && row < g.M && k < kend;
            xr[q] = bload16(rX, ok ? (uint32_t)((row * g.K + k) * 2) : 0xFFFFFFF0u);
        }
    };
    auto store_x = [&](uint8_t *dst) {
#pragma unroll
        for (int q = 0; q < XCH; ++q) {
            const int c = tid + NT * q;
            const int row = c / C8, col8 = c % C8;
            if (c < XCHUNKS)
                *reinterpret_cast<u32x4 *>(dst + (row * XROW + col8 * 8) * 2) = to_planar(xr[q]);
        }
    };

    struct WStage {
        u32x4 w[2];
        uint32_t c2, c1;
    };
    auto load_w = [&](int ms, WStage &st) {
        const int64_t blk = (int64_t)ms * 4 + lg;
        const bool live = ms < ms_end && blk < nblk;
        const uint32_t off = (uint32_t)(ln * wrow_bytes + blk * 32);
        st.w[0] = bload16(rW, live ? off : 0xFFFFFFF0u);
        st.w[1] = bload16(rW, live ? off + 16 : 0xFFFFFFF0u);
        const uint32_t b = (uint32_t)(n * nblk + blk);
        const bool okr = live && n < g.N;
        st.c2 = bload1(rC2, okr ? b : 0xFFFFFFF0u);
        st.c1 = bload4(rC1, okr ? (b >> 8) * 4 : 0xFFFFFFF0u);
    };

    f32x4 acc[G];
#pragma unroll
    for (int q = 0; q < G; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto macro_step = [&](int ms, const WStage &st, const uint8_t *Xw) {
        const int kin = (ms * MACRO) % XWIN;             // column offset inside the window
        const int64_t blk = (int64_t)ms * 4 + lg;
        float a = block_scale(st.c2, __uint_as_float(st.c1), mean, dq_i8);
        if (ms >= ms_end || blk >= nblk) a = 0.0f;        // past the split or K: contributes nothing
        const Lut t = make_lut(g.cb, a);
        const uint32_t wd[8] = {st.w[0].x, st.w[0].y, st.w[0].z, st.w[0].w,
                                st.w[1].x, st.w[1].y, st.w[1].z, st.w[1].w};
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            const u32x4 b = dequant8_planar(t, wd[d]);
            // A of group q: X row 16 q + ln, columns kin + 64 lg + 8 d .. +7 (planar, as b)
#pragma unroll
            for (int q = 0; q < G; ++q) {
                const u32x4 av =
                    *reinterpret_cast<const u32x4 *>(Xw + ((16 * q + ln) * XROW + kin + lg * 64 + d * 8) * 2);
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                                 __builtin_bit_cast(bf16x8, b), acc[q], 0, 0, 0);
            }
        }
    };

    // WPW macro steps per X window; W is fetched four macro steps ahead.  Window w+1 is fetched
    // at the first macro step of window w, written to the other LDS buffer halfway through it,
    // and made visible by the barrier that closes window w.  ms_begin and the split length are
    // multiples of 4 (whole windows); one loop pass is 4 macro steps.
    WStage S[4];
    fetch_x(ms_begin / WPW);
    store_x(Xs0);
#pragma unroll
    for (int h = 0; h < 4; ++h) load_w(ms_begin + h, S[h]);

    // s T (the last split, which adds the LoRA term) and T (workgroup 0) from T's partials while
    // the first weight steps stream in
    if (!g.Tp) {
        if (split == g.ksplit - 1) {
            const uint2 *src = reinterpret_cast<const uint2 *>(g.sT);
            for (int i = tid; i < (int)((g.M * g.r) >> 2); i += NT) reinterpret_cast<uint2 *>(sTs)[i] = src[i];
        }
    } else if (split == g.ksplit - 1 || blockIdx.x == 0) {
        typedef float f32v4 __attribute__((ext_vector_type(4)));
        const int64_t E = g.M * g.r;
        const f32v4 *Tp = reinterpret_cast<const f32v4 *>(g.Tp);
        for (int i = tid; i < (int)(E >> 2); i += NT) {
            f32v4 acc = Tp[i];
            for (int k0 = 1; k0 < g.ksT; k0 += 8) {
                f32v4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (k0 + u < g.ksT) v[u] = Tp[(int64_t)(k0 + u) * (E >> 2) + i];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (k0 + u < g.ksT) acc += v[u];
            }
            const float sc = g.tscale;
            *reinterpret_cast<uint2 *>(sTs + 4 * i) = uint2{pack_bf16x2(sc * acc.x, sc * acc.y),
                                                            pack_bf16x2(sc * acc.z, sc * acc.w)};
            if (blockIdx.x == 0 && g.T_out)
                reinterpret_cast<uint2 *>(g.T_out)[i] = uint2{pack_bf16x2(1.0f * acc.x, 1.0f * acc.y),
                                                              pack_bf16x2(1.0f * acc.z, 1.0f * acc.w)};
        }
    }
    __syncthreads();
    for (int ms = ms_begin; ms < ms_end; ms += 4) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int m = ms + h;
            const bool odd = (((m - ms_begin) / WPW) & 1) != 0;   // window parity
            uint8_t *Xcur = odd ? Xs1 : Xs0;
            uint8_t *Xnxt = odd ? Xs0 : Xs1;
            if (h % WPW == 0) fetch_x(m / WPW + 1);               // past the split's end: zeros
            macro_step(m, S[h], Xcur);
            load_w(m + 4, S[h]);
            if (h % WPW == WPW / 2 - 1) store_x(Xnxt);
            if (h % WPW == WPW - 1) __syncthreads();
        }
    }

    // ---- LoRA (last split): acc += (s T) L2 over r in steps of 32 (two MFMAs for r = 64) ----
    const __amdgpu_buffer_rsrc_t rL2 = make_rsrc(g.L2, (int64_t)g.r * g.N * 2);
    const int rlora = split == g.ksplit - 1 ? g.r : 0;
    for (int j0 = 0; j0 < rlora; j0 += 32) {
        // A of group q: sT row 16 q + ln, j = j0 + 8 lg .. +7 (natural order); B: L2[j][n] for
        // the same j
        const int jj = j0 + lg * 8;
        uint32_t bw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ja = jj + 2 * i, jb = ja + 1;
            const uint32_t lo = bload2(rL2, (ja < g.r && n < g.N) ? (uint32_t)(((int64_t)ja * g.N + n) * 2) : 0xFFFFFFF0u);
            const uint32_t hi = bload2(rL2, (jb < g.r && n < g.N) ? (uint32_t)(((int64_t)jb * g.N + n) * 2) : 0xFFFFFFF0u);
            bw[i] = (lo & 0xFFFFu) | (hi << 16);
        }
        const u32x4 bv = {bw[0], bw[1], bw[2], bw[3]};
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const int64_t row = 16 * q + ln;
            const bool oka = row < g.M && jj < g.r;
            const u32x4 av = oka ? *reinterpret_cast<const u32x4 *>(sTs + row * g.r + jj) : u32x4{0u, 0u, 0u, 0u};
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                             __builtin_bit_cast(bf16x8, bv), acc[q], 0, 0, 0);
        }
    }

    // ---- store: lane holds rows 16 q + 4 lg + i (tokens) of group q, column n ----
    if (n < g.N) {
        float *P = g.P + (int64_t)split * g.M * g.N;
#pragma unroll
        for (int q = 0; q < G; ++q) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t m = 16 * q + lg * 4 + i;
                if (m < g.M) {
                    if (g.ksplit > 1) P[m * g.N + n] = acc[q][i];
                    else g.Y[m * g.N + n] = (uint16_t)f32_to_bf16(acc[q][i]);
                }
            }
        }
    }
}

// 16 token rows: 1 to 8 waves; 32 and 64 rows: 4 to 8 (fewer waves would hold a larger share of
// the X window in registers)
template <int MROWS, bool I8>
void launch_i8(const GemvArgs &a, int nw, int grid, hipStream_t stream) {
    const dim3 gd(grid);
    switch (nw) {
        case 1: if constexpr (MROWS == 16) hipLaunchKernelGGL((gemv_kernel<MROWS, I8, 1>), gd, dim3(64), 0, stream, a); break;
        case 2: if constexpr (MROWS == 16) hipLaunchKernelGGL((gemv_kernel<MROWS, I8, 2>), gd, dim3(128), 0, stream, a); break;
        case 3: if constexpr (MROWS == 16) hipLaunchKernelGGL((gemv_kernel<MROWS, I8, 3>), gd, dim3(192), 0, stream, a); break;
        case 4: hipLaunchKernelGGL((gemv_kernel<MROWS, I8, 4>), gd, dim3(256), 0, stream, a); break;
        case 5: hipLaunchKernelGGL((gemv_kernel<MROWS, I8, 5>), gd, dim3(320), 0, stream, a); break;
        case 6: hipLaunchKernelGGL((gemv_kernel<MROWS, I8, 6>), gd, dim3(384), 0, stream, a); break;
        case 7: hipLaunchKernelGGL((gemv_kernel<MROWS, I8, 7>), gd, dim3(448), 0, stream, a); break;
        default: hipLaunchKernelGGL((gemv_kernel<MROWS, I8, 8>), gd, dim3(512), 0, stream, a); break;
    }
}
void launch_nw(const GemvArgs &a, int nw, int grid, hipStream_t stream) {
    if (a.M > 32) {
        if (a.dq_int8) launch_i8<64, true>(a, nw, grid, stream);
        else launch_i8<64, false>(a, nw, grid, stream);
    } else if (a.M > 16) {
        if (a.dq_int8) launch_i8<32, true>(a, nw, grid, stream);
        else launch_i8<32, false>(a, nw, grid, stream);
    } else {
        if (a.dq_int8) launch_i8<16, true>(a, nw, grid, stream);
        else launch_i8<16, false>(a, nw, grid, stream);
    }
}

// waves per block: about one block per CU, and at least 4 (each block stages the whole X window
// for its rows, so fewer waves would read X from L2 more often than W from HBM); 32 and 64 token
// rows keep 4 waves even for fewer row groups (the idle waves store nothing)
int wide_waves(int64_t M, int64_t N) {
    const int64_t groups = (N + 15) / 16;
    int nw = (int)((groups + 255) / 256);
    nw = nw < 4 ? 4 : (nw > NWAVE_MAX ? NWAVE_MAX : nw);
    if (groups < nw && M <= 16) nw = (int)groups;
    return nw;
}
}  // namespace

// Split the reduction when the row blocks leave CUs idle: S = 256 / blocks workgroups per row
// block, each over a whole number of 4 macro steps (whole X windows), no split empty.  A block
// with little work (macro steps x 16-token groups under 32, e.g. 16 tokens at K = 4096) is not
// split: the partials' reduction launch costs more than the idle CUs (measured 1-3 us either way).
SplitPlan gemv_wide_split(int64_t M, int64_t N, int64_t K) {
    const int nw = wide_waves(M, N);
    const int64_t blocks = ((N + 15) / 16 + nw - 1) / nw;
    const int64_t nmacro = (K + MACRO - 1) / MACRO, nwin = (nmacro + 3) / 4;
    const int64_t groups = M > 32 ? 4 : (M > 16 ? 2 : 1);
    if (nmacro * groups < 32) return SplitPlan{1, nwin * 4};
    int64_t s = blocks > 0 ? 256 / blocks : 1;
    if (s > nwin) s = nwin;
    if (s > 16) s = 16;
    if (s <= 1) return SplitPlan{1, nwin * 4};
    const int64_t wper = (nwin + s - 1) / s;
    s = (nwin + wper - 1) / wper;
    return s <= 1 ? SplitPlan{1, nwin * 4} : SplitPlan{(int)s, wper * 4};
}

hipError_t launch_gemv_wide_fwd(const WeightView &w, const uint16_t *X, const Reduction *Tred, const uint16_t *sT,
                                const uint16_t *L2, int32_t r, int64_t M, uint16_t *Y, const SplitK &sk,
                                hipStream_t stream) {
    if (M < 1 || M > 64) return hipErrorInvalidValue;
    GemvArgs a;
    a.X = X;
    a.packed = w.packed; a.c2 = w.c2; a.c1 = w.c1; a.mean = w.mean; a.dq_int8 = w.dq_int8;
    a.L2 = L2; a.Y = Y;
    if (r < 8 || r > R_MAX || r % 8 || (Tred == nullptr) == (sT == nullptr)) return hipErrorInvalidValue;
    if (Tred) {
        if (Tred->n != M * r || Tred->nsplit < 1 || Tred->s1 != 1.0f || Tred->stride) return hipErrorInvalidValue;
        a.Tp = Tred->P; a.ksT = Tred->nsplit; a.tscale = Tred->s2; a.T_out = Tred->out; a.sT = nullptr;
    } else {
        a.Tp = nullptr; a.ksT = 0; a.tscale = 0.0f; a.T_out = nullptr; a.sT = sT;
    }
    a.M = M; a.N = w.rows; a.K = w.cols; a.r = r;
    for (int j = 0; j < 16; ++j) a.cb.v[j] = w.cb[j];
    const int nw = wide_waves(M, w.rows);
    if (M > 16 && nw < 4) return hipErrorInvalidValue;
    const int64_t nmacro = (w.cols + MACRO - 1) / MACRO;
    a.ksplit = sk.ksplit > 1 ? sk.ksplit : 1;
    a.kper = (int32_t)(a.ksplit > 1 ? sk.per : (nmacro + 3) / 4 * 4);
    a.P = sk.P;
    // every split non-empty and made of whole windows: what the kernel's window loop assumes
    if (a.ksplit > 1 && (!sk.P || sk.per % 4 || (int64_t)(a.ksplit - 1) * sk.per >= nmacro ||
                         (int64_t)a.ksplit * sk.per < nmacro))
        return hipErrorInvalidValue;
    const int64_t groups = (w.rows + 15) / 16;
    const int grid = (int)((groups + nw - 1) / nw) * a.ksplit;
    timing_before(stream, 2);
    launch_nw(a, nw, grid, stream);
    hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace nf4k
