// Decode-size forward (M <= 4 tokens) of the QLoRA linear layer (gfx950):
//   Y = X deq(W)^T + s (X L1) L2
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (5) / eq. (6); section 4 eq. (3).
//
// This shape streams the 4-bit weight once from HBM; the work to hide behind that stream is the
// decoding of the codes.  Two launches:
//
// gemv_main_kernel: workgroups of 8 waves.  "T" workgroups (first in the grid, so dispatched
//   first) compute K-slices of T = X L1; "W" workgroups own 64 weight rows and one K segment.
//   - v_mfma_f32_4x4x4_16b_bf16: B lane l holds 4 codes of one weight row, so M <= 4 tokens waste
//     no MFMA row; A (X) is broadcast inside pairs of blocks (CBSZ = 1).
//   - every weight load reads whole 128-byte lines: a load covers 8 rows x 128 bytes and each
//     lane's 16 bytes feed 8 MFMAs directly (no LDS staging of W).
//   - codes are decoded through a pair table in LDS: entry e (one packed byte) holds the bf16
//     codebook values of its two nibbles; 64 copies side by side so that lane l always reads
//     bank l (conflict-free).  The address is one v_perm (the code byte next to the lane offset),
//     the lookup one ds_read_b32 per two weights.
//   - the table is the plain codebook, so each block is accumulated on its own and the block
//     constant a = c2 * s2 + mean (eq. 6, rebuilt in fp32) multiplies the fp32 partial:
//     y = sum_blocks a_b sum_{k in b} x_k cb[q_k].  This equals X deq(W)^T up to rounding, with
//     the codebook rounded to bf16 instead of each product cb * a.
//   - the block constants of the workgroup's rows and K segment are staged in LDS once.
// gemv_epilogue_kernel: sums the K-segment partials of X deq(W)^T and the K-slices of T, rounds
//   s T to bf16 and adds (s T) L2, stores bf16 Y (and T when asked).

#include "common.h"
#include "launch.h"

namespace nf4k {

namespace {

constexpr int NWAVE = 8;                       // waves per main-kernel workgroup
constexpr int NTHR = 64 * NWAVE;
constexpr int EWAVE = 4;                       // waves per epilogue workgroup
constexpr int MACRO_BLOCKS = 4;                // quantization blocks (of 64 columns) per macro step
constexpr int TCHUNK = 64 * 4 * NWAVE;         // K columns of T per T workgroup (four blocks per wave)
constexpr int TAB_COPIES = 64;                 // table copies: lane l reads copy l (bank l)
constexpr int SEG_BLOCKS = 128;                // max quantization blocks per K segment of a workgroup
constexpr int C2_ROW = SEG_BLOCKS + 4;         // staged code row (bytes): rows start one bank apart
constexpr int C1_MAX = 512;                    // max second-level constants per workgroup
constexpr uint32_t OOB = 0xFFFFFE00u;          // buffer offset past any range: loads return 0

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int64_t clamped = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0LL : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)clamped, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

template <int V>
struct IntC {
    static constexpr int value = V;
};
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(IntC<B>{});
        static_for<B + 1, E>(f);
    }
}

// C += A[block ABID] (broadcast to all 16 blocks) x B
template <int ABID>
__device__ __forceinline__ f32x4 mfma4(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                  c, 4, ABID, 0);
}

struct GemvArgs {
    const uint16_t *X;       // [M, K]
    const uint8_t *packed;   // [N, K/2]
    const uint8_t *c2;
    const float *c1;
    const float *mean;
    const uint16_t *L1;      // [K, r]
    float *Yp;               // [S, M, N] fp32 partials of X deq(W)^T
    float *Tp;               // [nkc, M, r] fp32 partials of X L1
    int64_t M, N, K;
    int32_t r, nseg, nrg, nt;   // K segments, 64-row groups, T workgroups
    Codebook cb;
};

// X fragment of one 64-column block for m-tile mt: lane (b = l / 4, i = l % 4) holds
// X[4 mt + i][k0 + 4 b .. + 3]
__device__ __forceinline__ u32x2 load_xfrag(__amdgpu_buffer_rsrc_t rX, const GemvArgs &g, int lane, int mt,
                                            int64_t blk, bool live) {
    const int64_t m = mt * 4 + (lane & 3);
    const int64_t k = blk * 64 + 4 * (lane >> 2);
    const bool ok = live && m < g.M && blk < (g.K >> 6);
    return bload8(rX, ok ? (uint32_t)((m * g.K + k) * 2) : OOB);
}

// C += A[block 2 g + ABID of each pair g of blocks] x B
template <int ABID>
__device__ __forceinline__ f32x4 mfma4_g2(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                  c, 1, ABID, 0);
}

// Work of one workgroup: RH x RS sets of 8 weight rows over one K segment.  Wave (h, k) of the
// NWAVE = RH x KW waves takes row sets h RS .. h RS + RS - 1 and every KW-th macro step of the
// segment starting at k, so that neighbouring waves read neighbouring bytes of the same rows.
// A macro step is four quantization blocks (256 columns, one 128-byte line of each row); its
// load q covers the 8 rows of row set q: lane l takes row 8 q + l % 8, bytes 16 (l / 8) .. + 15,
// so every load reads whole lines.  Those 16 bytes (32 columns, inside one quantization block)
// are the B operand of 8 MFMAs: MFMA t uses codes 4 t .. 4 t + 3.  The 8 lanes of one chunk g
// form broadcast pair g (blocks 2 g, 2 g + 1; rows 0..3 and 4..7), whose A operand (X) comes
// from block 2 g + t / 4: lane 8 g + 4 v + i holds X[i][32 g + 16 v .. + 15] for MFMAs 4 v .. 4 v + 3.
// Macro steps stream through a ring of NST register stages.
template <int MT, int RS, int RH, int NST>
__device__ void w_part(const GemvArgs &g, uint32_t *tab, int rg, int seg) {
    constexpr int KW = NWAVE / RH;
    constexpr int R = 8 * RS * RH;                       // rows of the workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wh = wave / KW, wk = wave % KW;
    const int64_t n0 = (int64_t)rg * R;
    const int64_t nw0 = n0 + wh * (8 * RS);              // first row of this wave
    const int64_t wrow = g.K >> 1, nblk = g.K >> 6;
    const int64_t nmacro = (nblk + MACRO_BLOCKS - 1) / MACRO_BLOCKS;
    const int64_t per_seg = (nmacro + g.nseg - 1) / g.nseg;
    const int64_t s0 = min((int64_t)seg * per_seg, nmacro), s1 = min(s0 + per_seg, nmacro);

    const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.packed + nw0 * wrow, (g.N - nw0) * wrow);
    const __amdgpu_buffer_rsrc_t rC2 = make_rsrc(g.c2, g.N * nblk);
    const __amdgpu_buffer_rsrc_t rC1 = make_rsrc(g.c1, ((g.N * nblk + 255) >> 8) * 4);
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(g.X, g.M * g.K * 2);
    const float mean = g.mean[0];

    const int G = lane >> 3, rl = lane & 7;            // chunk of the macro step, row in an 8-row set
    const int xv = (lane >> 2) & 1, xi = lane & 3;     // X half (MFMAs 4 xv ..) and token of this lane
    // byte offsets of row set 0; row set q adds 8 q rows (wave-uniform)
    const uint32_t wb = (uint32_t)(rl * wrow + 16 * G), wstep = (uint32_t)(8 * wrow);
    uint32_t xb[MT];
    bool xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = mt * 4 + xi;
        xrow[mt] = m < g.M;
        xb[mt] = (uint32_t)((m * g.K + 32 * G + 16 * xv) * 2);
    }

    struct Stage {
        u32x4 w[RS];            // rows 8 q + rl: 32 codes each
        u32x4 x[MT][2];         // X[4 mt + xi][32 G + 16 xv + 8 h .. + 7]
    };
    // Loads past the wave's range need no guard except X: W then reads other finite data (or
    // zeros past the end), which the zero X fragments cancel.
    auto load = [&](int64_t ms, Stage &S) {
        const uint32_t wo = (uint32_t)(ms * (MACRO_BLOCKS * 32));
#pragma unroll
        for (int q = 0; q < RS; ++q) S.w[q] = bload16(rW, wb + q * wstep + wo);
        // 32-bit lane-uniform test plus a per-lane mask: no branches around the loads
        const uint32_t msu = (uint32_t)ms;
        const uint32_t xo = msu * (MACRO_BLOCKS * 128);
        const bool live = msu < (uint32_t)s1 && msu * MACRO_BLOCKS + (uint32_t)(G >> 1) < (uint32_t)nblk;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint32_t xa = (live && xrow[mt]) ? xb[mt] + xo : OOB;
#pragma unroll
            for (int h = 0; h < 2; ++h) S.x[mt][h] = bload16(rX, xa + 16 * h);
        }
    };

    // the first NST macro steps are in flight before the tables are built
    Stage st[NST];
    const int64_t msb = s0 + wk;                         // first macro step of this wave
#pragma unroll
    for (int i = 0; i < NST; ++i) load(msb + (int64_t)i * KW, st[i]);

    // ---- block constants of the workgroup's rows and K segment, staged in LDS once ----
    // (per-lane loads of single code bytes would touch a cache line each)
    __shared__ uint8_t c2s[R * C2_ROW];
    __shared__ float c1s[C1_MAX];
    const int64_t b_lo = s0 * MACRO_BLOCKS, b_hi = min(s1 * MACRO_BLOCKS, nblk);
    const int nb = (int)(b_hi - b_lo);
    const int64_t c1_lo = (n0 * nblk + b_lo) >> 8;
    {
        for (int i = tid; i < R * SEG_BLOCKS; i += NTHR) {
            const int row = i / SEG_BLOCKS, b = i % SEG_BLOCKS;
            c2s[row * C2_ROW + b] = (uint8_t)bload1(rC2, b < nb ? (uint32_t)((n0 + row) * nblk + b_lo + b) : OOB);
        }
        const int64_t c1_hi = ((n0 + R - 1) * nblk + b_hi - 1) >> 8;
        for (int i = tid; i <= (int)(c1_hi - c1_lo); i += NTHR)
            c1s[i] = __uint_as_float(bload4(rC1, (uint32_t)((c1_lo + i) * 4)));
    }

    // ---- LDS pair table: entry e, copy c at byte e * 256 + 4 c ----
    __shared__ uint32_t cbh[16];
    if (tid < 16) {
        float v = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) v = (tid == j) ? g.cb.v[j] : v;
        cbh[tid] = f32_to_bf16(v);
    }
    __syncthreads();
    {
        const int c = tid & 63;
#pragma unroll 8
        for (int q = 0; q < 256 / NWAVE; ++q) {
            const int e = wave + NWAVE * q;
            tab[e * TAB_COPIES + c] = cbh[e & 15] | (cbh[e >> 4] << 16);
        }
    }
    __syncthreads();

    const uint32_t lb = (uint32_t)lane << 2;
    const char *tabc = reinterpret_cast<const char *>(tab);
    f32x4 acc[RS][MT];
#pragma unroll
    for (int q = 0; q < RS; ++q)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // B fragments of MFMA t for the row sets (two table lookups each)
    auto lookup = [&](const Stage &S, auto tc, u32x2 (&bv)[RS]) {
        constexpr int t = decltype(tc)::value;
        // byte 2 t (2 t + 1) of the chunk goes to address bits 8..15 next to the lane offset
        constexpr uint32_t sel0 = 0x0C0C0000u | ((4u + 2u * (t & 1)) << 8);
        constexpr uint32_t sel1 = 0x0C0C0000u | ((5u + 2u * (t & 1)) << 8);
#pragma unroll
        for (int q = 0; q < RS; ++q) {
            const uint32_t wd = S.w[q][t >> 1];
            bv[q].x = *reinterpret_cast<const uint32_t *>(tabc + __builtin_amdgcn_perm(wd, lb, sel0));
            bv[q].y = *reinterpret_cast<const uint32_t *>(tabc + __builtin_amdgcn_perm(wd, lb, sel1));
        }
    };
    // Each row set and 32-column chunk is one quantization block: its 8 MFMAs accumulate from
    // zero and the block constant then scales the fp32 partial.  Lookups run one MFMA step ahead.
    auto compute = [&](const Stage &S, int64_t ms) {
        // block constants of this step: row 8 q + rl, block 4 ms + G / 2 (eq. 6, fp32)
        float a[RS];
#pragma unroll
        for (int q = 0; q < RS; ++q) {
            const int row = wh * (8 * RS) + 8 * q + rl;
            const int b = (int)(ms * MACRO_BLOCKS - b_lo) + (G >> 1);
            const int bc = b < nb ? b : 0;                  // past the segment: X is zero
            const int64_t qi = (n0 + row) * nblk + b_lo + bc;
            a[q] = block_scale(c2s[row * C2_ROW + bc], c1s[(int)((qi >> 8) - c1_lo)], mean);
        }
        f32x4 tmp[RS][MT];
#pragma unroll
        for (int q = 0; q < RS; ++q)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) tmp[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x2 bv[2][RS];
        lookup(S, IntC<0>{}, bv[0]);
        static_for<0, 8>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            if constexpr (t + 1 < 8) lookup(S, IntC<t + 1>{}, bv[(t + 1) % 2]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                // X of MFMA t: elements 4 (t % 4) .. + 3 of this lane's 16-element half
                const u32x4 &xx = S.x[mt][(t % 4) >> 1];
                const u32x2 xf = (t & 1) ? u32x2{xx.z, xx.w} : u32x2{xx.x, xx.y};
#pragma unroll
                for (int q = 0; q < RS; ++q) tmp[q][mt] = mfma4_g2<t / 4>(xf, bv[t % 2][q], tmp[q][mt]);
            }
        });
#pragma unroll
        for (int q = 0; q < RS; ++q)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[q][mt] += a[q] * tmp[q][mt];
    };

    for (int64_t ms = msb; ms < s1; ms += NST * KW) {
        static_for<0, NST>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            compute(st[i], ms + i * KW);
            load(ms + (i + NST) * KW, st[i]);
        });
    }

    // ---- the eight chunks of a row live in lanes rl, rl + 8, ..., rl + 56 ----
#pragma unroll
    for (int q = 0; q < RS; ++q)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = acc[q][mt][i];
                v += __shfl_xor(v, 8);
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                acc[q][mt][i] = v;
            }
    // ---- sum the KW waves of each row set through LDS (the table is no longer read) ----
    __syncthreads();
    f32x4 *red = reinterpret_cast<f32x4 *>(tab);            // [wave][q][mt][rl]
    if (G == 0) {
#pragma unroll
        for (int q = 0; q < RS; ++q)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) red[((wave * RS + q) * MT + mt) * 8 + rl] = acc[q][mt];
    }
    __syncthreads();
    float *Yp = g.Yp + (int64_t)seg * g.M * g.N;
    for (int idx = tid; idx < MT * 4 * R; idx += NTHR) {
        const int m = idx / R, nl = idx % R;                // nl = 8 (h RS + q) + rl
        const int mt = m >> 2, i = m & 3;
        const int h = nl / (8 * RS), q = (nl / 8) % RS, r8 = nl & 7;
        float v = 0.0f;
#pragma unroll
        for (int k = 0; k < KW; ++k) v += red[(((h * KW + k) * RS + q) * MT + mt) * 8 + r8][i];
        if (m < g.M && n0 + nl < g.N) Yp[m * g.N + n0 + nl] = v;
    }
}

template <int MT>
__device__ void t_part(const GemvArgs &g, uint32_t *lds, int t) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rt = (g.r + 63) >> 6;
    const int kc = t / rt, ct = t % rt;
    const int64_t c = (int64_t)ct * 64 + lane;          // this lane's T column
    const int64_t nblk = g.K >> 6;
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(g.X, g.M * g.K * 2);
    const __amdgpu_buffer_rsrc_t rL1 = make_rsrc(g.L1, g.K * g.r * 2);

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int64_t blk0 = ((int64_t)kc * TCHUNK + wave * (TCHUNK / NWAVE)) >> 6;
#pragma unroll 1
    for (int b = 0; b < TCHUNK / NWAVE / 64; ++b) {
        const int64_t blk = blk0 + b;
        const bool live = blk < nblk;
        u32x2 xf[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) xf[mt] = load_xfrag(rX, g, lane, mt, blk, live);
        uint32_t e[64];
        const uint32_t cbase = (live && c < g.r) ? (uint32_t)((blk * 64 * g.r + c) * 2) : OOB;
        const uint32_t rstride = (uint32_t)(g.r * 2);
#pragma unroll
        for (int q = 0; q < 64; ++q) e[q] = bload2(rL1, cbase == OOB ? OOB : cbase + q * rstride);
        static_for<0, 16>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            u32x2 bv;
            bv.x = __builtin_amdgcn_perm(e[4 * s + 1], e[4 * s], 0x05040100u);
            bv.y = __builtin_amdgcn_perm(e[4 * s + 3], e[4 * s + 2], 0x05040100u);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma4<s>(xf[mt], bv, acc[mt]);
        });
    }
    f32x4 *red = reinterpret_cast<f32x4 *>(lds);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[(wave * MT + mt) * 64 + lane] = acc[mt];
    __syncthreads();
    float *Tp = g.Tp + (int64_t)kc * g.M * g.r;
    for (int idx = tid; idx < MT * 4 * 64; idx += NTHR) {
        const int m = idx >> 6, cl = idx & 63;
        const int mt = m >> 2, i = m & 3;
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < NWAVE; ++w) v += red[(w * MT + mt) * 64 + cl][i];
        const int64_t cc = (int64_t)ct * 64 + cl;
        if (m < g.M && cc < g.r) Tp[m * g.r + cc] = v;
    }
}

// Row sets per wave (RS), row groups per workgroup (RH) and register stages (NST), chosen so
// that a wave stays within 128 registers (four waves per SIMD).  MT = 1: up to 4 tokens.
template <int MT>
struct WCfg {
    static constexpr int RS = 2;
    static constexpr int RH = 4;
    static constexpr int NST = 2;
    static constexpr int ROWS = 8 * RS * RH;
};

template <int MT>
__global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(4, 4))) void gemv_main_kernel(GemvArgs g) {
    __shared__ __align__(16) uint32_t tab[256 * TAB_COPIES];
    // the T workgroups come first so that they are dispatched first
    const int wg = blockIdx.x;
    if (wg < g.nt)
        t_part<MT>(g, tab, wg);
    else
        w_part<MT, WCfg<MT>::RS, WCfg<MT>::RH, WCfg<MT>::NST>(g, tab, (wg - g.nt) % g.nrg, (wg - g.nt) / g.nrg);
}

struct EpiArgs {
    const float *Yp;         // [S, M, N]
    const float *Tp;         // [nkc, M, r]
    const uint16_t *L2;      // [r, N]
    uint16_t *Y;             // [M, N]
    uint16_t *T_out;         // [M, r] or null
    int64_t M, N;
    int32_t r, nseg, nkc;
    float scale;
};

// One workgroup per 64 output columns: s T is rebuilt from the K-slice partials, each wave adds
// a quarter of the r terms of (s T) L2 for every token, and the quarters meet in LDS.  All global
// loads are unconditional buffer loads (out-of-range ones return zero) issued before the first
// barrier, so the kernel waits for memory once.
template <int MT>
__global__ __launch_bounds__(256) void gemv_epilogue_kernel(EpiArgs e) {
    constexpr int MM = 4 * MT;
    constexpr int TB = 16;                        // T partials per entry loaded together
    __shared__ float sT[MM][128];
    __shared__ float part[EWAVE][MM][64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * 64, n = n0 + lane;
    const int jq = e.r / EWAVE, j0 = wave * jq;   // r <= 128 and a multiple of 8: jq <= 32
    const int E = (int)e.M * e.r;
    const __amdgpu_buffer_rsrc_t rL2 = make_rsrc(e.L2, (int64_t)e.r * e.N * 2);
    const __amdgpu_buffer_rsrc_t rY = make_rsrc(e.Yp, (int64_t)e.nseg * e.M * e.N * 4);
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(e.Tp, (int64_t)e.nkc * E * 4);

    uint32_t l2raw[32];
#pragma unroll
    for (int q = 0; q < 32; ++q)
        l2raw[q] = bload2(rL2, (q < jq && n < e.N) ? (uint32_t)(((int64_t)(j0 + q) * e.N + n) * 2) : OOB);
    // base products of this thread's outputs (m, column) = (idx / 64, idx % 64), summed over segments
    float ybase[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int idx = tid + 256 * j, m = idx >> 6;
        const int64_t nn = n0 + (idx & 63);
        const bool ok = m < e.M && nn < e.N;
        float y = 0.0f;
        for (int sg = 0; sg < e.nseg; ++sg)
            y += __uint_as_float(bload4(rY, ok ? (uint32_t)((((int64_t)sg * e.M + m) * e.N + nn) * 4) : OOB));
        ybase[j] = y;
    }
    // T partials of this thread's entries of s T (at most MM * 128 / 256 = 2 MT entries)
    float tsum[2 * MT];
#pragma unroll
    for (int j = 0; j < 2 * MT; ++j) {
        const int idx = tid + 256 * j;
        float t = 0.0f;
        for (int k0 = 0; k0 < e.nkc; k0 += TB) {
            float v[TB];
#pragma unroll
            for (int q = 0; q < TB; ++q)
                v[q] = __uint_as_float(bload4(rT, (idx < E && k0 + q < e.nkc)
                                                     ? (uint32_t)(((int64_t)(k0 + q) * E + idx) * 4) : OOB));
#pragma unroll
            for (int q = 0; q < TB; ++q) t += v[q];
        }
        tsum[j] = t;
    }
    // s T rounded to bf16, zero outside [0, M) x [0, r)
#pragma unroll
    for (int j = 0; j < MM * 128 / 256; ++j) {
        const int idx = tid + 256 * j;
        reinterpret_cast<float *>(sT)[idx] = 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2 * MT; ++j) {
        const int idx = tid + 256 * j;
        if (idx < E) {
            if (blockIdx.x == 0 && e.T_out) e.T_out[idx] = (uint16_t)f32_to_bf16(tsum[j]);
            sT[idx / e.r][idx % e.r] = bf16_to_f32(f32_to_bf16(e.scale * tsum[j]));
        }
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        float acc = 0.0f;
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            const int j = min(j0 + q, 127);          // past r: l2 is zero and sT is zero
            acc = __builtin_fmaf(sT[m][j], bf16_to_f32(l2raw[q] & 0xFFFFu), acc);
        }
        part[wave][m][lane] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MT; ++j) {
        const int idx = tid + 256 * j, m = idx >> 6, nl = idx & 63;
        const int64_t nn = n0 + nl;
        if (m < e.M && nn < e.N) {
            const float y = ybase[j] + part[0][m][nl] + part[1][m][nl] + part[2][m][nl] + part[3][m][nl];
            e.Y[m * e.N + nn] = (uint16_t)f32_to_bf16(y);
        }
    }
}

template <int MT>
hipError_t launch_mt(const GemvArgs &a, const EpiArgs &e, int grid_main, hipStream_t stream) {
    timing_before(stream, 2);
    hipLaunchKernelGGL(gemv_main_kernel<MT>, dim3(grid_main), dim3(NTHR), 0, stream, a);
    hipError_t err = hipGetLastError();
    timing_after(stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(gemv_epilogue_kernel<MT>, dim3((unsigned)((e.N + 63) / 64)), dim3(256), 0, stream, e);
    return hipGetLastError();
}

int rows_per_wg(int64_t) { return WCfg<1>::ROWS; }

}  // namespace

GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K, int32_t r) {
    GemvPlan p;
    const int64_t nrg = (N + rows_per_wg(M) - 1) / rows_per_wg(M);
    const int64_t nmacro = ((K >> 6) + MACRO_BLOCKS - 1) / MACRO_BLOCKS;
    // about two workgroups per CU (16 waves), each wave keeping at least two macro steps
    int64_t s = 512 / nrg;
    if (s > nmacro / 8) s = nmacro / 8;
    if (s < 1) s = 1;
    // a segment's block constants fit the LDS staging area
    const int64_t min_seg = (nmacro * MACRO_BLOCKS + SEG_BLOCKS - 1) / SEG_BLOCKS;
    if (s < min_seg) s = min_seg;
    p.nseg = (int)s;
    p.nkc = (int)((K + TCHUNK - 1) / TCHUNK);
    p.yp_floats = (size_t)s * M * N;
    p.tp_floats = (size_t)p.nkc * M * r;
    (void)r;
    return p;
}

hipError_t launch_gemv_fwd(const WeightView &w, const uint16_t *X, const uint16_t *L1, const uint16_t *L2,
                           float scale, int32_t r, int64_t M, uint16_t *Y, uint16_t *T_out, float *Yp,
                           float *Tp, hipStream_t stream) {
    const GemvPlan p = gemv_plan(M, w.rows, w.cols, r);
    // second-level constants of one workgroup's rows must fit the LDS staging area
    if ((rows_per_wg(M) - 1) * (w.cols / 64) / 256 + 3 > C1_MAX) return hipErrorNotSupported;
    GemvArgs a;
    a.X = X;
    a.packed = w.packed; a.c2 = w.c2; a.c1 = w.c1; a.mean = w.mean;
    a.L1 = L1; a.Yp = Yp; a.Tp = Tp;
    a.M = M; a.N = w.rows; a.K = w.cols; a.r = r;
    a.nseg = p.nseg;
    a.nrg = (int)((w.rows + rows_per_wg(M) - 1) / rows_per_wg(M));
    for (int j = 0; j < 16; ++j) a.cb.v[j] = w.cb[j];
    const int rt = (r + 63) / 64;
    a.nt = p.nkc * rt;
    const int grid = a.nrg * a.nseg + a.nt;
    EpiArgs e;
    e.Yp = Yp; e.Tp = Tp; e.L2 = L2; e.Y = Y; e.T_out = T_out;
    e.M = M; e.N = w.rows; e.r = r; e.nseg = p.nseg; e.nkc = p.nkc; e.scale = scale;
    if (M > 4) return hipErrorInvalidValue;           // larger token counts take another path
    return launch_mt<1>(a, e, grid, stream);
}

}  // namespace nf4k
