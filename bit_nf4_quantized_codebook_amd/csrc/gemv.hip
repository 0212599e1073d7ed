// Decode-size forward (M <= 8 tokens) of the QLoRA linear layer (gfx950):
//   Y = X deq(W)^T + s (X L1) L2
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (5) / eq. (6); section 4 eq. (3).
//
// This shape streams the 4-bit weight once from HBM; everything else has to hide behind that
// stream.  Two launches:
//
// T's partials: gemv_t_kernel computes T = X L1 in slices of 64 rows of L1 for M <= 4; from 5
//   tokens the split-K skinny product of the LoRA kernels does.
//   Either way the fp32 partials are summed by the next launch in a fixed chunked order.
//
// gemv_rows_kernel: one workgroup of up to 16 waves per CU owns a run of R weight rows over the
//   whole reduction, so it finishes its outputs itself:
//   - KW waves side by side cover a row; a lane always takes the same 16-byte chunks (32
//     columns, half a quantization block), so its X values are loaded once and stay in
//     registers for every row.  The workgroup runs S = 16 / KW such row streams, each walking its
//     rows with U loads in flight per lane.
//   - one token: the 64 lanes of a wave take 64 chunks of the same row, one v_dot2_f32_bf16 per
//     code pair.  2 to 8 tokens: lane 4 b + j takes chunk b of row j of a 4-row group, and each
//     chunk feeds 8 v_mfma_f32_4x4x4_16b_bf16 per group of 4 tokens (v_dot2 issues at about a
//     quarter of the VALU rate, so more than one token goes to the matrix cores).
//   - codes are decoded through a pair table in LDS: entry e (one packed byte) holds the bf16
//     codebook values of its two nibbles, 64 copies side by side so that lane l reads bank l.
//     The address is one v_perm (the code byte next to the lane offset), the lookup one
//     ds_read_b32.
//   - the table is the plain codebook, so each half-block partial is scaled afterwards by its
//     block constant a = fma(e4m3(c2), c1, mean) (eq. 6, fp32), staged with the codes in LDS:
//     y = sum_blocks a_b sum_{k in b} x_k cb[q_k].  This equals X deq(W)^T up to rounding, with
//     the codebook rounded to bf16 instead of each product cb * a.
//   - lane partials are summed across the wave with lane swaps and DPP, across the KW waves in
//     LDS; the LoRA term (s T) L2 of the workgroup's rows (s T rounded to bf16, L2 staged in LDS
//     at the start) is added before the bf16 store.

#include "common.h"
#include "dqtile.h"
#include "launch.h"

namespace nf4k {

namespace {

constexpr uint32_t OOB = 0x80000000u;          // buffer offset past any range: loads return 0
constexpr int MAX_WAVES = 16;
constexpr int TAB_COPIES = 64;                 // lane l reads copy l
constexpr int TAB_WORDS = 256 * TAB_COPIES;    // 64 KB
constexpr int C2_CAP = 16384;                  // staged code bytes per workgroup
constexpr int C1_CAP = C2_CAP / 256 + 2;       // staged second-level constants
constexpr int R_MAX = 128;                     // rows per workgroup
constexpr int R_MAX_LORA = 128;                // r
constexpr int CSUM_CAP = 8192;                 // shared scratch: T's chunk sums, then the row partials
constexpr int PART_CAP = 2048;                 // KW * R partial sums (one token)
constexpr int RES_OFF = 4096;                  // 4x4-MFMA layout: batch partials below, row sums above
constexpr int T_THREADS = 256;
// rows of L1 per T workgroup: short slices spread the 1 MB-scale L1 read over many CUs (one CU
// alone pulls only a few tens of GB/s); their partials are summed by the consumer
constexpr int T_ROWS = 64;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    // lanes whose source is outside the 16-lane row read 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// bf16 codebook value of code j (selects over the kernel-argument copy; no indexed registers)
__device__ __forceinline__ uint32_t cb_bf16(const Codebook &cb, uint32_t j) {
    float v = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) v = (j == (uint32_t)q) ? cb.v[q] : v;
    return f32_to_bf16(v);
}

// ---------------------------------------------------------------------------------------------
// T = X L1, slice of T_ROWS rows of L1 per workgroup: Tp[slice][m][j]
// ---------------------------------------------------------------------------------------------
struct TArgs {
    const uint16_t *X;       // [M, K]
    const uint16_t *L1;      // [K, r]
    float *Tp;               // [nkc, M, r]
    int64_t M, K;
    int32_t r;
};

// T's slice partials are summed in chunks of 8 slices, each chunk from -0 in slice order, then the
// chunk sums from -0 in order.  Both consumers (the row kernel and the backward's recompute of T)
// run exactly these additions, so T has the same bits in the forward and the backward.
__device__ __forceinline__ void tp_chunk_load(__amdgpu_buffer_rsrc_t rT, int nkc, int E, int e, int c, bool ok,
                                              float (&v)[8]) {
    // conditions combined with & (not &&): the offset stays a select, with no branch around the load
    const bool base_ok = ok & (e < E);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t off = (uint32_t)(((8 * c + q) * E + e) * 4);
        v[q] = __uint_as_float(bload4(rT, (base_ok & (8 * c + q < nkc)) ? off : OOB));
    }
}
__device__ __forceinline__ float tp_chunk_add(int nkc, int c, const float (&v)[8]) {
    float t = -0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q)
        if (8 * c + q < nkc) t += v[q];
    return t;
}
__device__ __forceinline__ float tp_chunk_sum(__amdgpu_buffer_rsrc_t rT, int nkc, int E, int e, int c) {
    float v[8];
    tp_chunk_load(rT, nkc, E, e, c, true, v);
    return tp_chunk_add(nkc, c, v);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
constexpr int LGKM0_IMM = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// workgroup barrier for LDS traffic only: loads still in flight (weight rows, LDS copies issued
// later) stay in flight; __syncthreads would wait for them
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(LGKM0_IMM);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// T (unscaled, bf16) from the partials alone: thread per element
__global__ __launch_bounds__(256) void gemv_tsum_kernel(const float *Tp, int nkc, int E, uint16_t *T) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(Tp, (int64_t)nkc * E * 4);
    float t = -0.0f;
    for (int c = 0; c < (nkc + 7) >> 3; ++c) t += tp_chunk_sum(rT, nkc, E, e, c);
    if (e < E) T[e] = (uint16_t)f32_to_bf16(t);
}

template <int MM>
__global__ __launch_bounds__(T_THREADS) void gemv_t_kernel(TArgs a) {
    constexpr int T_PT = 4;                       // 16-byte L1 pieces per thread (r <= 128)
    __shared__ float xs[MM][T_ROWS];
    __shared__ __align__(16) float red[MM * T_THREADS * 8];   // [m][row lane][r]
    __shared__ float red2[MM * (T_THREADS + R_MAX_LORA)];    // [m][group][r]
    const int tid = threadIdx.x;
    const int CG = a.r >> 3;                      // 16-byte column groups of an L1 row
    const int RPS = T_THREADS / CG;               // rows per load step
    const int cg = tid % CG, rl = tid / CG;
    const int64_t k0 = (int64_t)blockIdx.x * T_ROWS;
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.X, a.M * a.K * 2);
    const __amdgpu_buffer_rsrc_t rL1 = make_rsrc(a.L1, a.K * a.r * 2);

    u32x4 v[T_PT];
#pragma unroll
    for (int i = 0; i < T_PT; ++i) {
        const int k = rl + RPS * i;
        const bool ok = rl < RPS && k < T_ROWS && k0 + k < a.K;
        v[i] = bload16(rL1, ok ? (uint32_t)(((k0 + k) * a.r + 8 * cg) * 2) : OOB);
    }
    constexpr int NXD = MM * T_ROWS / 2;          // dwords of the X chunk
#pragma unroll
    for (int q = 0; q < (NXD + T_THREADS - 1) / T_THREADS; ++q) {
        const int i = tid + T_THREADS * q;        // dword i: token m, columns 2 kp, 2 kp + 1
        const int m = i / (T_ROWS / 2), kp = i % (T_ROWS / 2);
        if (i < NXD) {
            const bool ok = m < a.M && k0 + 2 * kp < a.K;
            const uint32_t xv = bload4(rX, ok ? (uint32_t)((m * a.K + k0 + 2 * kp) * 2) : OOB);
            xs[m][2 * kp] = bf16_to_f32(xv & 0xFFFFu);
            xs[m][2 * kp + 1] = bf16_to_f32(xv >> 16);
        }
    }
    __syncthreads();
    float acc[MM][8];
#pragma unroll
    for (int m = 0; m < MM; ++m)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[m][e] = 0.0f;
#pragma unroll
    for (int i = 0; i < T_PT; ++i) {
        const int k = min(rl + RPS * i, T_ROWS - 1);  // invalid pieces are zero
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t wv = v[i][e >> 1];
            const float l = bf16_to_f32((e & 1) ? (wv >> 16) : (wv & 0xFFFFu));
#pragma unroll
            for (int m = 0; m < MM; ++m) acc[m][e] = __builtin_fmaf(xs[m][k], l, acc[m][e]);
        }
    }
    // sum over the RPS row lanes of each column: groups of 8 row lanes (the last may be short),
    // then the groups
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        reinterpret_cast<f32x4 *>(red)[(m * T_THREADS + tid) * 2] = f32x4{acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
        reinterpret_cast<f32x4 *>(red)[(m * T_THREADS + tid) * 2 + 1] = f32x4{acc[m][4], acc[m][5], acc[m][6], acc[m][7]};
    }
    __syncthreads();
    const int G1 = (RPS + 7) >> 3;                // groups of 8 row lanes per column
    for (int t0 = tid; t0 < G1 * a.r; t0 += T_THREADS) {
        const int g = t0 / a.r, j = t0 - g * a.r;
#pragma unroll
        for (int m = 0; m < MM; ++m) {
            float t = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int rl2 = 8 * g + q;
                if (rl2 < RPS) t += red[(m * T_THREADS + rl2 * CG) * 8 + j];
            }
            red2[(m * G1 + g) * a.r + j] = t;
        }
    }
    __syncthreads();
    for (int e = tid; e < MM * a.r; e += T_THREADS) {
        const int m = e / a.r, j = e - m * a.r;
        float t = 0.0f;
        for (int g = 0; g < G1; ++g) t += red2[(m * G1 + g) * a.r + j];
        if (m < a.M) a.Tp[((int64_t)blockIdx.x * a.M + m) * a.r + j] = t;
    }
}

// ---------------------------------------------------------------------------------------------
// X deq(W)^T + (s T) L2 for R rows per workgroup
// ---------------------------------------------------------------------------------------------
struct RowsArgs {
    const uint16_t *X;       // [M, K]
    const uint8_t *packed;   // [N, K/2]
    const uint8_t *c2;
    const float *c1;
    const float *mean;
    uint32_t dq_int8;        // second-level codes are int8 (else E4M3)
    const uint16_t *L2;      // [r, N]
    const float *Tp;         // [nkc, M, r]
    uint16_t *Y;             // [M, N]
    uint16_t *T_out;         // [M, r] or null
    int64_t M, N, K;
    int32_t r, nkc, KW, S, RS, R;
    float scale;
    Codebook cb;
};

// Sum p[g][m] over the 64 lanes for each row g of the batch.  Afterwards the lane `holder` of
// row g (BR = 8: lane 8 g + 7; BR = 4: lane 16 g + 15) has the total.
template <int BR, int MM>
__device__ __forceinline__ void reduce_rows(float (&p)[BR][MM], float (&out)[MM], int lane) {
#pragma unroll
    for (int m = 0; m < MM; ++m) {
        // lane bit 5: rows g and g + BR/2 trade halves
        float q[BR / 2];
#pragma unroll
        for (int g = 0; g < BR / 2; ++g) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[g][m]),
                                                             __float_as_uint(p[g + BR / 2][m]), false, false);
            q[g] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);   // row g + (BR/2) bit5
        }
        // lane bit 4: rows g and g + BR/4 of what is left
        float u[BR / 4];
#pragma unroll
        for (int g = 0; g < BR / 4; ++g) {
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(q[g]),
                                                             __float_as_uint(q[g + BR / 4]), false, false);
            u[g] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        float t;
        if constexpr (BR == 8) {
            // lane bit 3: exchange with lane ^ 8 (rotate the 16-lane row by 8)
            const bool b3 = (lane >> 3) & 1;
            const float keep = b3 ? u[1] : u[0], send = b3 ? u[0] : u[1];
            t = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x128, 0xF, 0xF, false));
            // the 8 lanes of a group: prefix sums end in lane 8 g + 7
            t += dpp<0x111>(t);
            t += dpp<0x112>(t);
            t += dpp<0x114>(t);
        } else {
            t = u[0];
            t += dpp<0x111>(t);
            t += dpp<0x112>(t);
            t += dpp<0x114>(t);
            t += dpp<0x118>(t);
        }
        out[m] = t;
    }
}

// Lane partials of the 4 x 4 MFMA layout, f32x4 c = tokens 0..3 of the lane's row j = lane % 4 at
// block b = lane / 4: summed over the 16 blocks.  Afterwards lane l with (l & 12) == 12 holds
// row l % 4, token 2 (l >> 5) + ((l >> 4) & 1).
__device__ __forceinline__ float reduce_blocks4(f32x4 c) {
    // lane bit 5: tokens 0, 1 stay in the lower half-wave, 2, 3 in the upper
    const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(c.x), __float_as_uint(c.z), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(c.y), __float_as_uint(c.w), false, false);
    const float q0 = __uint_as_float(s0[0]) + __uint_as_float(s0[1]);
    const float q1 = __uint_as_float(s1[0]) + __uint_as_float(s1[1]);
    // lane bit 4: token 2 b5 + b4
    const auto s2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(q0), __float_as_uint(q1), false, false);
    float t = __uint_as_float(s2[0]) + __uint_as_float(s2[1]);
    // lane bits 2, 3 (same row j, four blocks of the 16-lane row): prefix sums end in lanes 12..15
    t += dpp<0x114>(t);
    t += dpp<0x118>(t);
    return t;
}

// C += A B over 16 independent 4 x 4 x 4 blocks (bf16 inputs, fp32 accumulation)
__device__ __forceinline__ f32x4 mfma4x4(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4, u32x2{a0, a1}),
                                                  __builtin_bit_cast(s16x4, u32x2{b0, b1}), c, 0, 0, 0);
}

// MF = false: one token (M = 1): lanes of a wave take 64 consecutive 16-byte chunks of the same
//   row, products with v_dot2_f32_bf16, BR rows summed per cross-lane reduction.
// MF = true: MM = 4 or 8 tokens: lane 4 b + j takes chunk b of row j of a 4-row group, and
//   each 16-byte chunk (32 codes) feeds 8 v_mfma_f32_4x4x4_16b_bf16 per group of 4 tokens
//   (B = the four rows' decoded pairs, A = X of four tokens over the same 4 columns).
//   v_dot2_f32_bf16 issues at about a quarter of the VALU rate, so beyond one token the
//   products go to the matrix cores.  With 4 tokens the waves' partials of every row wait in LDS
//   for the epilogue (as with one token); with 8 they do not fit, and the cross-wave sums run
//   per batch of ITER row steps.
// I8: the second-level codes are int8 (else E4M3); a template parameter so that the E4M3 kernel
// carries no per-block select (it cost 2-3 % here).
template <int MM, int BR, int U, int NWMAX, bool MF, bool I8>
__global__ __launch_bounds__(NWMAX * 64) void gemv_rows_kernel(RowsArgs a) {
    // ring of 2 U register slots, loads U row steps ahead: step i sits in slot i % 2U, and the
    // load of step i + U lands in a slot whose step is already consumed, so no value moves
    // between registers (a move would wait for the load).  One loop iteration covers ITER steps.
    constexpr int RING = 2 * U;
    constexpr int ITER = BR > RING ? BR : RING;
    static_assert(ITER % BR == 0 && ITER % RING == 0, "static ring slots per iteration");
    constexpr int NX = MF ? MM / 4 : MM;        // X register groups (tokens, or groups of 4)
    constexpr int ROWS_STEP = MF ? 4 : 1;        // rows per row step and lane group
    constexpr int LANES_ROW = MF ? 16 : 64;      // 16-byte chunks of a row per wave and step
    constexpr int BROWS = ITER * ROWS_STEP;      // rows per batch of the cross-wave sums (MF)
    // 4 tokens: every row's wave partials stay in LDS (part [KW][R][4]) and the epilogue sums
    // them, as for one token; 8 tokens: the waves' partials of each batch of rows are summed
    // after the batch (all rows' would not fit)
    constexpr bool DEFER = MF && MM == 4;
    // staging areas are filled by whole-wave DMA copies (1 KB or 256 bytes per wave and step)
    __shared__ __align__(16) uint32_t tab[TAB_WORDS];
    __shared__ __align__(16) uint32_t c2s[(C2_CAP + 2048) / 4];
    __shared__ __align__(16) float c1s[128];
    __shared__ float sTs[MM * R_MAX_LORA];        // [MM][r]
    __shared__ __align__(16) uint16_t l2s[R_MAX_LORA * R_MAX];   // [r][R]
    __shared__ uint32_t cbh[16];
    // T's chunk sums in the prologue; afterwards the wave partials of the rows
    //   MF = false or 4 tokens: part [KW][R][MM];  8 tokens: part [wave][BROWS][MM] and res [R][MM]
    //   at RES_OFF
    __shared__ float scr[CSUM_CAP];
    float *csum = scr, *part = scr, *res = scr + RES_OFF;
    typedef __attribute__((address_space(3))) uint8_t lds_u8;

    const int tid = threadIdx.x, lane = tid & 63;
    const int nthr = blockDim.x, nw = nthr >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = wave / a.KW, kw = wave - s * a.KW;
    const int64_t n0 = (int64_t)blockIdx.x * a.R;
    const int nrows = (int)min((int64_t)a.R, a.N - n0);
    const int64_t nblk = a.K >> 6, wrow = a.K >> 1;
    const int nchunk = (int)(a.K >> 5);
    const int c = kw * LANES_ROW + (MF ? (lane >> 2) : lane);   // this lane's 16-byte chunk of a row
    const int jrow = MF ? (lane & 3) : 0;         // its row in a 4-row group
    const bool lane_ok = c < nchunk;
    const int rs0 = s * a.RS;                     // first local row of this stream
    const int nsteps = a.RS / ROWS_STEP;          // row steps of a stream
    auto lrow = [&](int i) { return rs0 + ROWS_STEP * i + jrow; };   // this lane's row at step i

    const __amdgpu_buffer_rsrc_t rW = make_rsrc(a.packed, a.N * wrow);
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(a.X, a.M * a.K * 2);
    auto wload = [&](int i) -> u32x4 {
        const bool ok = lane_ok & (i < nsteps) & (lrow(i) < nrows);
        const uint32_t off = (uint32_t)((n0 + lrow(i)) * wrow + 16 * c);
        return bload16(rW, ok ? off : OOB);
    };

    // ---- prologue.  Issue order: the LDS copies (codes, second-level constants, L2 columns), X,
    //      the first chunk of T's partials, then the first U weight steps.  The waits below stop
    //      short of the weight rows, which stream in while the workgroup sets up. ----
    const int64_t q0 = n0 * nblk;                 // first code of the workgroup
    const int nc2 = nrows * (int)nblk;
    const uintptr_t c2a = reinterpret_cast<uintptr_t>(a.c2 + q0);
    const int sh = (int)(c2a & 15);               // 16-byte pieces from the aligned address below
    const int n16 = (nc2 + sh + 15) >> 4;         // (never past the page holding the last code)
    {
        const __amdgpu_buffer_rsrc_t rC2 = make_rsrc(reinterpret_cast<const void *>(c2a - sh), (int64_t)n16 * 16);
        for (int i0 = wave * 64; i0 < n16; i0 += nthr)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rC2, (lds_void *)((lds_u8 *)c2s + i0 * 16), 16,
                                                     (uint32_t)((i0 + lane) * 16), 0, 0, 0);
    }
    const int64_t c1lo = q0 >> 8;
    const int nc1 = (int)(((q0 + nc2 - 1) >> 8) - c1lo + 1);
    if (wave < 2) {
        const __amdgpu_buffer_rsrc_t rC1 = make_rsrc(a.c1, ((a.N * nblk + 255) >> 8) * 4);
        const int i = wave * 64 + lane;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rC1, (lds_void *)((lds_u8 *)c1s + wave * 256), 4,
                                                 i < nc1 ? (uint32_t)((c1lo + i) * 4) : OOB, 0, 0, 0);
    }
    // L2 columns of the rows (used at the end): piece i = (j, p8) is L2[j][n0 + 8 p8 .. + 7]
    {
        const int R8 = a.R >> 3, npc = a.r * R8;
        const __amdgpu_buffer_rsrc_t rL2 = make_rsrc(a.L2, (int64_t)a.r * a.N * 2);
        for (int i0 = wave * 64; i0 < npc; i0 += nthr) {
            const int i = i0 + lane;
            const int j = i / R8, p8 = i - j * R8;
            const bool ok = i < npc && 8 * p8 < nrows;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rL2, (lds_void *)((lds_u8 *)l2s + i0 * 16), 16,
                                                     ok ? (uint32_t)(((int64_t)j * a.N + n0 + 8 * p8) * 2) : OOB,
                                                     0, 0, 0);
        }
    }
    // X[token][32 c + 2 i .. + 1] as bf16 pairs; token q (MF = false) or 4 q + jrow (MF = true)
    uint32_t x[NX][16];
#pragma unroll
    for (int q = 0; q < NX; ++q) {
        const int tok = MF ? 4 * q + jrow : q;
        const bool ok = lane_ok & (tok < a.M);
        const uint32_t off = (uint32_t)((tok * a.K + 32 * c) * 2);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const u32x4 v = bload16(rX, ok ? off + 16 * h : OOB);
            x[q][4 * h] = v.x; x[q][4 * h + 1] = v.y; x[q][4 * h + 2] = v.z; x[q][4 * h + 3] = v.w;
        }
    }
    // T's partials: pair p = (chunk p / EM, element p % EM); this thread's first pair
    const int E = (int)a.M * a.r, EM = MM * a.r, nch = (a.nkc + 7) >> 3, npair = nch * EM;
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(a.Tp, (int64_t)a.nkc * E * 4);
    // (the first PF pairs of each thread are loaded here; the 4 x 4 layout sums 4 M' x r elements)
    constexpr int PF = MF ? 4 : 1;
    float tv[PF][8];
#pragma unroll
    for (int f = 0; f < PF; ++f) {
        const int p = tid + f * nthr, pc = p / EM;
        tp_chunk_load(rT, a.nkc, E, p - pc * EM, pc, p < npair, tv[f]);
    }
    const float mean = a.mean[0];                 // (a load pending inside the loop would drain the ring)
    constexpr bool dq_i8 = I8;
    __builtin_amdgcn_sched_barrier(0);            // the weight rows go out last
    u32x4 ring[RING];
#pragma unroll
    for (int u = 0; u < U; ++u) ring[u] = wload(u);
    __builtin_amdgcn_sched_barrier(0);

    // pair table: dword e * 64 + copy holds cb[e & 15] | cb[e >> 4] << 16 (no loads involved)
    if (tid < 16) cbh[tid] = cb_bf16(a.cb, (uint32_t)tid);
    lds_barrier();
    for (int i = tid; i < TAB_WORDS / 4; i += nthr) {
        const uint32_t e = (uint32_t)i >> 4;
        const uint32_t v = cbh[e & 15u] | (cbh[e >> 4] << 16);
        reinterpret_cast<u32x4 *>(tab)[i] = u32x4{v, v, v, v};
    }
    // s T rounded to bf16 (zero past M): chunk sums, then the chunks in order
#pragma unroll
    for (int f = 0; f < PF; ++f) {
        const int p = tid + f * nthr;
        if (p < npair) csum[p] = tp_chunk_add(a.nkc, p / EM, tv[f]);
    }
    for (int p = tid + PF * nthr; p < npair; p += nthr) {
        const int cc = p / EM, e = p - cc * EM;
        csum[p] = tp_chunk_sum(rT, a.nkc, E, e, cc);
    }
    lds_barrier();
    for (int e = tid; e < EM; e += nthr) {
        float t = -0.0f;
        for (int cc = 0; cc < nch; ++cc) t += csum[cc * EM + e];
        sTs[e] = e < E ? bf16_to_f32(f32_to_bf16(a.scale * t)) : 0.0f;
        if (blockIdx.x == 0 && a.T_out && e < E) a.T_out[e] = (uint16_t)f32_to_bf16(t);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(U));     // all but the weight rows: the LDS copies landed
    lds_barrier();                                // (and the chunk sums were read: scr is free)

    // ---- the row steps of this stream ----
    const char *tabc = reinterpret_cast<const char *>(tab);
    const uint8_t *c2b = reinterpret_cast<const uint8_t *>(c2s) + sh;
    const uint32_t lb = (uint32_t)lane << 2;
    const int bcol = min(c >> 1, (int)nblk - 1);  // quantization block of the lane's columns
    // decode step i's 16 bytes (32 codes) into 16 bf16 pairs; returns the block constant
    auto decode = [&](int i, const u32x4 &w, uint32_t (&pr)[16]) -> float {
        // rows past the stream read zero codes; their clamped constant keeps sums finite
        const int rl = min(lrow(i), nrows - 1);
        const int qi = rl * (int)nblk + bcol;
        static_for<0, 16>([&](auto bc) {
            constexpr int bi = decltype(bc)::value;
            constexpr uint32_t sel = 0x0C0C0000u | ((4u + (bi & 3)) << 8);
            pr[bi] = *reinterpret_cast<const uint32_t *>(tabc + __builtin_amdgcn_perm(w[bi >> 2], lb, sel));
        });
        return block_scale(c2b[qi], c1s[(int)(((q0 + qi) >> 8) - c1lo)], mean, dq_i8);
    };
    const int nit = (nsteps + ITER - 1) / ITER;
    if constexpr (!MF) {
        const int gsel = BR == 8 ? (lane >> 3) : (lane >> 4);
        const bool holder = BR == 8 ? ((lane & 7) == 7) : ((lane & 15) == 15);
        for (int it = 0; it < nit; ++it) {
            static_for<0, ITER / BR>([&](auto sbc) {
                constexpr int sb = decltype(sbc)::value;
                float p[BR][MM];
                static_for<0, BR>([&](auto rc) {
                    constexpr int rq = decltype(rc)::value;
                    constexpr int rr = sb * BR + rq;      // step within the iteration
                    const int i = it * ITER + rr;
                    const u32x4 w = ring[rr % RING];
                    // the load of step i + U goes out here, before step i's arithmetic (left to
                    // itself the scheduler bunches the loads late and the ring stops hiding them)
                    __builtin_amdgcn_sched_barrier(0);
                    ring[(rr + U) % RING] = wload(i + U);
                    __builtin_amdgcn_sched_barrier(0);
                    uint32_t pr[16];
                    const float sc = decode(i, w, pr);
                    float d[MM];
#pragma unroll
                    for (int m = 0; m < MM; ++m) d[m] = 0.0f;
#pragma unroll
                    for (int bi = 0; bi < 16; ++bi)
#pragma unroll
                        for (int m = 0; m < MM; ++m) d[m] = dot2(pr[bi], x[m][bi], d[m]);
#pragma unroll
                    for (int m = 0; m < MM; ++m) p[rq][m] = sc * d[m];
                });
                float rs[MM];
                reduce_rows<BR, MM>(p, rs, lane);
                const int i = it * ITER + sb * BR + gsel;
                if (holder && i < nsteps && lrow(i) < nrows) {
#pragma unroll
                    for (int m = 0; m < MM; ++m) part[(kw * a.R + lrow(i)) * MM + m] = rs[m];
                }
            });
        }
    } else {
        const bool holder = (lane & 12) == 12;
        const int htok = 2 * (lane >> 5) + ((lane >> 4) & 1);   // token (within a group) held
        for (int it = 0; it < nit; ++it) {
            static_for<0, ITER>([&](auto rc) {
                constexpr int rr = decltype(rc)::value;
                const int i = it * ITER + rr;
                const u32x4 w = ring[rr % RING];
                __builtin_amdgcn_sched_barrier(0);
                ring[(rr + U) % RING] = wload(i + U);
                __builtin_amdgcn_sched_barrier(0);
                uint32_t pr[16];
                const float sc = decode(i, w, pr);
#pragma unroll
                for (int q = 0; q < NX; ++q) {
                    f32x4 cq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int t = 0; t < 8; ++t) cq = mfma4x4(x[q][2 * t], x[q][2 * t + 1], pr[2 * t], pr[2 * t + 1], cq);
                    const float v = reduce_blocks4(sc * cq);
                    if constexpr (DEFER) {
                        if (holder & (i < nsteps)) part[(kw * a.R + lrow(i)) * MM + 4 * q + htok] = v;
                    } else {
                        if (holder) part[(wave * BROWS + ROWS_STEP * rr + jrow) * MM + 4 * q + htok] = v;
                    }
                }
            });
            if constexpr (DEFER) continue;
            // the KW waves of each row meet here: batch `it` of every stream, 8 lanes per sum (lane
            // q adds waves q, q + 8, ..., then a prefix sum over the 8 ends in lane 7)
            lds_barrier();
            const int nsum = a.S * BROWS * MM;
            for (int i0 = 0; i0 < nsum * 8; i0 += nthr) {     // uniform trip count (DPP below)
                const int e = (i0 + tid) >> 3, q = tid & 7;
                const int ss = e / (BROWS * MM), rem = e - ss * (BROWS * MM);
                const int br = rem / MM, m = rem - br * MM;
                float t = 0.0f;
                if (e < nsum)
                    for (int k = q; k < a.KW; k += 8) t += part[((ss * a.KW + k) * BROWS + br) * MM + m];
                t += dpp<0x111>(t);
                t += dpp<0x112>(t);
                t += dpp<0x114>(t);
                const int st = it * ITER + br / ROWS_STEP;          // the row's step in its stream
                const int row = ss * a.RS + ROWS_STEP * st + (br % ROWS_STEP);
                if (e < nsum && q == 7 && st < nsteps && row < nrows) res[row * MM + m] = t;
            }
            lds_barrier();
        }
    }
    __syncthreads();

    // ---- rows' sums (over the KW waves), plus (s T) L2, stored bf16: 8 lanes per output, lane q
    //      of the 8 taking every 8th term of the r-long dot product ----
    const int jn = a.r >> 3;
    for (int i0 = 0; i0 < a.R * MM * 8; i0 += nthr) {     // uniform trip count (DPP below)
        const int idx = (i0 + tid) >> 3, q = tid & 7;
        const int m = idx / a.R, rl = idx - m * a.R;
        const bool ok = idx < a.R * MM && m < a.M && rl < nrows;
        float lo = 0.0f;
        if (ok) {
            for (int jj = 0; jj < jn; ++jj) {
                const int j = 8 * jj + q;
                lo = __builtin_fmaf(sTs[m * a.r + j], bf16_to_f32(l2s[j * a.R + rl]), lo);
            }
            if constexpr (MF && !DEFER) {
                if (q == 0) lo += res[rl * MM + m];
            } else if (q < a.KW) {
                for (int k = q; k < a.KW; k += 8) lo += part[(k * a.R + rl) * MM + m];
            }
        }
        lo += dpp<0x111>(lo);
        lo += dpp<0x112>(lo);
        lo += dpp<0x114>(lo);
        if (ok && q == 7) a.Y[m * a.N + n0 + rl] = (uint16_t)f32_to_bf16(lo);
    }
}

struct RowsPlan {
    int KW, S, R, RS, grid;
};

// The row kernel serves M = 1 with dot products (mm = 1) and M = 2..8 with the 4 x 4 MFMA layout
// (mm = 4 or 8 tokens).  Beyond 8 tokens the 4 x 4 x 4 MFMAs (a fraction of the rate of the large
// shapes) bound it: 16 tokens took 70 us against 63 us for the 16 x 16 x 32 GEMV.
int rows_mm(int64_t M) { return M == 1 ? 1 : (M <= 4 ? 4 : 8); }

RowsPlan rows_plan(int64_t N, int64_t K, int mm) {
    RowsPlan p;
    const bool mf = mm > 1;
    const int64_t nchunk = K >> 5, nblk = K >> 6;
    p.KW = (int)((nchunk + (mf ? 15 : 63)) / (mf ? 16 : 64));
    p.S = p.KW <= MAX_WAVES ? MAX_WAVES / p.KW : 0;
    // one workgroup per CU when the rows allow it; each stream a whole number of 4-row groups
    const int64_t unit = mf ? 8 * (p.S > 0 ? p.S : 1) : 8;
    int64_t R = (N + 255) / 256;
    R = (R + unit - 1) / unit * unit;
    int64_t cap = R_MAX;
    if (cap > C2_CAP / nblk) cap = C2_CAP / nblk;
    if (!mf && cap > PART_CAP / p.KW) cap = PART_CAP / p.KW;
    if (mm == 4 && cap > CSUM_CAP / (4 * p.KW)) cap = CSUM_CAP / (4 * p.KW);   // all rows' partials
    if (mm == 8 && cap > (CSUM_CAP - RES_OFF) / mm) cap = (CSUM_CAP - RES_OFF) / mm;
    cap = cap / unit * unit;
    if (R > cap) R = cap;
    p.R = (int)R;
    p.RS = p.S > 0 ? (int)(R / p.S) : 0;
    if (!mf && p.S > 0) p.RS = (int)((R + p.S - 1) / p.S);
    p.grid = R > 0 ? (int)((N + R - 1) / R) : 0;
    return p;
}

int mm_of(int64_t M) { return M == 1 ? 1 : (M == 2 ? 2 : 4); }   // tokens of the T kernel
int t_slices(int64_t K) { return (int)((K + T_ROWS - 1) / T_ROWS); }
// T's partials: the slice kernel below for M <= 4, the split-K skinny product above
int t_parts(int64_t M, int64_t K, int32_t r) {
    if (M <= 4) return t_slices(K);
    return choose_split(((M + 63) / 64) * ((r + 63) / 64), (K + 63) / 64);
}

template <int MM>
hipError_t launch_t(const TArgs &t, int nkc, hipStream_t stream) {
    hipLaunchKernelGGL(gemv_t_kernel<MM>, dim3(nkc), dim3(T_THREADS), 0, stream, t);
    return hipGetLastError();
}

hipError_t launch_t_parts(const uint16_t *X, const uint16_t *L1, int32_t r, int64_t M, int64_t K, float *Tp,
                          hipStream_t stream) {
    const int nkc = t_parts(M, K, r);
    if (M > 4) return launch_skinny_nt(X, L1, /*b_rows_k=*/true, Tp, M, r, K, nkc, stream);
    TArgs t;
    t.X = X; t.L1 = L1; t.Tp = Tp; t.M = M; t.K = K; t.r = r;
    switch (mm_of(M)) {
        case 1: return launch_t<1>(t, nkc, stream);
        case 2: return launch_t<2>(t, nkc, stream);
        default: return launch_t<4>(t, nkc, stream);
    }
}

template <int MM, bool I8>
void launch_rows_fmt(const RowsArgs &a, int threads, int grid, hipStream_t stream) {
    if constexpr (MM == 1)
        hipLaunchKernelGGL((gemv_rows_kernel<1, 4, 2, MAX_WAVES, false, I8>), dim3(grid), dim3(threads), 0, stream, a);
    else
        hipLaunchKernelGGL((gemv_rows_kernel<MM, 4, 2, MAX_WAVES, true, I8>), dim3(grid), dim3(threads), 0, stream, a);
}

template <int MM>
hipError_t launch_rows(const RowsArgs &a, int threads, int grid, hipStream_t stream) {
    timing_before(stream, 2);
    if (a.dq_int8)
        launch_rows_fmt<MM, true>(a, threads, grid, stream);
    else
        launch_rows_fmt<MM, false>(a, threads, grid, stream);
    const hipError_t err = hipGetLastError();
    timing_after(stream);
    return err;
}

}  // namespace

GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K, int32_t r) {
    GemvPlan p;
    (void)N;
    p.nseg = 1;
    p.nkc = t_parts(M, K, r);
    p.yp_floats = 0;
    p.tp_floats = (size_t)p.nkc * M * r;
    return p;
}

hipError_t launch_gemv_T(const uint16_t *X, const uint16_t *L1, int32_t r, int64_t M, int64_t K, float *Tp,
                        uint16_t *T, hipStream_t stream) {
    if (M < 1 || M > 8 || r < 8 || r > R_MAX_LORA || r % 8) return hipErrorInvalidValue;
    hipError_t err = launch_t_parts(X, L1, r, M, K, Tp, stream);
    if (err != hipSuccess) return err;
    const int E = (int)M * r;
    hipLaunchKernelGGL(gemv_tsum_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, Tp, t_parts(M, K, r), E, T);
    return hipGetLastError();
}

bool gemv_fits(int64_t M, int64_t N, int64_t K, int32_t r) {
    if (M < 1 || M > 8 || r < 8 || r > R_MAX_LORA || r % 8 || N % 8 || K % 64) return false;
    const int mm = rows_mm(M);
    const RowsPlan p = rows_plan(N, K, mm);
    const int64_t nch = (t_parts(M, K, r) + 7) / 8;
    if (p.S < 1 || p.R < 8 || p.R > R_MAX || p.R * (K >> 6) > C2_CAP || nch * mm * r > CSUM_CAP) return false;
    if (mm == 1) return (int64_t)p.KW * p.R <= PART_CAP;
    if (mm == 4) return (int64_t)p.KW * p.R * 4 <= CSUM_CAP;   // every row's wave partials
    // cross-wave partials of one batch, and the row sums
    return (int64_t)p.S * p.KW * 16 * mm <= RES_OFF && (int64_t)p.R * mm <= CSUM_CAP - RES_OFF;   // 16 rows a batch
}

hipError_t launch_gemv_fwd(const WeightView &w, const uint16_t *X, const uint16_t *L1, const uint16_t *L2,
                           float scale, int32_t r, int64_t M, uint16_t *Y, uint16_t *T_out, float *Yp,
                           float *Tp, hipStream_t stream) {
    (void)Yp;
    if (!gemv_fits(M, w.rows, w.cols, r)) return hipErrorNotSupported;
    const int mm = rows_mm(M);
    const GemvPlan g = gemv_plan(M, w.rows, w.cols, r);
    const RowsPlan p = rows_plan(w.rows, w.cols, mm);
    const int threads = p.S * p.KW * 64;
    hipError_t err = launch_t_parts(X, L1, r, M, w.cols, Tp, stream);
    if (err != hipSuccess) return err;
    RowsArgs a;
    a.X = X;
    a.packed = w.packed; a.c2 = w.c2; a.c1 = w.c1; a.mean = w.mean; a.dq_int8 = w.dq_int8;
    a.L2 = L2; a.Tp = Tp; a.Y = Y; a.T_out = T_out;
    a.M = M; a.N = w.rows; a.K = w.cols;
    a.r = r; a.nkc = g.nkc; a.KW = p.KW; a.S = p.S; a.RS = p.RS; a.R = p.R;
    a.scale = scale;
    for (int j = 0; j < 16; ++j) a.cb.v[j] = w.cb[j];
    switch (mm) {
        case 1: return launch_rows<1>(a, threads, p.grid, stream);
        case 4: return launch_rows<4>(a, threads, p.grid, stream);
        default: return launch_rows<8>(a, threads, p.grid, stream);
    }
}

}  // namespace nf4k
