// Fused double-dequantize + bf16 MFMA GEMM for the backward of the QLoRA linear layer below
// 1024 tokens (gfx950):
//   dX = dY . deq(W) + dT . L1^T       reduction over N (the W rows), output cols = W cols
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (6) (double dequantization to BF16) and the backward description (gradient to
// X through the BF16 weight only); section 4 eq. (3) (scalar s, inside dT).
//
// The LoRA product is appended as extra reduction steps: A' = [dY | dT], B' = [deq(W) ; L1^T],
// so it costs r/64 more steps of the same MFMA loop and no extra pass over the activations.
//
// Block tile 256 x 256 outputs, reduction step 64 (one quantization block per W row), 4 waves
// in 2 x 2, each 128 x 128 with v_mfma_f32_32x32x16_bf16 (16 tiles, 256 fp32 accumulators).
// Up to 64 tokens the tile is 64 x 256 (4 waves side by side, each 64 x 64): a 256-row tile
// would spend three quarters or more of its MFMA work on padding rows, while the weight's
// decode, the same per step either way, then bounds the step.
//
// A (activations, reduction-contiguous) goes straight from global memory to LDS with
// buffer_load ... lds (no registers, no ds_write), 32 KB per stage, 16-byte chunks XOR-swizzled
// by (row / 2) so the 16-byte fragment reads are bank-conflict free.
//
// B (the frozen weight) is dequantized by all 256 threads into LDS in natural row layout
// [W row][W col], one thread per (row, 64-column block), i.e. one quantization block:
//   a' = fma(e4m3(c2), c1, mean);  lut[j] = bf16(cb[j] * a') for the 16 codes
// The 16-entry bf16 table lives in 8 registers as byte planes, and each packed dword (8 codes)
// is expanded with v_perm_b32 byte selects (no LDS lookups, no per-element multiply).  The W rows
// are the reduction, so fragments come from ds_read_b64_tr_b16, which transposes 4 x 16 bf16
// blocks across each 16-lane group.
// Register stages of W are fetched two steps ahead; the dequantization of step s+1 is spread
// over the four MFMA sub-steps of step s.
//
// Few output tiles (few tokens): the reduction is split over up to 16 workgroups per tile, each
// writing a float32 partial tile that a fixed-order reduction sums (and adds to dX when
// accumulating).

#include "common.h"
#include "dqtile.h"
#include "launch.h"

namespace nf4k {

namespace {

constexpr int TN = 256;          // output cols per block tile
constexpr int TK = 64;           // reduction per step (= one quantization block)
constexpr int NTHREADS = 256;
// s_waitcnt immediate: vmcnt <= 4 (the W loads issued after the A loads may stay in flight),
// expcnt unchecked, lgkmcnt = 0.  gfx9 layout: vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14
constexpr int kWaitA = 4 | (7 << 4) | (0 << 8);

// B stage layouts: the main loop's dequantized W step is [red][out col] (544-byte rows); the
// LoRA extension step's L1 [K, r] is read in its natural layout, [out col][red] (144-byte rows).
// A stage is sized for both.
constexpr int ROWB_RED = (TK + 8) * 2;     // [256][64 + 8]
constexpr int ROWB_OUT = (TN + 16) * 2;    // [64][256 + 16]
constexpr int B_STAGE_BYTES = (TN * ROWB_RED > TK * ROWB_OUT) ? TN * ROWB_RED : TK * ROWB_OUT;

struct GemmArgs {
    const uint16_t *A;       // [M, Kred] bf16
    const uint8_t *packed;   // W codes [wrows, wcols/2]
    const uint8_t *c2;       // E4M3 block constants
    const float *c1;         // 256-block multipliers
    const float *mean;       // [1]
    uint32_t dq_int8;        // second-level codes are int8 (else E4M3)
    const uint16_t *Ae;      // dT [M, r] bf16 (extension A)
    const uint16_t *Be;      // L1 [Nout, r] (natural layout)
    uint16_t *C;             // [M, Nout] bf16
    int64_t M, Nout, Kred;
    int64_t wrows, wcols;
    int32_t r;
    uint32_t accumulate;
    Codebook cb;
    // split reduction (ksplit > 1): workgroup b takes tile b % tiles and steps [split per,
    // (split + 1) per) with split = b / tiles, writing float32 partials P + split M Nout
    int32_t ksplit, split_per;
    float *P;
};


// TM: output rows per block tile, 256 (waves 2 x 2) or 64 (waves 1 x 4)
template <int TM>
__global__ __launch_bounds__(NTHREADS, 1) void dqgemm_bwd_kernel(GemmArgs g) {
    constexpr int B_STAGE = B_STAGE_BYTES;
    constexpr int A_STAGE = TM * TK * 2;              // 32 or 8 KB, swizzled, unpadded
    constexpr int WN_WAVES = TM == 256 ? 2 : 4;       // waves along the output columns
    constexpr int WT_M = TM * WN_WAVES / 4;           // wave tile: WT_M x WT_N
    constexpr int WT_N = TN / WN_WAVES;
    constexpr int IM = WT_M / 32, JN = WT_N / 32;     // 32 x 32 MFMA tiles of a wave
    constexpr int QA = TM / 32;                       // A loads (1 KB each) per wave and step
    static_assert(TM == 256 || TM == 64, "block tile rows");
    // separate LDS objects, so the compiler sees that the direct-to-LDS A loads never alias the
    // B tile reads and adds no memory-counter waits of its own before them
    // each stage is its own object: a read of stage 0 provably never aliases the loads in flight
    // into stage 1 (and vice versa)
    __shared__ __align__(16) uint8_t As0[A_STAGE];
    __shared__ __align__(16) uint8_t As1[A_STAGE];
    __shared__ __align__(16) uint8_t Bs0[B_STAGE];
    __shared__ __align__(16) uint8_t Bs1[B_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
    const int wm = wave >> (WN_WAVES == 2 ? 1 : 2), wn = wave & (WN_WAVES - 1);
    const int r32 = lane & 31, hh = lane >> 5;

    const int ntm = (int)((g.M + TM - 1) / TM);
    const int ntn = (int)((g.Nout + TN - 1) / TN);
    const int ntiles = ntm * ntn;
    const int split = (int)(blockIdx.x / (uint32_t)ntiles);
    int tm, tn;
    tile_coords(ntm, ntn, (int)blockIdx.x - split * ntiles, tm, tn);
    const int64_t m0 = (int64_t)tm * TM;
    const int64_t o0 = (int64_t)tn * TN;

    // this workgroup's steps: kb .. kb + main_steps - 1; the loops below count from 0
    const int kb = split * g.split_per;
    const int main_steps = min((int)((g.Kred + TK - 1) / TK) - kb, g.split_per);
    const int ext_steps = split == g.ksplit - 1 ? (g.r + TK - 1) / TK : 0;

    const float mean = g.mean[0];

    const bool dq_i8 = g.dq_int8 != 0;
    const int64_t wblk_per_row = g.wcols >> 6;
    const int64_t wrow_bytes = g.wcols >> 1;

    // tile-relative buffer descriptors: reads past the end return zeros (no edge branches)
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + m0 * g.Kred, (g.M - m0) * g.Kred * 2);
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.packed, g.wrows * wrow_bytes);
    const __amdgpu_buffer_rsrc_t rC2 = make_rsrc(g.c2, g.wrows * wblk_per_row);
    const __amdgpu_buffer_rsrc_t rC1 = make_rsrc(g.c1, ((g.wrows * wblk_per_row + 255) >> 8) * 4);

    // ---- A: direct global -> LDS.  Each wave issues QA x 1 KB per step: instruction q writes
    // LDS rows 8u..8u+7 (u = QA*wave + q); lane l -> row 8u + l/8, physical chunk l%8, which
    // holds logical chunk (l%8) ^ ((row/2) % 8). ----
    uint32_t a_voff[QA];
    int a_col[QA];
#pragma unroll
    for (int q = 0; q < QA; ++q) {
        const int row = 8 * (QA * wave + q) + (lane >> 3);
        a_col[q] = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
        a_voff[q] = (uint32_t)((row * g.Kred + a_col[q]) * 2);
    }
    // reduction columns up to the end of this workgroup's steps
    const int kred32 = (int)min(g.Kred, (int64_t)(kb + main_steps) * TK);
    auto load_A = [&](int step, uint8_t *Ad) {
        step += kb;
        // reduction columns left from this step on; <= 0 past the last step (loads read zeros),
        // < 64 on a ragged last step (its columns past N read zeros)
        const int rem = kred32 - step * TK;
        typedef __attribute__((address_space(3))) uint8_t lds_u8;
        lds_u8 *dst = (lds_u8 *)Ad + wave * (QA * 1024);
#pragma unroll
        for (int q = 0; q < QA; ++q) {
            uint32_t off = a_voff[q] + (uint32_t)step * TK * 2;
            if (a_col[q] >= rem) off = 0xFFFFFFF0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void *)(dst + q * 1024), 16, off, 0, 0, 0);
        }
    };

    // ---- W: thread -> (W row step*64 + tid%64, 64-column block o0/64 + tid/64) ----
    const int bw_row = tid & 63;
    const int bw_blk = tid >> 6;
    struct WStage {
        u32x4 w[2];
        uint32_t c2, c1;
    };
    auto load_W = [&](int step, WStage &ws) {
        const bool live = step < main_steps;
        const int64_t n = (int64_t)(kb + step) * TK + bw_row, blk = (o0 >> 6) + bw_blk;
        const uint32_t off = (uint32_t)(n * wrow_bytes + blk * 32);
        const uint32_t b = (uint32_t)(n * wblk_per_row + blk);
        ws.w[0] = bload16(rW, live ? off : 0xFFFFFFF0u);
        ws.w[1] = bload16(rW, live ? off + 16 : 0xFFFFFFF0u);
        ws.c2 = bload1(rC2, live ? b : 0xFFFFFFF0u);
        ws.c1 = bload4(rC1, live ? (b >> 8) * 4 : 0xFFFFFFF0u);
    };
    // dequantize a W stage: part `part` (0..3) handles packed dwords 2*part, 2*part+1
    Lut lut;
    auto write_B = [&](int step, const WStage &ws, uint8_t *Bst, int part) {
        if (part == 0) {
            float a = block_scale(ws.c2, __uint_as_float(ws.c1), mean, dq_i8);
            if ((int64_t)(kb + step) * TK + bw_row >= g.wrows) a = 0.0f;   // ragged reduction
            lut = make_lut(g.cb, a);
        }
        uint8_t *Bd = Bst + bw_row * ROWB_OUT + bw_blk * 128;
#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {
            const int d = part * 2 + dd;
            const uint32_t w = ws.w[d >> 2][d & 3];
            *reinterpret_cast<u32x4 *>(Bd + d * 16) = dequant8_planar(lut, w);
        }
    };

    f32x16 acc[IM][JN];
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // ---- fragments of sub-step s (16 reduction elements): lane (r32, hh) takes elements
    // 16 s + 8 hh .. +7 of its row (A) / column (B) ----
    auto frag_A = [&](const uint8_t *Ast, int s, int i) -> bf16x8 {
        const int row = wm * WT_M + i * 32 + r32;
        const int c = (2 * s + hh) ^ ((row >> 1) & 7);
        return *reinterpret_cast<const bf16x8 *>(Ast + row * 128 + c * 16);
    };
    // B fragment of the extension step, from its [out col][red] tile (row reads)
    auto frag_rowread = [&](const uint8_t *Bst, int s, int j) -> bf16x8 {
        const int row = wn * WT_N + j * 32 + r32;
        return *reinterpret_cast<const bf16x8 *>(Bst + row * ROWB_RED + (s * 16 + hh * 8) * 2);
    };
    // B fragment of a main-loop step, from its [red][out col] tile: 16-lane group (hh, half):
    // lane i of the group reads row 16s + 8hh + i/4 (+4), columns col0 + 4(i%4) .. +3; after
    // the transpose, lane i holds column col0 + i.
    auto frag_B = [&](const uint8_t *Bst, int s, int j) -> bf16x8 {
        const int i16 = lane & 15, half = (lane >> 4) & 1;
        const int col0 = wn * WT_N + j * 32 + half * 16;
        const int rowb = s * 16 + hh * 8 + (i16 >> 2);
        const uint8_t *base = Bst + (col0 + 4 * (i16 & 3)) * 2;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + rowb * ROWB_OUT));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + (rowb + 4) * ROWB_OUT));
        const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    };
    struct Frags {
        bf16x8 a[IM], b[JN];
    };
    auto load_frags = [&](const uint8_t *Ast, const uint8_t *Bst, int s, Frags &f) {
#pragma unroll
        for (int i = 0; i < IM; ++i) f.a[i] = frag_A(Ast, s, i);
#pragma unroll
        for (int j = 0; j < JN; ++j) f.b[j] = frag_B(Bst, s, j);
    };
    auto mma = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < IM; ++i)
#pragma unroll
            for (int j = 0; j < JN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    };
    auto mfma_sub = [&](const uint8_t *Ast, const uint8_t *Bst, int s) {
        Frags f;
        load_frags(Ast, Bst, s, f);
        mma(f);
    };

    // Interleave one sub-step: its 16 MFMAs, the fragment reads of the next sub-step, a quarter
    // of the next step's dequantization (VALU + 2 LDS writes) and the direct-to-LDS A loads.
    // MFMA (32 cycles each) and VALU issue from the same wave co-execute when interleaved.
    auto interleave = [&]() {
        if constexpr (TM == 256) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);      // 5 VALU
                if (k < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
                if (k == 9 || k == 13) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
                if (k == 2 || k == 6 || k == 10) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM
            }
        } else {
            // 4 MFMAs per sub-step: the same quarter of the decode spread over them
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);     // 20 VALU
                if (k < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 DS reads
                if (k == 1 || k == 3) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
                if (k == 0 || k == 2) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM
            }
        }
    };

    // one step: compute stage (Ac, Bc), fill stage Bn with the dequantized W registers `ws` of
    // step `wstep`; fragments run one sub-step ahead
    auto half_step = [&](const uint8_t *Ac, const uint8_t *Bc, uint8_t *Bn, int wstep, const WStage &ws) {
        Frags f0, f1;
        load_frags(Ac, Bc, 0, f0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            Frags &cur = (s & 1) ? f1 : f0;
            Frags &nxt = (s & 1) ? f0 : f1;
            if (s < 3) load_frags(Ac, Bc, s + 1, nxt);
            mma(cur);
            write_B(wstep, ws, Bn, s);
            interleave();
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- main loop ----
    // LDS stages alternate per step.  A for step+1 is loaded straight into LDS at the start of
    // step; W for step+2 into registers at the start of step, and the W registers of step+1 are
    // dequantized into the other B stage in four parts interleaved with the MFMA sub-steps.
    WStage R0, R1;
    load_A(0, As0);
    load_W(0, R0);
#pragma unroll
    for (int part = 0; part < 4; ++part) write_B(0, R0, Bs0, part);
    load_W(1, R1);
    __builtin_amdgcn_s_waitcnt(0);     // A of step 0 landed (all counters drained)
    __syncthreads();
    int step = 0;
    for (; step + 1 < main_steps; step += 2) {
        load_A(step + 1, As1);
        load_W(step + 2, R0);
        half_step(As0, Bs0, Bs1, step + 1, R1);
        // A of step+1 (issued before the 4 W loads of step+2) has landed; LDS writes done
        __builtin_amdgcn_s_waitcnt(kWaitA);
        __syncthreads();
        load_A(step + 2, As0);
        load_W(step + 3, R1);
        half_step(As1, Bs1, Bs0, step + 2, R0);   // zeros past the end; read again only if live
        __builtin_amdgcn_s_waitcnt(kWaitA);
        __syncthreads();
    }
    if (step < main_steps) {   // odd number of steps: the last one sits in stage 0
#pragma unroll
        for (int s = 0; s < 4; ++s) mfma_sub(As0, Bs0, s);
        __syncthreads();
    }

    // ---- LoRA extension: [dY | dT] . [deq(W) ; L1^T], r/64 more steps (zero padded past r) ----
    // L1 [K, r]: tile [out col][j] (144-byte rows, columns at their planar positions), row reads
    if (ext_steps > 0) {
        const __amdgpu_buffer_rsrc_t rAe = make_rsrc(g.Ae + m0 * g.r, (g.M - m0) * (int64_t)g.r * 2);
        const __amdgpu_buffer_rsrc_t rBe = make_rsrc(g.Be + o0 * g.r, (g.Nout - o0) * (int64_t)g.r * 2);
        for (int e = 0; e < ext_steps; ++e) {
            const int st = (main_steps + e) & 1;
            uint8_t *Ast = st ? As1 : As0;
            uint8_t *Bst = st ? Bs1 : Bs0;
            const int j0 = e * TK;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                // A (rows < TM): row (tid/8) + 32 q, reduction chunk tid % 8 (columns past r read
                // zeros); B: output column o0 + row, the same reduction chunk
                const int row = (tid >> 3) + 32 * q, chunk = tid & 7;
                const int jj = j0 + chunk * 8;
                if (q < TM / 32) {
                    const uint32_t offa = jj < g.r ? (uint32_t)((row * (int64_t)g.r + jj) * 2) : 0xFFFFFFF0u;
                    const u32x4 va = bload16(rAe, offa);
                    *reinterpret_cast<u32x4 *>(Ast + row * 128 + (chunk ^ ((row >> 1) & 7)) * 16) = va;
                }
                const uint32_t off = jj < g.r ? (uint32_t)((row * (int64_t)g.r + jj) * 2) : 0xFFFFFFF0u;
                const u32x4 vb = bload16(rBe, off);
                const int pos = (row & ~7) | ((row & 1) << 2) | ((row & 7) >> 1);
                *reinterpret_cast<u32x4 *>(Bst + pos * ROWB_RED + chunk * 16) = vb;
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                Frags f;
#pragma unroll
                for (int i = 0; i < IM; ++i) f.a[i] = frag_A(Ast, s, i);
#pragma unroll
                for (int j = 0; j < JN; ++j) f.b[j] = frag_rowread(Bst, s, j);
                mma(f);
            }
            __syncthreads();
        }
    }

    // ---- epilogue: fp32 -> bf16 ----
    // Lane (r32, hh) of tile (i, j) holds column j*32 + r32 (permuted back from the planar
    // dequant order) and rows i*32 + 8*(v/4) + 4*hh + v%4.  Stores go through a buffer
    // descriptor: rows past M fall outside it, row offsets are scalars, the column offset is a
    // per-lane constant, so no per-element address arithmetic remains.
    const int colw = (r32 & ~7) | planar_col(r32 & 7);
    if (g.ksplit > 1) {
        // float32 partial tile (rows past M fall outside the descriptor)
        const __amdgpu_buffer_rsrc_t rP = make_rsrc(g.P + (int64_t)split * g.M * g.Nout + m0 * g.Nout,
                                                    (g.M - m0) * g.Nout * 4);
        const uint32_t prow = (uint32_t)(g.Nout * 4);
        const uint32_t poff = (uint32_t)((wm * WT_M + hh * 4) * prow) + (uint32_t)((o0 + wn * WT_N + colw) * 4);
#pragma unroll
        for (int j = 0; j < JN; ++j) {
            if (o0 + wn * WT_N + j * 32 + colw >= g.Nout) continue;
#pragma unroll
            for (int i = 0; i < IM; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const uint32_t rows = (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3));
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]), rP, poff + j * 128,
                                                          rows * prow, 0);
                }
            }
        }
    } else if (!g.accumulate) {
        const __amdgpu_buffer_rsrc_t rC = make_rsrc(g.C + m0 * g.Nout, (g.M - m0) * g.Nout * 2);
        const uint32_t row_bytes = (uint32_t)(g.Nout * 2);
        const uint32_t lane_off = (uint32_t)((wm * WT_M + hh * 4) * row_bytes) +
                                  (uint32_t)((o0 + wn * WT_N + colw) * 2);
#pragma unroll
        for (int j = 0; j < JN; ++j) {
            if (o0 + wn * WT_N + j * 32 + colw >= g.Nout) continue;
#pragma unroll
            for (int i = 0; i < IM; ++i) {
#pragma unroll
                for (int v = 0; v < 16; v += 2) {
                    const uint32_t rows = (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3));
                    const uint32_t pk = pack_bf16x2(acc[i][j][v], acc[i][j][v + 1]);
                    const uint32_t soff = rows * row_bytes;
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)pk, rC, lane_off + j * 64, soff, 0);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pk >> 16), rC, lane_off + j * 64,
                                                          soff + row_bytes, 0);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < IM; ++i) {
#pragma unroll
            for (int j = 0; j < JN; ++j) {
                const int64_t col = o0 + wn * WT_N + j * 32 + colw;
                if (col >= g.Nout) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = m0 + wm * WT_M + i * 32 + (v >> 2) * 8 + hh * 4 + (v & 3);
                    if (row < g.M) {
                        uint16_t *p = g.C + row * g.Nout + col;
                        *p = (uint16_t)f32_to_bf16(acc[i][j][v] + bf16_to_f32(*p));
                    }
                }
            }
        }
    }
}

// up to this many tokens the 64-row block tile
constexpr int64_t kSmallTileM = 64;

hipError_t launch_impl(GemmArgs &a, const SplitK &sk, hipStream_t stream) {
    const int TM = a.M <= kSmallTileM ? 64 : 256;
    const int ntm = (int)((a.M + TM - 1) / TM);
    const int ntn = (int)((a.Nout + TN - 1) / TN);
    const int64_t steps = (a.Kred + TK - 1) / TK;
    a.ksplit = sk.ksplit > 1 ? sk.ksplit : 1;
    a.split_per = (int32_t)(a.ksplit > 1 ? sk.per : steps);
    a.P = sk.P;
    if (a.ksplit > 1 && (!sk.P || (int64_t)(a.ksplit - 1) * sk.per >= steps || (int64_t)a.ksplit * sk.per < steps))
        return hipErrorInvalidValue;
    timing_before(stream, 1);
    if (TM == 64)
        hipLaunchKernelGGL(dqgemm_bwd_kernel<64>, dim3(ntm * ntn * a.ksplit), dim3(NTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL(dqgemm_bwd_kernel<256>, dim3(ntm * ntn * a.ksplit), dim3(NTHREADS), 0, stream, a);
    hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace

hipError_t launch_dqgemm_bwd(const WeightView &w, const uint16_t *dY, const uint16_t *dT,
                             const uint16_t *L1, int32_t r, int64_t M, uint16_t *dX,
                             bool accumulate, const SplitK &sk, hipStream_t stream) {
    GemmArgs a;
    a.A = dY;
    a.packed = w.packed; a.c2 = w.c2; a.c1 = w.c1; a.mean = w.mean; a.dq_int8 = w.dq_int8;
    a.Ae = dT; a.Be = L1; a.C = dX;
    a.M = M; a.Nout = w.cols; a.Kred = w.rows;
    a.wrows = w.rows; a.wcols = w.cols;
    a.r = r; a.accumulate = accumulate ? 1u : 0u;
    for (int j = 0; j < 16; ++j) a.cb.v[j] = w.cb[j];
    return launch_impl(a, sk, stream);
}

}  // namespace nf4k
