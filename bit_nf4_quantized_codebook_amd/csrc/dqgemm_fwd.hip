// Forward fused double-dequantize + bf16 MFMA GEMM of the QLoRA linear layer (gfx950):
//   Y = X . deq(W)^T + (sT) . L2          X [M, K], W [N, K] NF4, sT [M, r], L2 [r, N]
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (5) (forward) and eq. (6) (double dequantization to BF16); section 4 eq. (3)
// (the LoRA scalar s).
//
// Block tile 256 x 256 outputs, reduction step 64 (one quantization block of each W row), four
// waves side by side along N: wave w owns output columns 64w .. 64w+63 for all 256 rows, as
// 8 x 2 tiles of v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators).
//
// The weight never passes through LDS.  In the forward the W rows are the output columns, so the
// 8 reduction elements that an MFMA lane holds for its column are 8 consecutive codes of one W
// row: 4 packed bytes.  Each lane loads the 16 packed bytes it needs per step straight into
// registers and expands them with the per-block bf16 table (v_perm_b32 byte selects) into the
// B operand.  To make that one 16-byte load, the 64 reduction elements of a step are visited in
// a fixed order that both operands share: lane half hh takes elements 32 hh .. 32 hh + 31 and
// sub-step s the 8 of them at 32 hh + 8 s (the sum over a step is order-free).
//
// Only X goes through LDS, straight from global memory (buffer_load ... lds, no registers), in a
// ring of four 32 KB stages: loads run three steps ahead, and since a stage is complete one step
// before it is read, the fragments of a step's first sub-step are read before the barrier that
// ends the previous step, so the MFMA chain resumes right after it.
//
// The LoRA product is appended as r/64 more reduction steps: A' = [X | sT], B' = [deq(W) ; L2].
// L2 [r, N] is read in its natural layout into LDS and its fragments come from transposing
// reads (ds_read_b64_tr_b16).
//
// Few output tiles (few tokens: one 256-row tile up to 256 of them): the reduction is split over
// up to 16 workgroups per tile (a multiple of 4 steps each, so the grouped codes stay aligned),
// each writing a float32 partial tile that a fixed-order reduction sums; the weight is then
// still decoded once per tile row, by 16 times as many workgroups.

#include "common.h"
#include "dqtile.h"
#include "launch.h"

namespace nf4k {

namespace {

constexpr int TM = 256;
constexpr int TN = 256;
constexpr int TK = 64;
constexpr int NTHREADS = 256;
constexpr int A_STAGE = TM * TK * 2;        // 32 KB, 16-byte chunks XOR-swizzled by (row / 2)
constexpr int EXT_ROWB = (TN / 2 + 16) * 2; // LoRA B tile: two halves of [64 j][128 n + 16]
// VMEM instructions each wave issues per step: 8 direct-to-LDS X loads, then per W row (2) the
// 16 packed bytes and, unless grouped, the E4M3 code and the 256-block multiplier.  Grouped
// (K % 256 == 0): a row's codes of 4 consecutive steps are one aligned dword and share one
// multiplier, loaded once per 4 steps (4 more loads in the second step of each group).
constexpr int vmem_per_step(bool grouped, int phase) {
    return grouped ? 8 + 2 + (phase == 1 ? 4 : 0) : 8 + 2 * 3;
}
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | ((n >> 4) << 14); }

struct FwdArgs {
    const uint16_t *X;
    const uint8_t *packed;   // [N, K/2]
    const uint8_t *c2;       // [N*K/64]
    const float *c1;         // [ceil(N*K/64 / 256)]
    const float *mean;       // [1]
    uint32_t dq_int8;        // second-level codes are int8 (else E4M3)
    const uint16_t *sT;      // [M, r]
    const uint16_t *L2;      // [r, N]
    uint16_t *Y;             // [M, N]
    int64_t M, N, K;
    int32_t r;
    Codebook cb;
    // split reduction (ksplit > 1): workgroup b takes tile b % tiles and steps [split per,
    // (split + 1) per) with split = b / tiles, writing float32 partials P + split M N ([M, N])
    int32_t ksplit, split_per;
    float *P;
};

// packed bytes (and, unless grouped, block code and multiplier) of the two W rows of a lane at
// one step; GRegs: codes of 4 steps and their multiplier (grouped)
struct WRegs {
    u32x4 w[2];
    uint32_t c2[2], c1[2];
};
struct GRegs {
    uint32_t c2w[2], c1[2];
};

template <bool GROUPED>
__global__ __launch_bounds__(NTHREADS, 1) void dqgemm_fwd_kernel(FwdArgs g) {
    // one LDS object per stage, so the compiler can tell that a fragment read of one stage never
    // aliases the direct-to-LDS loads in flight into another and adds no waits of its own
    __shared__ __align__(16) uint8_t As0[A_STAGE];
    __shared__ __align__(16) uint8_t As1[A_STAGE];
    __shared__ __align__(16) uint8_t As2[A_STAGE];
    __shared__ __align__(16) uint8_t As3[A_STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r32 = lane & 31, hh = lane >> 5;

    const int ntm = (int)((g.M + TM - 1) / TM);
    const int ntn = (int)((g.N + TN - 1) / TN);
    const int ntiles = ntm * ntn;
    const int split = (int)(blockIdx.x / (uint32_t)ntiles);
    int tm, tn;
    tile_coords(ntm, ntn, (int)blockIdx.x - split * ntiles, tm, tn);
    const int64_t m0 = (int64_t)tm * TM;
    const int64_t n0 = (int64_t)tn * TN;

    // this workgroup's steps: kbeg .. kend - 1 (kbeg a multiple of 4); the loops below count
    // from 0, the loads add kbeg
    const int kbeg = split * g.split_per;
    const int kend = min((int)(g.K / TK), kbeg + g.split_per);
    const int main_steps = kend - kbeg;
    const int ext_steps = split == g.ksplit - 1 ? (g.r + TK - 1) / TK : 0;
    const float mean = g.mean[0];
    const bool dq_i8 = g.dq_int8 != 0;
    const int64_t nblk_row = g.K >> 6;
    const int64_t row_bytes_w = g.K >> 1;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.X + m0 * g.K, (g.M - m0) * g.K * 2);
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.packed, g.N * row_bytes_w);
    const __amdgpu_buffer_rsrc_t rC2 = make_rsrc(g.c2, g.N * nblk_row);
    const __amdgpu_buffer_rsrc_t rC1 = make_rsrc(g.c1, ((g.N * nblk_row + 255) >> 8) * 4);

    // ---- X: instruction q of wave w writes stage rows 8u .. 8u+7 (u = 8w + q); lane l takes
    // row 8u + l/8 and physical chunk l%8, which holds logical chunk (l%8) ^ ((row/2) % 8).
    // Since (row/2) % 8 = (4q + l/16) % 8, the lane's column depends only on the parity of q:
    // two per-lane offsets, the rest (q, step) goes into the scalar offset. ----
    uint32_t a_voff[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = 8 * (8 * wave + q) + (lane >> 3);
        const int col = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
        a_voff[q] = (uint32_t)(((lane >> 3) * g.K + col) * 2);
    }
    const uint32_t a_wave_off = (uint32_t)(64 * wave * g.K * 2);
    const int last = kend - 1;   // absolute
    // The main loop runs a multiple of 4 steps.  X loads of the padding steps (and of the
    // prefetches past the end) get an offset beyond the buffer, so they land as zeros and the
    // padding steps add nothing; W loads past the end re-read the last block (in bounds, finite).
    // Both without a branch: the out-of-range mask is a uniform bit OR-ed into the lane offset.
    auto load_A = [&](int step, uint8_t *Ad) {
        typedef __attribute__((address_space(3))) uint8_t lds_u8;
        lds_u8 *dst = (lds_u8 *)Ad + wave * 8192;
        // the whole offset sits in the lane offset (scalar offset 0), so rows past M are out of
        // range for the descriptor's bound check
        const uint32_t oob = step < main_steps ? 0u : 0x80000000u;
        const uint32_t base = a_wave_off + (uint32_t)min(kbeg + step, last) * (TK * 2);
        const uint32_t v0 = (a_voff[0] + base) | oob, v1 = (a_voff[1] + base) | oob;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t v = ((q & 1) ? v1 : v0) + (uint32_t)(8 * q) * (uint32_t)(g.K * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void *)(dst + q * 1024), 16, v, 0, 0, 0);
        }
    };

    // ---- W: lane (r32, hh) holds W rows n0 + 64 wave + 32 j + r32 (j = 0, 1); per step the 16
    // packed bytes of reduction elements 32 hh .. 32 hh + 31 of the step's block ----
    uint32_t w_voff[2], b_idx[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t n = n0 + 64 * wave + 32 * j + r32;
        w_voff[j] = (uint32_t)(n * row_bytes_w + hh * 16);
        b_idx[j] = (uint32_t)(n * nblk_row);
    }
    auto load_W = [&](int step, WRegs &R) {
        const uint32_t st = (uint32_t)min(kbeg + step, last);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            R.w[j] = __builtin_amdgcn_raw_buffer_load_b128(rW, w_voff[j], st * 32, 0);
            if (!GROUPED) {
                R.c2[j] = __builtin_amdgcn_raw_buffer_load_b8(rC2, b_idx[j], st, 0);
                R.c1[j] = bload4(rC1, ((b_idx[j] + st) >> 8) * 4);
            }
        }
    };
    // grouped: codes of steps 4 grp .. 4 grp + 3 (b_idx is a multiple of 4, so the dword is
    // aligned and the 4 blocks never straddle a 256-block boundary)
    auto load_G = [&](int grp, GRegs &G) {
        const uint32_t st = (uint32_t)min(kbeg + 4 * grp, last & ~3);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            G.c2w[j] = __builtin_amdgcn_raw_buffer_load_b32(rC2, b_idx[j], st, 0);
            G.c1[j] = bload4(rC1, ((b_idx[j] + st) >> 8) * 4);
        }
    };
    // tables of step u (phase u % 4 when grouped)
    auto make_luts = [&](const WRegs &R, const GRegs &G, int phase, Lut *L) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t code = GROUPED ? (G.c2w[j] >> (8 * phase)) & 0xFFu : R.c2[j];
            const uint32_t mult = GROUPED ? G.c1[j] : R.c1[j];
            L[j] = make_lut(g.cb, block_scale(code, __uint_as_float(mult), mean, dq_i8));
        }
    };
    auto dequant_B = [&](const WRegs &R, const Lut *L, int s, bf16x8 *B) {
#pragma unroll
        for (int j = 0; j < 2; ++j) B[j] = __builtin_bit_cast(bf16x8, dequant8(L[j], R.w[j][s]));
    };
    // A fragment (i, s): row 32 i + r32, reduction elements 32 hh + 8 s .. +7 (logical chunk
    // 4 hh + s); (row/2) % 8 = (r32/2) % 8 for every i
    uint32_t lds_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) lds_off[s] = (uint32_t)(r32 * 128 + (((4 * hh + s) ^ ((r32 >> 1) & 7)) * 16));
    auto read_A1 = [&](const uint8_t *Ast, int s, int i) -> bf16x8 {
        return *reinterpret_cast<const bf16x8 *>(Ast + lds_off[s] + i * 4096);
    };

    f32x16 acc[8][2];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // One sub-step: the 16 MFMAs of fragments (A, Bc); each A fragment is reloaded with the
    // next sub-step's (stage An, sub-step sn) right after its two MFMAs have read it.
    bf16x8 A[8];
    auto sub_step = [&](const bf16x8 *Bc, const uint8_t *An, int sn) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[i], Bc[j], acc[i][j], 0, 0, 0);
            A[i] = read_A1(An, sn, i);
        }
    };
    // per MFMA pair: 2 MFMAs, one fragment read, a few VALU of the next B fragments, and the
    // step's loads spread over the first sub-steps
    auto interleave = [&](int nvmem) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (2 * k < nvmem) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        }
    };

    // One step t.  Entering: A holds the fragments of (t, sub-step 0), B0 the B fragments of
    // (t, 0), Lc the tables of t.  Ac: stage of t; An: stage of t+1 (complete since the previous
    // barrier); Al: stage that receives X of step t+3.  Wc/Wn: W registers of t and t+1; Wl
    // receives W of t+2.  Ln receives the tables of t+1.
    // ph = t % 4.  Grouped: Gc holds the codes of t's group, Gn receives (at ph 1) those of the
    // next group, first needed for the tables of step t+1 at ph 3.
    bf16x8 B0[2], B1[2];
    GRegs Gc, Gn;
    auto step_body = [&](int t, int ph, const uint8_t *Ac, const uint8_t *An, uint8_t *Al, const WRegs &Wc,
                         const WRegs &Wn, WRegs &Wl, const Lut *Lc, Lut *Ln) {
        load_A(t + 3, Al);
        load_W(t + 2, Wl);
        if (GROUPED && ph == 1) load_G((t >> 2) + 1, Gn);
        dequant_B(Wc, Lc, 1, B1);
        sub_step(B0, Ac, 1);
        interleave(14);
        __builtin_amdgcn_sched_barrier(0);
        dequant_B(Wc, Lc, 2, B0);
        sub_step(B1, Ac, 2);
        interleave(0);
        __builtin_amdgcn_sched_barrier(0);
        // the tables of t+1 are built after the last use of t's
        dequant_B(Wc, Lc, 3, B1);
        make_luts(Wn, ph == 3 ? Gn : Gc, (ph + 1) & 3, Ln);
        sub_step(B0, Ac, 3);
        interleave(0);
        __builtin_amdgcn_sched_barrier(0);
        // next: (t+1, 0), from the next stage and the next W registers
        dequant_B(Wn, Ln, 0, B0);
        sub_step(B1, An, 0);
        interleave(0);
        __builtin_amdgcn_sched_barrier(0);
        // X of t+2 landed (everything issued before this step's loads) and this wave's fragment
        // reads are done; then a bare barrier.  __syncthreads() would add a workgroup release
        // fence, which waits for every LDS write in flight, including the direct-to-LDS loads of
        // t+3 issued at the top of this step, and so would cut their slack to one step.  The
        // signal fences keep the compiler from moving memory operations across the barrier.
        if (vmem_per_step(GROUPED, ph) == 14) __builtin_amdgcn_s_waitcnt(vmcnt_imm(14));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(10));
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // ---- prologue: X of steps 0, 1, 2 and W of 0, 1 in flight; X of 0 and 1 landed ----
    WRegs W0, W1, W2, W3;
    Lut L0[2], L1[2];
    load_A(0, As0);
    load_W(0, W0);
    if (GROUPED) load_G(0, Gc);
    load_A(1, As1);
    load_W(1, W1);
    load_A(2, As2);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(8));   // only the X loads of step 2 pending
    __syncthreads();
    make_luts(W0, Gc, 0, L0);
#pragma unroll
    for (int i = 0; i < 8; ++i) A[i] = read_A1(As0, 0, i);
    dequant_B(W0, L0, 0, B0);

    for (int t = 0; t < main_steps; t += 4) {
        step_body(t, 0, As0, As1, As3, W0, W1, W2, L0, L1);
        step_body(t + 1, 1, As1, As2, As0, W1, W2, W3, L1, L0);
        step_body(t + 2, 2, As2, As3, As1, W2, W3, W0, L0, L1);
        step_body(t + 3, 3, As3, As0, As2, W3, W0, W1, L1, L0);
        if (GROUPED) Gc = Gn;
    }
    // the prefetches past the end are still landing in the ring: drain them before reusing LDS
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- LoRA extension: [X | sT] . [deq(W) ; L2], r/64 more steps (zero padded past r) ----
    if (ext_steps > 0) {
        const __amdgpu_buffer_rsrc_t rAe = make_rsrc(g.sT + m0 * g.r, (g.M - m0) * (int64_t)g.r * 2);
        const __amdgpu_buffer_rsrc_t rBe = make_rsrc(g.L2, (int64_t)g.r * g.N * 2);
        for (int e = 0; e < ext_steps; ++e) {
            const int j0 = e * TK;
            typedef __attribute__((address_space(3))) uint8_t lds_u8;
            lds_u8 *dst = (lds_u8 *)As0 + wave * 8192;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                // same stage layout as X: row 8u + lane/8, logical chunk (lane%8) ^ ((row/2)%8)
                const int row = 8 * (8 * wave + q) + (lane >> 3);
                const int jj = j0 + ((lane & 7) ^ ((row >> 1) & 7)) * 8;
                const uint32_t off = jj < g.r ? (uint32_t)((row * (int64_t)g.r + jj) * 2) : 0xFFFFFFF0u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rAe, (lds_void *)(dst + q * 1024), 16, off, 0, 0, 0);
            }
            // L2 rows j0 .. j0+63, columns n0 .. n0+255: the first 128 columns into stage 2,
            // the rest into stage 3, rows of EXT_ROWB bytes
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int jr = (tid >> 5) + 8 * q, ch = tid & 31;
                const int64_t col = n0 + ch * 8;
                const bool ok = j0 + jr < g.r && col < g.N;
                const u32x4 v = bload16(rBe, ok ? (uint32_t)(((int64_t)(j0 + jr) * g.N + col) * 2) : 0xFFFFFFF0u);
                uint8_t *Bh = (ch < 16) ? As2 : As3;
                *reinterpret_cast<u32x4 *>(Bh + jr * EXT_ROWB + (ch & 15) * 16) = v;
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            const uint8_t *Bh = (wave < 2) ? As2 : As3;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 Be[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // 16-lane group (hh, half): lane i reads rows 32 hh + 8 s + i/4 (+4), columns
                    // c0 + 4 (i%4) .. +3; after the transpose lane i holds column c0 + i
                    const int i16 = lane & 15, half = (lane >> 4) & 1;
                    const int c0 = (wave & 1) * 64 + 32 * j + 16 * half;
                    const int rowb = 32 * hh + 8 * s + (i16 >> 2);
                    const uint8_t *base = Bh + (c0 + 4 * (i16 & 3)) * 2;
                    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + rowb * EXT_ROWB));
                    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + (rowb + 4) * EXT_ROWB));
                    const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    Be[j] = __builtin_bit_cast(bf16x8, v);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const bf16x8 a = read_A1(As0, s, i);
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, Be[j], acc[i][j], 0, 0, 0);
                }
            }
            __syncthreads();
        }
    }

    // ---- epilogue: fp32 -> bf16.  Lane (r32, hh) of tile (i, j) holds column 64 w + 32 j + r32
    // and rows 32 i + 8 (v/4) + 4 hh + v%4; rows past M fall outside the store descriptor ----
    if (g.ksplit > 1) {
        // float32 partial tile
        const __amdgpu_buffer_rsrc_t rP = make_rsrc(g.P + (int64_t)split * g.M * g.N + m0 * g.N, (g.M - m0) * g.N * 4);
        const uint32_t prow = (uint32_t)(g.N * 4);
        const uint32_t poff = (uint32_t)(hh * 4) * prow + (uint32_t)((n0 + 64 * wave + r32) * 4);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (n0 + 64 * wave + 32 * j + r32 >= g.N) continue;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const uint32_t rows = (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3));
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]), rP, poff + j * 128,
                                                          rows * prow, 0);
                }
            }
        }
        return;
    }
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(g.Y + m0 * g.N, (g.M - m0) * g.N * 2);
    const uint32_t row_bytes = (uint32_t)(g.N * 2);
    const uint32_t lane_off = (uint32_t)(hh * 4) * row_bytes + (uint32_t)((n0 + 64 * wave + r32) * 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (n0 + 64 * wave + 32 * j + r32 >= g.N) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
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
}

}  // namespace

hipError_t launch_dqgemm_fwd(const WeightView &w, const uint16_t *X, const uint16_t *sT,
                             const uint16_t *L2, int32_t r, int64_t M, uint16_t *Y,
                             const SplitK &sk, hipStream_t stream) {
    FwdArgs a;
    a.X = X;
    a.packed = w.packed; a.c2 = w.c2; a.c1 = w.c1; a.mean = w.mean; a.dq_int8 = w.dq_int8;
    a.sT = sT; a.L2 = L2; a.Y = Y;
    a.M = M; a.N = w.rows; a.K = w.cols;
    a.r = r;
    for (int j = 0; j < 16; ++j) a.cb.v[j] = w.cb[j];
    const int ntm = (int)((M + TM - 1) / TM);
    const int ntn = (int)((w.rows + TN - 1) / TN);
    const int64_t steps = w.cols / TK;
    a.ksplit = sk.ksplit > 1 ? sk.ksplit : 1;
    a.split_per = (int32_t)(a.ksplit > 1 ? sk.per : steps);
    a.P = sk.P;
    if (a.ksplit > 1 && (!sk.P || sk.per % 4 || (int64_t)(a.ksplit - 1) * sk.per >= steps ||
                         (int64_t)a.ksplit * sk.per < steps))
        return hipErrorInvalidValue;
    const dim3 grid(ntm * ntn * a.ksplit);
    timing_before(stream, 0);
    if (w.cols % 256 == 0)
        hipLaunchKernelGGL(dqgemm_fwd_kernel<true>, grid, dim3(NTHREADS), 0, stream, a);
    else
        hipLaunchKernelGGL(dqgemm_fwd_kernel<false>, grid, dim3(NTHREADS), 0, stream, a);
    hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace nf4k
