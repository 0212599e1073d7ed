// K-extended bf16 MFMA GEMM of the QLoRA linear layer at large token counts (gfx950):
//   C = [A | Ae] . [B | Be]^T         (optionally C += ...)
//   forward : A = X [M, K],  B = deq(W) [N, K],  Ae = sT [M, r],  Be = L2^T [N, r]
//   backward: A = dY [M, N], B = deq(W)^T [K, N], Ae = dT [M, r], Be = L1 [K, r]
// B is the frozen weight after the double dequantization to bf16, written by a separate pass
// (row-major for the forward, transposed for the backward), so both products read B with the
// reduction index contiguous.
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (5) (forward: the BF16 weight from eq. (6) times X, plus the LoRA term) and the
// backward description (gradient to X through the BF16 weight); section 4 eq. (3) (scalar s).
//
// Block tile 256 x 256 outputs, reduction step 64, 4 waves in 2 x 2, each 128 x 128 with
// v_mfma_f32_32x32x16_bf16 (16 tiles, 256 fp32 accumulators).  Both operands go straight from
// global memory to LDS (buffer_load ... lds: no registers, no ds_write), two 32 KB stages each,
// 128-byte rows whose 16-byte chunks are XOR-swizzled by (row / 2) so the fragment reads are
// bank-conflict free.  The LoRA product is appended as r/64 more reduction steps.
//
// Linears sharing X (the q, k and v projections): B holds their expanded weights one after the
// other along N; each output tile belongs to one of them and takes that one's s T, L2^T and output
// buffer in the LoRA steps and the epilogue.
//
// Few output tiles (fewer than half the CUs): the reduction is split over up to 16 workgroups per
// tile, each writing a float32 partial tile, summed afterwards in a fixed order.
//
// Gated MLP backward (dX of gate and up as one product): the reduction runs over two segments,
// [dG | dU] . [deq(W_gate) ; deq(W_up)], each operand of a segment its own buffer, and the LoRA
// steps over [dT_gate | dT_up] . [L1_gate ; L1_up]^T.

#include "common.h"
#include "dqtile.h"
#include "launch.h"

namespace nf4k {

namespace {

constexpr int TM = 256;
constexpr int TN = 256;
constexpr int TK = 64;
constexpr int NTHREADS = 256;
constexpr int STAGE = TM * TK * 2;          // 32 KB per operand stage

struct GemmArgs {
    const uint16_t *A;    // [M, Kred]
    const uint16_t *B;    // [Nout, Kred]
    const uint16_t *Ae;   // [M, r]
    const uint16_t *Be;   // forward: L2^T [Nout, r]; backward: L1 [Nout, r]
    uint16_t *C;          // [M, Nout]
    int64_t M, Nout, Kred;
    int32_t r;
    uint32_t accumulate;
    // two-segment backward: A2 = dU, B2 = deq(W_up)^T, Ae2 = dT_up, Be2 = L1_up (A, B, Ae, Be: gate's);
    // Kred is one segment's length
    const uint16_t *Ae2;
    const uint16_t *Be2;
    const uint16_t *A2, *B2;
    // forward of up to three linears sharing X (their weights concatenated along N, each segment
    // a whole number of 256-column tiles): segment i covers columns seg_start[i] .. seg_start[i+1]
    // and has its own s T (seg_Ae [M, r]), L2^T (seg_Be [N_i, r]) and output (seg_C [M, N_i]).
    // A plain forward is one segment.
    int32_t nseg;
    int64_t seg_start[4];
    const uint16_t *seg_Ae[3];
    const uint16_t *seg_Be[3];
    uint16_t *seg_C[3];
    // split reduction (ksplit > 1): workgroup b takes output tile b % tiles and reduction steps
    // [split per, (split + 1) per) with split = b / tiles, and writes float32 partials:
    // P + split * M * Nout + M * seg_start[i], row-major [M, N_i] per segment
    int32_t ksplit;
    int32_t split_per;
    float *P;
};

template <bool BWD, bool DUAL>
__device__ __forceinline__ void gemm_body(const GemmArgs &g) {
    // one LDS object per stage: a fragment read of one stage provably never aliases the
    // direct-to-LDS loads in flight into the other
    __shared__ __align__(16) uint8_t As0[STAGE];
    __shared__ __align__(16) uint8_t As1[STAGE];
    __shared__ __align__(16) uint8_t Bs0[STAGE];
    __shared__ __align__(16) uint8_t Bs1[STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int r32 = lane & 31, hh = lane >> 5;

    const int ntm = (int)((g.M + TM - 1) / TM);
    const int ntn = (int)((g.Nout + TN - 1) / TN);
    const int ntiles = ntm * ntn;
    const int split = (int)(blockIdx.x / (uint32_t)ntiles);
    int tm, tn;
    tile_coords_grouped<4>(ntm, ntn, (int)blockIdx.x - split * ntiles, tm, tn);
    const int64_t m0 = (int64_t)tm * TM;
    const int64_t n0 = (int64_t)tn * TN;
    const int seg_steps = (int)((g.Kred + TK - 1) / TK);
    // this workgroup's reduction steps: kb .. kb + main_steps - 1 (all of them unless split)
    const int kb = split * g.split_per;
    const int main_steps = DUAL ? 2 * seg_steps : min(seg_steps - kb, g.split_per);
    const int ext_steps = split == g.ksplit - 1 ? (g.r + TK - 1) / TK : 0;

    // tile-relative descriptors: rows past M (or Nout) read zeros
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + m0 * g.Kred, (g.M - m0) * g.Kred * 2);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + n0 * g.Kred, (g.Nout - n0) * g.Kred * 2);
    const __amdgpu_buffer_rsrc_t rA2 = make_rsrc(DUAL ? g.A2 + m0 * g.Kred : g.A, DUAL ? (g.M - m0) * g.Kred * 2 : 0);
    const __amdgpu_buffer_rsrc_t rB2 = make_rsrc(DUAL ? g.B2 + n0 * g.Kred : g.B, DUAL ? (g.Nout - n0) * g.Kred * 2 : 0);

    // ---- loads: instruction q of wave w writes stage rows 8u .. 8u+7 (u = 8w + q); lane l
    // takes row 8u + l/8 and physical chunk l%8, which holds logical chunk (l%8) ^ ((row/2)%8).
    // (row/2) % 8 = (4q + l/16) % 8: the lane's column depends only on the parity of q. ----
    int a_col[2];
    uint32_t voff[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = 8 * (8 * wave + q) + (lane >> 3);
        a_col[q] = ((lane & 7) ^ ((row >> 1) & 7)) * 8;
        voff[q] = (uint32_t)(((lane >> 3) * g.Kred + a_col[q]) * 2);
    }
    const uint32_t wave_off = (uint32_t)(64 * wave * g.Kred * 2);
    const uint32_t row8_off = (uint32_t)(8 * g.Kred * 2);
    // reduction columns this workgroup reads: up to Kred, or to the end of its split
    const int kred32 = DUAL ? (int)g.Kred : (int)min(g.Kred, (int64_t)(kb + main_steps) * TK);
    // Columns at or past that (a ragged last step, or the steps past the end) read zeros.  The
    // whole offset sits in the lane offset (the scalar offset is 0), so rows past the end of the
    // operand are out of range for the descriptor's bound check.
    auto load = [&](__amdgpu_buffer_rsrc_t r, int step, uint8_t *st, int q0 = 0, int q1 = 8) {
        typedef __attribute__((address_space(3))) uint8_t lds_u8;
        lds_u8 *dst = (lds_u8 *)st + wave * 8192;
        const int rem = kred32 - step * TK;
        const uint32_t base = wave_off + (uint32_t)step * (TK * 2);
        const uint32_t v0 = a_col[0] < rem ? voff[0] + base : 0x80000000u;
        const uint32_t v1 = a_col[1] < rem ? voff[1] + base : 0x80000000u;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q < q0 || q >= q1) continue;
            const uint32_t v = ((q & 1) ? v1 : v0) + (uint32_t)q * row8_off;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dst + q * 1024), 16, v, 0, 0, 0);
        }
    };

    // operand A or B of a main-loop step.  Two segments: steps past the first read the second
    // operand pair, picked by a select of the (uniform) descriptor, no branch inside the pinned
    // schedule.
    auto load2 = [&](bool isA, int step, uint8_t *st, int q0 = 0, int q1 = 8) {
        __amdgpu_buffer_rsrc_t r = isA ? rA : rB;
        if (DUAL) {
            const bool second = step >= seg_steps;
            r = second ? (isA ? rA2 : rB2) : r;
            step -= second ? seg_steps : 0;
        } else {
            step += kb;
        }
        load(r, step, st, q0, q1);
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // fragment of sub-step s (16 reduction elements): lane (r32, hh) takes elements
    // 16 s + 8 hh .. +7 of its row; (row/2) % 8 = (r32/2) % 8 for every 32-row group
    uint32_t lds_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) lds_off[s] = (uint32_t)(r32 * 128 + (((2 * s + hh) ^ ((r32 >> 1) & 7)) * 16));
    struct Frags {
        bf16x8 a[4], b[4];
    };
    auto read = [&](const uint8_t *Ast, const uint8_t *Bst, int s, Frags &f) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            f.a[i] = *reinterpret_cast<const bf16x8 *>(Ast + lds_off[s] + (wm * 128 + 32 * i) * 128);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            f.b[j] = *reinterpret_cast<const bf16x8 *>(Bst + lds_off[s] + (wn * 128 + 32 * j) * 128);
    };
    auto mma = [&](const Frags &f) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    };
    // Fragment reads run one sub-step ahead of the MFMAs.  The schedule is pinned: left alone, the
    // scheduler sinks the next sub-step's reads below the current MFMAs (their registers can then
    // be reused), and every sub-step starts by waiting out the LDS latency.  Here each of the
    // first 8 MFMAs of a sub-step is followed by one fragment read, and in a sub-step that
    // carries loads every second MFMA is followed by one direct-to-LDS load (8 per sub-step):
    // the 64 loads of a step per CU, issued together, overfill the texture unit's address queue,
    // and the MFMAs queued behind them in each wave stall.
    auto interleave = [&](int nvmem) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                             // 1 MFMA
            if (k < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                  // 1 DS read
            if ((k & 1) && (k >> 1) < nvmem) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // 1 VMEM
        }
    };
    // One step computes stage (Ac, Bc) while step + 1 lands in (An, Bn).  The workgroup barrier
    // sits between sub-steps 2 and 3: by then every wave has its sub-step 3 fragments in
    // registers, so after it stage c is free for the loads of step + 2, and stage n (step + 1)
    // is complete, so its first fragments are read while sub-step 3's 16 MFMAs run.  (With the
    // barrier at the end of the step, each step opened with its MFMAs waiting on those reads.)
    // The loads of step + 2 go out in two halves, rows q 0-3 of each wave in sub-step 3 and q
    // 4-7 in sub-step 0 of the next step, at least three sub-steps before the barrier that
    // waits for them.  On entry f0 holds, or is receiving, sub-step 0 of stage c.
    Frags f0, f1;
    auto step_body = [&](int step, uint8_t *Ac, uint8_t *Bc, uint8_t *An, uint8_t *Bn) {
#pragma unroll
        for (int s = 0; s < 3; ++s) {
            Frags &cur = (s & 1) ? f1 : f0;
            Frags &nxt = (s & 1) ? f0 : f1;
            if (s == 0) {
                load2(true, step + 1, An, 4, 8);
                load2(false, step + 1, Bn, 4, 8);
            }
            read(Ac, Bc, s + 1, nxt);
            mma(cur);
            interleave(s == 0 ? 8 : 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        // step + 1 landed (this wave's loads) and this wave's fragment reads of stage c are done
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (0 << 8));
        __syncthreads();
        read(An, Bn, 0, f0);
        load2(true, step + 2, Ac, 0, 4);
        load2(false, step + 2, Bc, 0, 4);
        mma(f1);
        interleave(8);
        __builtin_amdgcn_sched_barrier(0);
    };

    load2(true, 0, As0);
    load2(false, 0, Bs0);
    load2(true, 1, As1, 0, 4);
    load2(false, 1, Bs1, 0, 4);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    read(As0, Bs0, 0, f0);
    int step = 0;
    for (; step + 1 < main_steps; step += 2) {
        step_body(step, As0, Bs0, As1, Bs1);
        step_body(step + 1, As1, Bs1, As0, Bs0);
    }
    if (step < main_steps) step_body(step, As0, Bs0, As1, Bs1);   // odd count: the last one
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // Lane indices for the code after the main loop, recomputed (mbcnt) rather than kept live
    // across it: held over the loop they were spilled, and a kernel with scratch memory costs
    // several microseconds more to dispatch.
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int r32_e = lane_e & 31, hh_e = lane_e >> 5;

    // The tile's output segment (forward): its adapter, its output buffer, and the tile's first
    // column within that buffer.  Uniform per workgroup.
    // (scalar: the segment index goes through readfirstlane, and the kernel-argument arrays are
    // indexed by it, so nothing here takes vector registers, which the main loop has used up)
    const uint16_t *Ae_t = g.Ae, *Be_t = g.Be;
    uint16_t *C_t = g.C;
    int64_t cN = g.Nout, cn0 = n0;
    if (!BWD && !DUAL) {
        const int sg = __builtin_amdgcn_readfirstlane(
            (g.nseg > 2 && n0 >= g.seg_start[2]) ? 2 : ((g.nseg > 1 && n0 >= g.seg_start[1]) ? 1 : 0));
        Ae_t = g.seg_Ae[sg];
        Be_t = g.seg_Be[sg];
        C_t = g.seg_C[sg];
        cN = g.seg_start[sg + 1] - g.seg_start[sg];
        cn0 = n0 - g.seg_start[sg];
    }

    // ---- LoRA extension: r/64 more steps (zero padded past r) ----
    //   A tile: Ae rows m0.., columns j (same swizzled layout, straight to LDS), in As0
    //   B tile: Be = L2^T (forward; transposed by the expansion launch) or L1 (backward) [Nout, r]:
    //           rows n, columns j -> swizzled layout in Bs0, straight to LDS, row reads
    if (ext_steps > 0) {
        const __amdgpu_buffer_rsrc_t rAe = make_rsrc(Ae_t + m0 * g.r, (g.M - m0) * (int64_t)g.r * 2);
        const __amdgpu_buffer_rsrc_t rBe = make_rsrc(Be_t + cn0 * g.r, (cN - cn0) * (int64_t)g.r * 2);
        typedef __attribute__((address_space(3))) uint8_t lds_u8;
        // two segments: the up adapter's steps follow the gate's
        const __amdgpu_buffer_rsrc_t rAeU = make_rsrc(DUAL ? g.Ae2 + m0 * g.r : g.Ae,
                                                      DUAL ? (g.M - m0) * (int64_t)g.r * 2 : 0);
        const __amdgpu_buffer_rsrc_t rBeU = make_rsrc(DUAL ? g.Be2 + n0 * g.r : g.Be,
                                                      DUAL ? (g.Nout - n0) * (int64_t)g.r * 2 : 0);
        for (int e = 0; e < (DUAL ? 2 : 1) * ext_steps; ++e) {
            const bool up = DUAL && e >= ext_steps;
            const int j0 = (up ? e - ext_steps : e) * TK;
            const __amdgpu_buffer_rsrc_t ra = up ? rAeU : rAe;
            const __amdgpu_buffer_rsrc_t rb = up ? rBeU : rBe;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int row = 8 * (8 * wave + q) + (lane_e >> 3);
                const int jj = j0 + a_col[q & 1];
                const uint32_t off = jj < g.r ? (uint32_t)((row * (int64_t)g.r + jj) * 2) : 0x80000000u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void *)((lds_u8 *)As0 + wave * 8192 + q * 1024),
                                                         16, off, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)((lds_u8 *)Bs0 + wave * 8192 + q * 1024),
                                                         16, off, 0, 0, 0);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                Frags f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    f.a[i] = *reinterpret_cast<const bf16x8 *>(As0 + lds_off[s] + (wm * 128 + 32 * i) * 128);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    f.b[j] = *reinterpret_cast<const bf16x8 *>(Bs0 + lds_off[s] + (wn * 128 + 32 * j) * 128);
                mma(f);
            }
            __syncthreads();
        }
    }

    // ---- epilogue: fp32 -> bf16.  Lane (r32, hh) of tile (i, j) holds column
    // wn*128 + 32 j + r32 and rows wm*128 + 32 i + 8 (v/4) + 4 hh + v%4 ----
    if (!DUAL && g.ksplit > 1) {
        // float32 partial tile: rows past M fall outside the descriptor
        // the segment's partials start at M * (its first column), n0 - cn0
        float *Pt = g.P + (int64_t)split * g.M * g.Nout + g.M * (n0 - cn0) + m0 * cN;
        const __amdgpu_buffer_rsrc_t rP = make_rsrc(Pt, (g.M - m0) * cN * 4);
        const uint32_t row_bytes = (uint32_t)(cN * 4);
        const uint32_t lane_off = (uint32_t)((wm * 128 + hh_e * 4) * row_bytes) + (uint32_t)((cn0 + wn * 128 + r32_e) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (cn0 + wn * 128 + j * 32 + r32_e >= cN) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const uint32_t rows = (uint32_t)(i * 32 + (v >> 2) * 8 + (v & 3));
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]), rP, lane_off + j * 128,
                                                          rows * row_bytes, 0);
                }
            }
        }
    } else if (!g.accumulate) {
        const __amdgpu_buffer_rsrc_t rC = make_rsrc(C_t + m0 * cN, (g.M - m0) * cN * 2);
        const uint32_t row_bytes = (uint32_t)(cN * 2);
        const uint32_t lane_off = (uint32_t)((wm * 128 + hh_e * 4) * row_bytes) + (uint32_t)((cn0 + wn * 128 + r32_e) * 2);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (cn0 + wn * 128 + j * 32 + r32_e >= cN) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
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
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t col = n0 + wn * 128 + j * 32 + r32_e;
                if (col >= g.Nout) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + hh_e * 4 + (v & 3);
                    if (row < g.M) {
                        uint16_t *p = g.C + row * g.Nout + col;
                        *p = (uint16_t)f32_to_bf16(acc[i][j][v] + bf16_to_f32(*p));
                    }
                }
            }
        }
    }
}

template <bool BWD>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(GemmArgs g) {
    gemm_body<BWD, false>(g);
}

__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_dual_kernel(GemmArgs g) {
    gemm_body<true, true>(g);
}

template <bool BWD>
hipError_t launch_impl(GemmArgs &a, const SplitK &sk, hipStream_t stream) {
    const int ntm = (int)((a.M + TM - 1) / TM);
    const int ntn = (int)((a.Nout + TN - 1) / TN);
    const int64_t steps = (a.Kred + TK - 1) / TK;
    a.ksplit = sk.ksplit > 1 ? sk.ksplit : 1;
    a.split_per = (int32_t)(a.ksplit > 1 ? sk.per : steps);
    a.P = sk.P;
    if (a.ksplit > 1 && (!sk.P || (int64_t)(a.ksplit - 1) * sk.per >= steps || (int64_t)a.ksplit * sk.per < steps))
        return hipErrorInvalidValue;
    timing_before(stream, BWD ? 1 : 0);
    hipLaunchKernelGGL(gemm_bf16_kernel<BWD>, dim3(ntm * ntn * a.ksplit), dim3(NTHREADS), 0, stream, a);
    hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace

hipError_t launch_gemm_bf16_fwd(const uint16_t *X, const uint16_t *Wd, const uint16_t *sT, const uint16_t *L2T,
                                int32_t r, int64_t M, int64_t N, int64_t K, uint16_t *Y, const SplitK &sk,
                                hipStream_t stream) {
    const FwdSegment seg{N, sT, L2T, Y};
    return launch_gemm_bf16_fwd_seg(X, Wd, &seg, 1, r, M, K, sk, stream);
}

hipError_t launch_gemm_bf16_fwd_seg(const uint16_t *X, const uint16_t *Wd, const FwdSegment *seg, int nseg, int32_t r,
                                    int64_t M, int64_t K, const SplitK &sk, hipStream_t stream) {
    if (nseg < 1 || nseg > 3) return hipErrorInvalidValue;
    GemmArgs a{};
    a.A = X; a.B = Wd;
    a.nseg = nseg;
    int64_t n = 0;
    for (int i = 0; i < nseg; ++i) {
        // every boundary but the last on a tile edge: a tile never spans two segments
        if (i + 1 < nseg && seg[i].N % TN) return hipErrorInvalidValue;
        a.seg_start[i] = n;
        a.seg_Ae[i] = seg[i].sT; a.seg_Be[i] = seg[i].L2T; a.seg_C[i] = seg[i].Y;
        n += seg[i].N;
    }
    for (int i = nseg; i < 4; ++i) a.seg_start[i] = n;
    a.Ae = seg[0].sT; a.Be = seg[0].L2T; a.C = seg[0].Y;
    a.M = M; a.Nout = n; a.Kred = K; a.r = r; a.accumulate = 0;
    return launch_impl<false>(a, sk, stream);
}

hipError_t launch_gemm_bf16_bwd_dual(const uint16_t *dG, const uint16_t *WdTg, const uint16_t *dTg, const uint16_t *L1g,
                                    const uint16_t *dU, const uint16_t *WdTu, const uint16_t *dTu, const uint16_t *L1u,
                                    int32_t r, int64_t M, int64_t F, int64_t K, uint16_t *dX, bool accumulate,
                                    hipStream_t stream) {
    GemmArgs a{};
    a.A = dG; a.B = WdTg; a.Ae = dTg; a.Be = L1g; a.C = dX;
    a.A2 = dU; a.B2 = WdTu; a.Ae2 = dTu; a.Be2 = L1u;
    a.M = M; a.Nout = K; a.Kred = F; a.r = r; a.accumulate = accumulate ? 1u : 0u;
    a.ksplit = 1; a.split_per = (int32_t)((F + TK - 1) / TK);
    const int ntm = (int)((M + TM - 1) / TM);
    const int ntn = (int)((K + TN - 1) / TN);
    timing_before(stream, 4);
    hipLaunchKernelGGL(gemm_bf16_dual_kernel, dim3(ntm * ntn), dim3(NTHREADS), 0, stream, a);
    hipError_t e = hipGetLastError();
    timing_after(stream);
    return e;
}

hipError_t launch_gemm_bf16_bwd(const uint16_t *dY, const uint16_t *WdT, const uint16_t *dT, const uint16_t *L1,
                                int32_t r, int64_t M, int64_t N, int64_t K, uint16_t *dX, bool accumulate,
                                const SplitK &sk, hipStream_t stream) {
    GemmArgs a{};
    a.A = dY; a.B = WdT; a.Ae = dT; a.Be = L1; a.C = dX;
    a.M = M; a.Nout = K; a.Kred = N; a.r = r; a.accumulate = accumulate ? 1u : 0u;
    return launch_impl<true>(a, sk, stream);
}

}  // namespace nf4k
