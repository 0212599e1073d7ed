// Internal launcher declarations shared by the kernel sources and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4k {

struct Reduction;

struct WeightView {
    const uint8_t *packed;
    const uint8_t *c2;
    const float *c1;
    const float *mean;
    int64_t rows, cols;
    float cb[16];
    uint32_t dq_int8;     // second-level codes: 0 = E4M3, 1 = int8
};

hipError_t launch_quantize(const float *W, int64_t numel, const float thr[15], uint32_t zero_code,
                           uint8_t *packed, float *absmax, hipStream_t stream);
size_t double_quant_ws(int64_t nb);
// int8: second-level codes by eq. (1) at 8 bits (scale max|y| / 127) instead of E4M3
hipError_t launch_double_quant(const float *absmax, int64_t nb, uint8_t *codes, float *scales,
                               float *mean, void *ws, bool int8, hipStream_t stream);
// absmax_plain != NULL: one-level dequantization (eq. 2) with those float32 block constants
hipError_t launch_dequant(const uint8_t *packed, const uint8_t *absmax_q, const float *absmax_scale,
                          const float *absmax_mean, const float *absmax_plain, uint32_t dq_int8,
                          int64_t numel, const float cb[16], uint16_t *out, hipStream_t stream);

// Split of a product's reduction over ksplit workgroups per output tile, for shapes whose output
// tiles alone would leave CUs idle.  Split k takes reduction steps [k per, (k + 1) per) (per from
// gemm_split); the last split also runs the LoRA steps.  With ksplit > 1 the kernel writes
// float32 partials P[k] (row-major [M, Nout]; the forward of several linears keeps each one's
// columns together, [M, N_i] at M * (its first column)) instead of the bf16 output, and a
// fixed-order reduction (launch_reduce_partials) sums them.
struct SplitK {
    int ksplit;
    int64_t per;     // reduction steps per split
    float *P;
};
// The split of a product with `tiles` output tiles and `steps` reduction steps: as many splits as
// keep the launch within one workgroup per CU (at most 16), each a multiple of `quantum` steps
// (per), none empty.  ksplit = 1 (per = steps) when the tiles fill the chip.
struct SplitPlan {
    int ksplit;
    int64_t per;
};
SplitPlan gemm_split(int64_t tiles, int64_t steps, int quantum);

hipError_t launch_dqgemm_fwd(const WeightView &w, const uint16_t *X, const uint16_t *sT,
                             const uint16_t *L2, int32_t r, int64_t M, uint16_t *Y,
                             const SplitK &sk, hipStream_t stream);
// small-batch forward (M <= 64: 9 or more tokens, or fewer on shapes the row kernel does not
// take); with sk.ksplit > 1 each workgroup takes sk.per macro steps (256
// columns each, a multiple of 4) of the reduction and writes float32 partials to sk.P ([ksplit][M][N],
// the LoRA term in the last split), which launch_reduce_partials then sums
SplitPlan gemv_wide_split(int64_t M, int64_t N, int64_t K);
// s T either reduced (sT, bf16 [M, r]) or as T's pending reduction (Tred: its partials, split
// count, T_out as out and s as s2), which the kernel then sums itself; exactly one is given
hipError_t launch_gemv_wide_fwd(const WeightView &w, const uint16_t *X, const Reduction *Tred, const uint16_t *sT,
                                const uint16_t *L2, int32_t r, int64_t M, uint16_t *Y, const SplitK &sk,
                                hipStream_t stream);
// decode-size forward (M <= 8): two launches; Tp is fp32 scratch of the size gemv_plan gives (Yp unused)
struct GemvPlan {
    int nseg, nkc;
    size_t yp_floats, tp_floats;
};
GemvPlan gemv_plan(int64_t M, int64_t N, int64_t K, int32_t r);
// whether launch_gemv_fwd takes this shape (M <= 8 and the reduction fits one workgroup's waves)
bool gemv_fits(int64_t M, int64_t N, int64_t K, int32_t r);
// T (bf16 [M, r]) exactly as launch_gemv_fwd computes it: its partials into Tp, then their sum
hipError_t launch_gemv_T(const uint16_t *X, const uint16_t *L1, int32_t r, int64_t M, int64_t K, float *Tp,
                        uint16_t *T, hipStream_t stream);
hipError_t launch_gemv_fwd(const WeightView &w, const uint16_t *X, const uint16_t *L1, const uint16_t *L2,
                           float scale, int32_t r, int64_t M, uint16_t *Y, uint16_t *T_out, float *Yp,
                           float *Tp, hipStream_t stream);
// large token counts: the weight is expanded to bf16 once per call (rows [N, K] for the forward,
// transposed [K, N] for the backward), then a K-extended bf16 GEMM
// red (optional): a partials reduction carried by extra workgroups of the same launch
// tr_in (optional, rows layout only): extra workgroups also transpose tr_in [tr_r, tr_n] into
// tr_out [tr_n, tr_r] (the forward GEMM's L2, so its LoRA step loads like the backward's L1)
hipError_t launch_expand_weight(const WeightView &w, bool transposed, uint16_t *out, const Reduction *red,
                                hipStream_t stream, const uint16_t *tr_in = nullptr,
                                uint16_t *tr_out = nullptr, int32_t tr_r = 0, int64_t tr_n = 0);
// L2T: the adapter's L2 transposed, [N, r]
hipError_t launch_gemm_bf16_fwd(const uint16_t *X, const uint16_t *Wd, const uint16_t *sT, const uint16_t *L2T,
                                int32_t r, int64_t M, int64_t N, int64_t K, uint16_t *Y, const SplitK &sk,
                                hipStream_t stream);
// up to three linears sharing X in one product: Wd holds their expanded weights one after the
// other ([sum N_i, K]); segment i has N_i output columns (a multiple of 256 but for the last),
// its s T [M, r], L2^T [N_i, r] and output Y_i [M, N_i]
struct FwdSegment {
    int64_t N;
    const uint16_t *sT, *L2T;
    uint16_t *Y;
};
hipError_t launch_gemm_bf16_fwd_seg(const uint16_t *X, const uint16_t *Wd, const FwdSegment *seg, int nseg, int32_t r,
                                    int64_t M, int64_t K, const SplitK &sk, hipStream_t stream);
// gated MLP backward: dX = [dG | dU] . [deq(W_gate) ; deq(W_up)] + [dT_gate | dT_up] . [L1_gate ; L1_up]^T,
// one product whose reduction runs over the two segments (WdT_*: [K, F] transposed expansions)
hipError_t launch_gemm_bf16_bwd_dual(const uint16_t *dG, const uint16_t *WdTg, const uint16_t *dTg, const uint16_t *L1g,
                                    const uint16_t *dU, const uint16_t *WdTu, const uint16_t *dTu, const uint16_t *L1u,
                                    int32_t r, int64_t M, int64_t F, int64_t K, uint16_t *dX, bool accumulate,
                                    hipStream_t stream);
// with sk.ksplit > 1, accumulate is the reduction's (the kernel writes partials)
hipError_t launch_gemm_bf16_bwd(const uint16_t *dY, const uint16_t *WdT, const uint16_t *dT, const uint16_t *L1,
                                int32_t r, int64_t M, int64_t N, int64_t K, uint16_t *dX, bool accumulate,
                                const SplitK &sk, hipStream_t stream);
hipError_t launch_dqgemm_bwd(const WeightView &w, const uint16_t *dY, const uint16_t *dT,
                             const uint16_t *L1, int32_t r, int64_t M, uint16_t *dX,
                             bool accumulate, const SplitK &sk, hipStream_t stream);

int choose_split(int64_t tiles, int64_t red_steps);
// b_rows_k: B given as [Kred, R] (true) or as [R, Kred] (false)
hipError_t launch_skinny_nt(const uint16_t *A, const uint16_t *B, bool b_rows_k, float *P, int64_t M,
                            int32_t R, int64_t Kred, int nsplit, hipStream_t stream);
// P[ms] = U[rows ms, :]^T . V[rows ms, :] (U [M, Pn], V [M, Qn]); one launch for one product, or
// two independent ones (b non-NULL)
struct TnProduct {
    const uint16_t *U, *V;
    float *P;
    int64_t Pn, Qn;
    int nsplit;
    // unsplit (nsplit == 1) with out set: bf16(scale * product) written to out [Pn, Qn] directly,
    // what the reduction of the one partial would write, and P unused
    uint16_t *out = nullptr;
    float scale = 1.0f;
};
hipError_t launch_skinny_tn(const TnProduct &a, const TnProduct *b, int64_t M, hipStream_t stream);
// out = bf16(s1 * sum of the nsplit partials), out2 (optional) = bf16(s2 * same); partial k of
// element i at P[k stride + i] (stride 0: n); accum: out = bf16(s1 * sum + out) (out2 unused).
// One launch for one to three reductions.
struct Reduction {
    const float *P;
    int nsplit;
    int64_t n;
    float s1;
    uint16_t *out;
    float s2;
    uint16_t *out2;
    int64_t stride = 0;
    bool accum = false;
};
hipError_t launch_reduce_partials(const Reduction &a, const Reduction *b, hipStream_t stream,
                                  const Reduction *c = nullptr);
struct RedProb;
RedProb red_prob(const Reduction &r, uint32_t &nblocks);

// Optional per-thread timing events recorded on the launch stream right before and after each
// instrumented launch (see nf4.h).
void timing_before(hipStream_t stream, int kind);
void timing_after(hipStream_t stream);

hipError_t launch_swiglu_fwd(const uint16_t *g, const uint16_t *u, uint16_t *h, int64_t n,
                             hipStream_t stream);
hipError_t launch_swiglu_bwd(const uint16_t *dh, const uint16_t *g, const uint16_t *u, uint16_t *dg,
                             uint16_t *du, int64_t n, hipStream_t stream);

}  // namespace nf4k
