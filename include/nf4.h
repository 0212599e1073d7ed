/*
 * nf4.h -- C ABI of the MI355X (gfx950) NF4 quantized-codebook linear layer with a LoRA branch.
 *
 * Citations refer to the page "QLoRA: Efficient Finetuning of Quantized LLMs" study notes
 * (gitcode.csdn.net/6a0046f754b52172bc72e356), by section and equation.
 *
 * Conventions shared by every entry point
 *   - Device pointers point to memory on the current HIP device; host pointers are marked.
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major and contiguous.
 *   - The frozen weight W is stored [rows = N_out, cols = K_in] row-major (the pages write
 *     W in R^{h x o}, i.e. its transpose), so the layer computes Y = X deq(W)^T + s (X L1) L2.
 *   - Ownership: the caller owns every buffer, including the workspace (sized by the matching
 *     *_workspace_size query).  The library never allocates, frees or synchronises device
 *     memory and keeps no mutable global state; calls are stream-ordered on `stream`
 *     (a hipStream_t; NULL means the default stream).
 *   - Errors: every argument check runs before any HIP call and returns a negative status.
 *     A failed launch returns NF4_ERR_HIP with the runtime's text in nf4_last_error().  Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Device pointers that kernels read or write with 16-byte accesses must be 16-byte aligned
 *     (NF4_ERR_ALIGN otherwise); allocator-returned pointers always are.
 *   - Determinism: identical inputs give identical output bits, run to run (no floating-point
 *     atomics; every reduction has a fixed order).
 */
#ifndef NF4_H
#define NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    NF4_OK = 0,
    NF4_ERR_NULL = -1,         /* a required pointer is NULL */
    NF4_ERR_SHAPE = -2,        /* a size is negative, zero where not allowed, or inconsistent */
    NF4_ERR_ALIGN = -3,        /* a device pointer is not 16-byte aligned */
    NF4_ERR_UNSUPPORTED = -4,  /* a valid but unimplemented parameter (block != 64, ...) */
    NF4_ERR_WORKSPACE = -5,    /* workspace missing or smaller than the size query returned */
    NF4_ERR_HIP = -6,          /* the HIP runtime reported an error; see nf4_last_error() */
    NF4_ERR_ARG = -7           /* any other invalid argument (NaN scale, bad delta, flags) */
};

/* Text for a status code (static storage, never NULL). */
const char *nf4_status_string(int status);
/* Detail of the last error on the calling thread (thread-local storage, never NULL). */
const char *nf4_last_error(void);

/* Library version, "major.minor.patch" (static storage). */
const char *nf4_version(void);

/*
 * NF4 codebook -- section 3.2, eq. (4) with the asymmetric exact-zero construction, and
 * section 5.1.2 (Fig. 7 text: 8 values on one half, 7 on the other, plus 0).
 * Each half of N(0,1) gets an evenly spaced probability grid from 0.5 to the tail probability
 * `delta` (9 points on the positive half, 8 on the negative, both counting 0.5); the quantiles
 * are divided by Phi^-1(delta), the negative half negated, merged with one 0, and rounded once
 * to float32.
 *   out_codebook: HOST float[16], written ascending; out[0] = -1, out[7] = 0, out[15] = +1.
 *   delta: tail probability in (0.5, 1); pass 0 for the default 1 - (1/32 + 1/30)/2.
 * Host-only and synchronous.  NF4_ERR_NULL, NF4_ERR_ARG on a bad delta.
 */
int nf4_build_codebook(float out_codebook[16], double delta);

/*
 * The 4-bit types NF4 is compared with -- abstract page (gitcode.csdn.net/69bbdcd90a2f6a37c5989d83),
 * section 1 (NF4 against 4-bit integers and 4-bit floats), and the study notes, section 5.1.2
 * (Table 2; QLoRA with FP4 and NF4 in Table 3).  The pages define neither layout; these tables
 * are readings.  Both go through the same quantize / dequant / linear entry points as NF4 (the
 * kernels only look codes up in the 16-entry table), so a weight quantized with one of them is
 * used by passing the same table in nf4_weight.codebook.
 *   nf4_build_int4_codebook: eq. (1) at 4 bits, round(7 x / absmax) in [-7, 7]: out[c] = (c - 8) / 7,
 *     the two's complement integers -8 .. 7 over 7 (out[8] = 0; out[0] = -8/7 is never nearest).
 *   nf4_build_fp4_codebook: E2M1 (sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6) over 6, ascending: out[0] = -1, out[7] = out[8] = 0 (E2M1's
 *     negative zero is stored as +0 and never produced), out[15] = +1.
 *   out_codebook: HOST float[16].  Host-only and synchronous.  NF4_ERR_NULL on a NULL pointer.
 */
int nf4_build_int4_codebook(float out_codebook[16]);
int nf4_build_fp4_codebook(float out_codebook[16]);

/*
 * Level-1 block-wise quantization -- section 3.1 (flatten, n = numel/B blocks of B consecutive
 * elements, one constant per block; eq. (1) in absmax form) and section 3.2 step 3 (absmax
 * normalisation to [-1, 1]).
 *   W:        device float32 [numel], the row-major flattening of the weight.
 *   numel:    >= 0.  A short last block's absmax covers only its valid elements.
 *   block:    must be 64 (section 3.5), else NF4_ERR_UNSUPPORTED.
 *   codebook: HOST float[16], ascending, containing 0.0f (from nf4_build_codebook, or
 *             nf4_build_int4_codebook / nf4_build_fp4_codebook).  Equal neighbours are allowed:
 *             the lower index is the one produced.  Copied into the kernel arguments.
 *   packed:   device uint8 [ceil(numel/2)].  Element 2i in bits 0-3 of byte i, element 2i+1 in
 *             bits 4-7; an odd tail is padded with the zero code.
 *   absmax:   device float32 [ceil(numel/64)], the per-block max |x|.
 * Per element: n = fp32(x / absmax) (IEEE division), code = nearest codeword, ties to the lower
 * index; an all-zero block gets the zero code (the first 0.0f entry) everywhere.  Inputs must be
 * finite.
 * W and packed must be 16-byte aligned.
 */
int nf4_quantize(const float *W, int64_t numel, int32_t block, const float codebook[16],
                 uint8_t *packed, float *absmax, void *stream);

/*
 * Level-2 (double) quantization of the block constants -- section 3.3: the constants are
 * centred by their mean and quantized to an 8-bit float in blocks of 256.
 *   absmax:       device float32 [nblocks] (from nf4_quantize), 16-byte aligned.
 *   dq_block:     must be 256, else NF4_ERR_UNSUPPORTED.
 *   absmax_q:     device uint8 [nblocks], OCP FP8 E4M3 codes of (absmax - mean) / scale.
 *   absmax_scale: device float32 [ceil(nblocks/256)], scale_j = fp32(max_j |absmax - mean| / 448),
 *                 the multiplier that undoes the scaling (the inverse of eq. (1)'s constant).
 *   absmax_mean:  device float32 [1], mean = fp32(S / nblocks) where S is the float64 sum taken as
 *                 a 256-ary tree: groups of 256 consecutive values, each summed in ascending order,
 *                 then the group sums the same way, level by level, until one value is left.
 *   workspace:    device, >= nf4_double_quant_workspace_size(nblocks, dq_block) bytes.
 * Codes: E4M3 round-to-nearest-even of clamp(fp32(y / scale_j), -448, 448), sign kept; all 0x00
 * when scale_j == 0.
 */
size_t nf4_double_quant_workspace_size(int64_t nblocks, int32_t dq_block);
int nf4_double_quant(const float *absmax, int64_t nblocks, int32_t dq_block, uint8_t *absmax_q,
                     float *absmax_scale, float *absmax_mean, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * The same second level with 8-bit integer codes instead of the 8-bit float: eq. (1) of
 * section 3.1 at 8 bits, applied to the mean-centred constants (a reading: the pages name the
 * second level's format only as an 8-bit float; Int8 is the integer alternative of eq. (1)).
 * Arguments, mean and workspace exactly as nf4_double_quant, except:
 *   absmax_q:     two's complement codes, rint(fp32(y / scale_j)) clamped to [-127, 127]
 *                 (ties to even); all 0 when scale_j == 0.
 *   absmax_scale: scale_j = fp32(max_j |absmax - mean| / 127).
 * A weight encoded this way is described with dq_format = NF4_DQ_INT8.
 */
int nf4_double_quant_int8(const float *absmax, int64_t nblocks, int32_t dq_block, uint8_t *absmax_q,
                          float *absmax_scale, float *absmax_mean, void *workspace,
                          size_t workspace_bytes, void *stream);

/* Second-level code formats (nf4_weight.dq_format). */
enum { NF4_DQ_E4M3 = 0, NF4_DQ_INT8 = 1 };

/*
 * One frozen NF4 weight in double-quantized form (section 3.5, eq. (5) and eq. (6)).
 * All pointers are device pointers produced by nf4_quantize + nf4_double_quant (or
 * nf4_double_quant_int8, with dq_format = NF4_DQ_INT8).
 */
typedef struct nf4_weight {
    const uint8_t *packed;        /* [rows*cols/2] 4-bit codes */
    const uint8_t *absmax_q;      /* [rows*cols/block] 8-bit codes of the block constants */
    const float *absmax_scale;    /* [ceil(nblocks/dq_block)] second-level multipliers */
    const float *absmax_mean;     /* [1] the mean removed before the second level */
    int64_t rows;                 /* N_out */
    int64_t cols;                 /* K_in */
    int32_t block;                /* 64 */
    int32_t dq_block;             /* 256 */
    float codebook[16];           /* the codebook used by nf4_quantize (host copy) */
    int32_t dq_format;            /* NF4_DQ_E4M3 (nf4_double_quant) or NF4_DQ_INT8
                                     (nf4_double_quant_int8); zero-initialised means E4M3 */
} nf4_weight;

/*
 * Double dequantization to BF16 -- section 3.5, eq. (6), with eq. (2) at each level:
 *   a'_b = fmaf(E4M3(absmax_q[b]), absmax_scale[b / dq_block], mean)   (one rounding;
 *          the code read as a signed integer when dq_format is NF4_DQ_INT8)
 *   out[i] = bf16_RNE(fp32(codebook[code_i] * a'_{i / block}))
 *   out_bf16: device uint16 [rows*cols], 16-byte aligned.  rows*cols must be even.
 */
int nf4_dequant(const nf4_weight *w, uint16_t *out_bf16, void *stream);

/*
 * Single-level dequantization to BF16 -- section 3.1, eq. (2), for a weight quantized without
 * the second level (the "no DQ" rows of section 5.1.2's comparison):
 *   out[i] = bf16_RNE(fp32(codebook[code_i] * absmax[i / block]))
 *   packed:   device uint8 [ceil(numel/2)] from nf4_quantize; 16-byte aligned.
 *   absmax:   device float32 [ceil(numel/block)] from nf4_quantize.
 *   numel:    >= 0 (0 is a no-op); block must be 64.
 *   codebook: HOST float[16], the table passed to nf4_quantize (same checks).
 *   out_bf16: device uint16 [numel], 16-byte aligned.
 */
int nf4_dequant_single(const uint8_t *packed, const float *absmax, int64_t numel, int32_t block,
                       const float codebook[16], uint16_t *out_bf16, void *stream);

/*
 * QLoRA linear forward -- section 3.5 eq. (5) with the LoRA scalar s of eq. (3) (section 4):
 *   T = X L1;  Y = X deq(W)^T + s T L2
 *   X: [M, K] bf16; L1: [K, r] bf16; L2: [r, N] bf16; Y: [M, N] bf16 (N = w->rows, K = w->cols).
 *   T_out: optional [M, r] bf16 (T = X L1, unscaled), kept for the backward pass; may be NULL.
 *   scale: s (finite).  M >= 1, 1 <= r <= 128, K % 64 == 0.
 *   The weight's block dequantization is fused into the matrix product; accumulation is fp32.
 *   workspace: >= qlora_linear_workspace_size(M, N, K, r) bytes.
 */
size_t qlora_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t r);

/*
 * How the linear layer runs a shape (host, no GPU work): info[0] = the forward's path (1: decode
 * GEMV, up to 8 tokens; 2: wide GEMV, up to 64; 3: fused dequant GEMM; 4: bf16 expansion of the
 * weight, then the bf16 GEMM), info[1] = the workgroups each output tile (each block of rows on
 * the wide GEMV) of the forward's product splits its reduction over (1: not split, as always on
 * the decode GEMV), info[2] = the same for the backward's dX product, info[3] = the backward's dX
 * path (3 or 4: the GEMVs are forward only).
 * Split products sum float32 partials in a fixed order, so a split and an unsplit product of the
 * same values can differ in their last bits.  Returns NF4_OK, or NF4_ERR_SHAPE / NF4_ERR_NULL.
 */
int qlora_linear_route(int64_t M, int64_t N, int64_t K, int32_t r, int32_t info[4]);
int qlora_linear_fwd(const nf4_weight *w, const uint16_t *X, const uint16_t *L1,
                     const uint16_t *L2, float scale, int64_t M, int32_t r, uint16_t *Y,
                     uint16_t *T_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The forward above for callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and results, bit for bit, with the
 * workspace taken from a static device array of QLORA_STATIC_SCRATCH_BYTES (128 MiB) that the
 * library holds on each GPU it runs on until the process ends.  The caller still passes the
 * inputs and outputs; the call allocates nothing and calls no allocating routine.
 *   Arguments, limits and results as qlora_linear_fwd.  Shapes whose forward needs more scratch
 *   than the array holds return NF4_ERR_WORKSPACE (nf4_last_error() gives the size needed): this
 *   covers decode and mid-size token counts for weights of up to tens of thousands of rows, and
 *   from 1024 tokens (where the weight is expanded to bf16) weights of up to about 60 M elements,
 *   fewer where the product's reduction is split (its float32 partials also live there).
 *   Every call on one GPU uses the same array: calls that overlap on one GPU (concurrent streams,
 *   threads) race and give undefined results.  The first call on a device looks the array's
 *   address up (hipGetSymbolAddress) with that device current.
 */
#define QLORA_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
int qlora_linear_fwd_static(const nf4_weight *w, const uint16_t *X, const uint16_t *L1,
                            const uint16_t *L2, float scale, int64_t M, int32_t r, uint16_t *Y,
                            uint16_t *T_out, void *stream);

/*
 * Up to three QLoRA linears that share their input -- the q, k and v projections of an attention
 * block, each with its own adapter (LoRA on every linear layer: section 4; each linear is
 * section 3.5 eq. (5)):   Y_i = X deq(W_i)^T + s (X L1_i) L2_i,  i = 0 .. n-1.
 *   n: 1 to 3.  w, L1, L2, Y: arrays of n entries (HOST arrays of device pointers); T_out: NULL
 *   or an array of n entries, each NULL or [M, r] (T_i = X L1_i, as qlora_linear_fwd's T_out).
 *   W_i [N_i, K] with the same K; Y_i [M, N_i]; other shapes and limits as qlora_linear_fwd.
 *   workspace: >= qlora_multi_workspace_size(n, N, K, M, r) bytes (N: HOST array of the N_i).
 * From 1024 tokens, when every N_i but the last is a multiple of 256, the weights are expanded
 * into one combined weight [sum N_i, K] and the n
 * products run as one bf16 GEMM whose tiles pick their adapter and output by column range;
 * otherwise the n forwards run as qlora_linear_fwd calls.  Either way Y_i and T_i equal
 * qlora_linear_fwd's bit for bit.  The backward of each linear is qlora_linear_bwd (with
 * QLORA_DX_ACCUMULATE for the second and third, to sum their dX).
 */
size_t qlora_multi_workspace_size(int32_t n, const int64_t *N, int64_t K, int64_t M, int32_t r);
int qlora_multi_fwd(int32_t n, const nf4_weight *const *w, const uint16_t *X, const uint16_t *const *L1,
                    const uint16_t *const *L2, float scale, int64_t M, int32_t r, uint16_t *const *Y,
                    uint16_t *const *T_out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * QLoRA linear backward/*
 * QLoRA linear backward -- section 3.5: only the adapters get gradients (dE/dL1, dE/dL2) and
 * the gradient flows to X through the BF16-dequantized frozen weight; W is never written.
 *   dT  = s dY L2^T          dL2 = s T^T dY  (T = X L1)
 *   dL1 = X^T dT             dX  = dY deq(W) + dT L1^T
 *   dY: [M, N] bf16; X: [M, K]; L1: [K, r]; L2: [r, N]; T: [M, r] from the forward or NULL
 *   (then recomputed).  dX: [M, K] bf16 or NULL (not computed); dL1: [K, r]; dL2: [r, N]; all
 *   bf16, fp32 accumulation.  flags: QLORA_DX_ACCUMULATE adds into dX instead of overwriting.
 *   dL1 and dL2 are overwritten.  Same shape limits and workspace query as the forward.
 */
#define QLORA_DX_ACCUMULATE 1u
int qlora_linear_bwd(const nf4_weight *w, const uint16_t *dY, const uint16_t *X,
                     const uint16_t *L1, const uint16_t *L2, const uint16_t *T, float scale,
                     int64_t M, int32_t r, uint16_t *dX, uint16_t *dL1, uint16_t *dL2,
                     uint32_t flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * SwiGLU glue for gated MLPs built from three such linears (not a step of the method):
 *   h = silu(g) * u, silu(g) = g * sigmoid(g);  dg = dh * u * sigmoid(g) * (1 + g (1 - sigmoid(g))),
 *   du = dh * silu(g).  All bf16 [n], fp32 arithmetic, 16-byte aligned, n >= 0.
 */
int qlora_swiglu_fwd(const uint16_t *g, const uint16_t *u, uint16_t *h, int64_t n, void *stream);

/*
 * Gated MLP forward: the gate and up linears of a LLaMA MLP block, each a QLoRA linear of
 * section 3.5 eq. (5) with its own adapter (LoRA on every linear: section 4), and the SwiGLU glue:
 *   G = X deq(W_gate)^T + s (X L1_gate) L2_gate;  U likewise with W_up;  H = silu(G) U.
 *   w_gate, w_up: weights of the same shape [F, K];  X: [M, K];  L1_*: [K, r];  L2_*: [r, F];
 *   G, U, H: [M, F] bf16 (G and U are kept for the backward of the glue);  T_gate_out,
 *   T_up_out: optional [M, r] (X L1, unscaled), as qlora_linear_fwd's T_out.
 *   workspace: >= qlora_gated_workspace_size(M, F, K, r) bytes (forward and backward).
 *   Limits as qlora_linear_fwd.
 * Gate and up run as qlora_multi_fwd (one bf16 GEMM over both weights from 1024 tokens when F is a
 * multiple of 256), then the glue; G and U equal qlora_linear_fwd's outputs and H equals
 * qlora_swiglu_fwd(G, U) bit for bit.  flags: 0 or QLORA_GATED_FUSE, which selects the backward's
 * fused product and changes nothing here (a forward with the glue in the product's epilogue
 * measured about 9 % slower than this and was removed).  Other flag bits: NF4_ERR_ARG.
 */
#define QLORA_GATED_FUSE 2u   /* distinct from QLORA_DX_ACCUMULATE */
size_t qlora_gated_workspace_size(int64_t M, int64_t F, int64_t K, int32_t r);
int qlora_gated_fwd(const nf4_weight *w_gate, const nf4_weight *w_up, const uint16_t *X,
                    const uint16_t *L1_gate, const uint16_t *L2_gate, const uint16_t *L1_up,
                    const uint16_t *L2_up, float scale, int64_t M, int32_t r, uint16_t *G, uint16_t *U,
                    uint16_t *H, uint16_t *T_gate_out, uint16_t *T_up_out, uint32_t flags,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Gated MLP backward, the chain rule through the glue and both linears (section 3.5: gradients
 * for the adapters and for X only, through the BF16 weights):
 *   dG, dU = the glue's backward of dH at (G, U);  then for A in {gate, up} with dA = dG, dU:
 *   dT_A = s dA L2_A^T;  dL2_A = s T_A^T dA;  dL1_A = X^T dT_A;
 *   dX = dG deq(W_gate) + dT_gate L1_gate^T + dU deq(W_up) + dT_up L1_up^T.
 *   dH, G, U: [M, F] (G and U from qlora_gated_fwd);  T_gate, T_up: [M, r] from the forward or
 *   NULL (recomputed);  dX: [M, K] or NULL (not computed);  dL1_*: [K, r];  dL2_*: [r, F].
 *   flags: QLORA_DX_ACCUMULATE adds into dX.  QLORA_GATED_FUSE (from 1024 tokens) computes dX as
 *   one bf16 GEMM whose reduction runs over both weights, [dG | dU] [deq(W_gate) ; deq(W_up)]
 *   plus both LoRA terms, rounded to bf16 once (about 1.5 % faster at the LLaMA-7B MLP shape);
 *   without it the two linears' backward run as qlora_linear_bwd calls, the second adding into
 *   dX.  dL1_* and dL2_* are the same bits either way.
 *   workspace: >= qlora_gated_workspace_size(M, F, K, r) bytes (covers both directions).
 */
int qlora_gated_bwd(const nf4_weight *w_gate, const nf4_weight *w_up, const uint16_t *dH,
                    const uint16_t *X, const uint16_t *G, const uint16_t *U, const uint16_t *L1_gate,
                    const uint16_t *L2_gate, const uint16_t *L1_up, const uint16_t *L2_up,
                    const uint16_t *T_gate, const uint16_t *T_up, float scale, int64_t M, int32_t r,
                    uint16_t *dX, uint16_t *dL1_gate, uint16_t *dL2_gate, uint16_t *dL1_up,
                    uint16_t *dL2_up, uint32_t flags, void *workspace, size_t workspace_bytes,
                    void *stream);
int qlora_swiglu_bwd(const uint16_t *dh, const uint16_t *g, const uint16_t *u, uint16_t *dg,
                     uint16_t *du, int64_t n, void *stream);

/*
 * Timing instrumentation (not part of the method).  While set on the calling thread, the library
 * records begin[i] and end[i] (hipEvent_t handles created by the caller) on the launch stream
 * immediately before and after the i-th subsequent launch of an instrumented kernel -- the
 * matrix products of the linear layer (forward and backward, fused-dequant or expanded-weight),
 * the gated MLP's products and the weight-streaming GEMV main kernels -- for i < n; launches
 * beyond n are not recorded.
 * nf4_gemm_timing_count() returns how many launches were recorded since the last set call.
 * Pass n = 0 to switch it off.  kinds (output, optional): for each recorded launch, 0 = forward
 * GEMM, 1 = backward GEMM (dX), 2 = GEMV, 3 = gated forward GEMM (gate and up as one product),
 * 4 = gated backward GEMM (dX over both weights).
 */
int nf4_set_gemm_timing_events(void **begin, void **end, int32_t *kinds, int32_t n);
int32_t nf4_gemm_timing_count(void);

#ifdef __cplusplus
}
#endif

#endif /* NF4_H */
