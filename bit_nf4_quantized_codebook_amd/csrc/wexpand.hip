// Double dequantization of the whole frozen weight to bf16, as the operand of the bf16 GEMM used
// at large token counts (gfx950).  Two layouts:
//   rows:       out [N, K] = deq(W)      (the forward reads W rows along the reduction)
//   transposed: out [K, N] = deq(W)^T    (the backward reduces over N)
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (6): w = bf16(cb[code] * a'), a' = fma(e4m3(c2), c1, mean), one rounding.
//
// Each 64-weight block builds its 16-entry bf16 table once (16 products, 8 conversions) and
// expands its codes with v_perm_b32 byte selects; the kernels are bound by HBM (0.5 B read and
// 2 B written per weight).

#include "common.h"
#include "dqtile.h"
#include "launch.h"
#include "reduce.h"

namespace nf4k {

namespace {

// nexp workgroups expand the weight; nred more (optional) sum a set of split-reduction partials
// that the caller needs at the same point of the stream, and (rows layout) ntr more transpose a
// small matrix; these short jobs take the lowest workgroup indices, so they run alongside the
// expansion rather than after it
struct ExpandArgs {
    const uint8_t *packed;
    const uint8_t *c2;
    const float *c1;
    const float *mean;
    uint32_t dq_int8;        // second-level codes are int8 (else E4M3)
    uint16_t *out;
    int64_t N, K;
    Codebook cb;
    RedProb red;
    uint32_t nexp, nred;
    // ntr more (optional, rows layout): transpose tr_in [tr_r, tr_n] into tr_out [tr_n, tr_r] (bf16)
    const uint16_t *tr_in;
    uint16_t *tr_out;
    int32_t tr_r;
    int64_t tr_n;
    uint32_t ntr;
};

// One 64 x 64 tile of the small transpose per workgroup (L2 [r, N] -> [N, r] for the GEMM's LoRA
// step, so that it loads like the backward's L1).  Thread t loads two 16-byte pieces of row t / 4
// of the tile (columns 16 (t % 4) ..), and stores two 16-byte pieces of output row t / 4; r and
// N are multiples of 8, so no piece straddles an edge.
__device__ __forceinline__ void transpose_block(const ExpandArgs &g, int64_t blk) {
    __shared__ uint16_t tt[64][64 + 8];
    const int64_t ncb = (g.tr_n + 63) / 64;
    const int64_t j0 = (blk / ncb) * 64, n0 = (blk % ncb) * 64;
    const int t = threadIdx.x, row = t >> 2, c0 = (t & 3) * 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t j = j0 + row, n = n0 + c0 + 8 * h;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j < g.tr_r && n < g.tr_n) v = *reinterpret_cast<const u32x4 *>(g.tr_in + j * g.tr_n + n);
        *reinterpret_cast<u32x4 *>(&tt[row][c0 + 8 * h]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t n = n0 + row, j = j0 + c0 + 8 * h;
        if (n < g.tr_n && j < g.tr_r) {
            uint32_t w[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                w[k] = (uint32_t)tt[c0 + 8 * h + 2 * k][row] | ((uint32_t)tt[c0 + 8 * h + 2 * k + 1][row] << 16);
            *reinterpret_cast<u32x4 *>(g.tr_out + n * g.tr_r + j) = u32x4{w[0], w[1], w[2], w[3]};
        }
    }
}

// Row layout: 8 lanes per block, one packed dword (8 weights) each, so a wave reads 256
// contiguous packed bytes and writes 1 KB of contiguous bf16 per store.  The 8 lanes of a block
// each build its table (the kernel is bound by HBM, not VALU).  Blocks run over the row-major
// flattening, so this needs only N*K % 64 == 0.
// Workgroups: the ntr transpose tiles and the nred reduction workgroups first (short jobs that
// then overlap the expansion instead of trailing it), the nexp expansion workgroups after them.
__global__ __launch_bounds__(256) void expand_rows_kernel(ExpandArgs g) {
    if (blockIdx.x < g.ntr) {
        transpose_block(g, blockIdx.x);
        return;
    }
    if (blockIdx.x < g.ntr + g.nred) {
        reduce_partials_block(g.red, blockIdx.x - g.ntr, g.nred);
        return;
    }
    const int64_t eb = blockIdx.x - g.ntr - g.nred;
    const int64_t nwords = (g.N * g.K) >> 3;
    const float mean = g.mean[0];
    const bool dq_i8 = g.dq_int8 != 0;
    for (int64_t wi = eb * 256 + threadIdx.x; wi < nwords; wi += (int64_t)g.nexp * 256) {
        const int64_t b = wi >> 3;
        const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(g.packed) + wi);
        const Lut t = make_lut(g.cb, block_scale(g.c2[b], g.c1[b >> 8], mean, dq_i8));
        __builtin_nontemporal_store(dequant8(t, w), reinterpret_cast<u32x4 *>(g.out) + wi);
    }
}

// Transposed layout, one tile of 128 W rows (n0 ..) by 256 W columns (4 blocks, k0 ..) per
// workgroup.  Thread t decodes block q = t % 4 of W rows n0 + 2p and n0 + 2p + 1 (p = t / 4): its
// 4 threads per row pair read each row's 128 packed bytes as one line.  It writes the bf16 pairs
// (w[n][k], w[n+1][k]) of its 64 columns into an LDS tile [256 k][64 pairs]; then 16 lanes write
// each output row k (128 n, 256 bytes) with 16-byte stores.  In the tile, the 16-byte group of 4
// pairs is XOR-ed with 4 (k / 64): the 4-byte writes of a wave (16 row pairs x 4 blocks at one
// column offset) then land on 64 different banks, and the 16 lanes reading one row take 16
// different groups.  N % 8 == 0, so an 8-column output group is wholly inside or outside N.
constexpr int TT_N = 128;        // W rows per tile (output columns)
constexpr int TT_K = 256;        // W columns per tile (output rows): 4 blocks
__global__ __launch_bounds__(256) void expand_transposed_kernel(ExpandArgs g) {
    __shared__ __align__(16) uint32_t tile[TT_K * (TT_N / 2)];   // 64 KB
    // the reduction workgroups first, so that they overlap the expansion instead of trailing it
    if (blockIdx.x < g.nred) {
        reduce_partials_block(g.red, blockIdx.x, g.nred);
        return;
    }
    const int64_t tb = blockIdx.x - g.nred;
    const int tid = threadIdx.x;
    const int64_t nbk = g.K >> 6;
    const int64_t ntn = (g.N + TT_N - 1) / TT_N;
    const int64_t kt = tb / ntn;
    const int64_t n0 = (tb % ntn) * TT_N;
    const float mean = g.mean[0];
    const bool dq_i8 = g.dq_int8 != 0;
    {
        const int p = tid >> 2, q = tid & 3;
        const int64_t n = n0 + 2 * p;
        const int64_t kb = kt * 4 + q;
        if (n < g.N && kb < nbk) {      // N is even: row n + 1 exists too
            const int64_t ba = n * nbk + kb, bb = ba + nbk;
            const u32x4 *pa = reinterpret_cast<const u32x4 *>(g.packed + ba * 32);
            const u32x4 *pb = reinterpret_cast<const u32x4 *>(g.packed + bb * 32);
            const u32x4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
            const Lut La = make_lut(g.cb, block_scale(g.c2[ba], g.c1[ba >> 8], mean, dq_i8));
            const Lut Lb = make_lut(g.cb, block_scale(g.c2[bb], g.c1[bb >> 8], mean, dq_i8));
            const uint32_t wa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            const uint32_t wb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            const int grp = (p >> 2) ^ (4 * q), sub = p & 3;
            uint32_t *col = tile + grp * 4 + sub;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const u32x4 ea = dequant8(La, wa[d]), eb = dequant8(Lb, wb[d]);
                const uint32_t ev[4] = {ea.x, ea.y, ea.z, ea.w}, fv[4] = {eb.x, eb.y, eb.z, eb.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kk = 64 * q + 8 * d + 2 * i;
                    col[kk * (TT_N / 2)] = __builtin_amdgcn_perm(fv[i], ev[i], 0x05040100u);
                    col[(kk + 1) * (TT_N / 2)] = __builtin_amdgcn_perm(fv[i], ev[i], 0x07060302u);
                }
            }
        }
    }
    __syncthreads();
    {
        const int c = tid & 15, r16 = tid >> 4;
        const int64_t n = n0 + 8 * c;
#pragma unroll 4
        for (int it = 0; it < TT_K / 16; ++it) {
            const int kk = r16 + 16 * it;
            const int64_t k = kt * TT_K + kk;
            if (k < g.K && n < g.N) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(tile + kk * (TT_N / 2) + ((c ^ (4 * (kk >> 6))) * 4));
                *reinterpret_cast<u32x4 *>(g.out + k * g.N + n) = v;
            }
        }
    }
}

}  // namespace

hipError_t launch_expand_weight(const WeightView &w, bool transposed, uint16_t *out, const Reduction *red,
                                hipStream_t stream, const uint16_t *tr_in, uint16_t *tr_out,
                                int32_t tr_r, int64_t tr_n) {
    ExpandArgs a;
    a.tr_in = tr_in; a.tr_out = tr_out; a.tr_r = tr_r; a.tr_n = tr_n;
    a.ntr = (!transposed && tr_in) ? (uint32_t)(((tr_r + 63) / 64) * ((tr_n + 63) / 64)) : 0u;
    a.packed = w.packed; a.c2 = w.c2; a.c1 = w.c1; a.mean = w.mean; a.dq_int8 = w.dq_int8;
    a.out = out; a.N = w.rows; a.K = w.cols;
    for (int j = 0; j < 16; ++j) a.cb.v[j] = w.cb[j];
    a.nred = 0;
    if (red) a.red = red_prob(*red, a.nred);
    if (!transposed) {
        const int64_t nwords = (w.rows * w.cols) >> 3;
        int64_t grid = (nwords + 255) / 256;
        if (grid > 256 * 64) grid = 256 * 64;
        if (grid < 1) grid = 1;
        a.nexp = (uint32_t)grid;
        hipLaunchKernelGGL(expand_rows_kernel, dim3(a.nexp + a.nred + a.ntr), dim3(256), 0, stream, a);
    } else {
        a.nexp = (uint32_t)(((w.rows + TT_N - 1) / TT_N) * ((w.cols + TT_K - 1) / TT_K));
        hipLaunchKernelGGL(expand_transposed_kernel, dim3(a.nexp + a.nred), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace nf4k
