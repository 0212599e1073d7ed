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
    int32_t slot;            // row layout: -1 plain; 0 / 1: rows to 32-row slot 0 / 1 of 64-row groups
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
        int64_t owi = wi;
        if (g.slot >= 0) {
            // gated MLP: gate rows (slot 0) and up rows (slot 1) alternate in groups of 32, so one
            // 32 x 32 MFMA tile of the GEMM holds gate and the next up for the same outputs
            const uint32_t kw = (uint32_t)(g.K >> 3), row = (uint32_t)wi / kw, cw = (uint32_t)wi - row * kw;
            owi = (int64_t)(((row >> 5) << 6) + ((uint32_t)g.slot << 5) + (row & 31u)) * kw + cw;
        }
        __builtin_nontemporal_store(dequant8(t, w), reinterpret_cast<u32x4 *>(g.out) + owi);
    }
}

// Transposed layout, one 64 x 64 tile (64 W rows n0.., one block column kb) per workgroup:
// thread t expands 16 weights of row n0 + t/4 (columns 16 (t%4) ..) into an LDS tile [k][n],
// then writes 16 consecutive n of one output row k.  In the tile, the 16-column group of n is
// XOR-ed with k/16, so the 2-byte writes of the four column groups of a wave land on different
// banks.
constexpr int TROW = 64 + 8;   // LDS row (k) length in bf16, padded
__global__ __launch_bounds__(256) void expand_transposed_kernel(ExpandArgs g) {
    __shared__ uint16_t tile[64 * TROW];
    // the reduction workgroups first, so that they overlap the expansion instead of trailing it
    if (blockIdx.x < g.nred) {
        reduce_partials_block(g.red, blockIdx.x, g.nred);
        return;
    }
    const int64_t tb = blockIdx.x - g.nred;
    const int tid = threadIdx.x;
    const int64_t nbk = g.K >> 6;
    const int64_t ntn = (g.N + 63) >> 6;
    const int64_t kb = tb / ntn;
    const int64_t n0 = (tb % ntn) * 64;
    const float mean = g.mean[0];
    const bool dq_i8 = g.dq_int8 != 0;
    {
        const int nl = tid >> 2, q = tid & 3;
        const int64_t n = n0 + nl;
        uint32_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (n < g.N) {
            const int64_t b = n * nbk + kb;
            const Lut t = make_lut(g.cb, block_scale(g.c2[b], g.c1[b >> 8], mean, dq_i8));
            const uint2 w = *reinterpret_cast<const uint2 *>(g.packed + b * 32 + q * 8);
            const u32x4 lo = dequant8(t, w.x), hi = dequant8(t, w.y);
            v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
            v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) tile[(16 * q + e) * TROW + (nl ^ (16 * q))] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
    {
        const int kl = tid >> 2, q = tid & 3;
        const int64_t k = kb * 64 + kl;
        const int64_t n = n0 + 16 * q;
        const u32x4 *s = reinterpret_cast<const u32x4 *>(tile + kl * TROW + 16 * (q ^ ((kl >> 4) & 3)));
        const u32x4 a = s[0], c = s[1];
        uint16_t *dst = g.out + k * g.N + n;
        // plain stores: the four 32-byte pieces of a 128-byte row segment combine in L2
        if (n + 16 <= g.N) {
            reinterpret_cast<u32x4 *>(dst)[0] = a;
            reinterpret_cast<u32x4 *>(dst)[1] = c;
        } else {
            // N % 8 == 0: the last tile ends on an 8-column boundary
            if (n < g.N) reinterpret_cast<u32x4 *>(dst)[0] = a;
        }
    }
}

}  // namespace

hipError_t launch_expand_weight(const WeightView &w, bool transposed, uint16_t *out, const Reduction *red,
                                hipStream_t stream, int slot, const uint16_t *tr_in, uint16_t *tr_out,
                                int32_t tr_r, int64_t tr_n) {
    ExpandArgs a;
    a.slot = transposed ? -1 : slot;
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
        a.nexp = (uint32_t)(((w.rows + 63) / 64) * (w.cols / 64));
        hipLaunchKernelGGL(expand_transposed_kernel, dim3(a.nexp + a.nred), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace nf4k
