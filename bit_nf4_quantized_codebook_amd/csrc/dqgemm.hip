// Fused double-dequantize + bf16 MFMA GEMM for the QLoRA linear layer (gfx950).
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (5) (forward), eq. (6) (double dequantization to BF16) and the backward
// description (gradient to X through the BF16 weight only); section 4 eq. (3) (scalar s).
//
// Two orientations of one kernel:
//   forward  Y  = X  . deq(W)^T + (sT) . L2        reduction over K, output cols = W rows
//   backward dX = dY . deq(W)   + dT  . L1^T       reduction over N, output cols = W cols
// The LoRA product is appended as extra reduction steps ("K-extension"): A' = [A | Ae] and
// B' = [deq(W) ; Be], so it costs r/64 more steps of the same MFMA loop and no extra pass.
//
// Block tile 256 x 256 outputs, reduction step 64, 4 waves in 2 x 2, each wave 128 x 128 with
// v_mfma_f32_32x32x16_bf16 (4 x 4 tiles, 256 fp32 accumulators per lane).  Both operands are
// staged in LDS as bf16 rows of 64 reduction elements padded to 72 (bank-conflict free 16-byte
// fragment reads), double buffered (144 KB of the 160 KB LDS).  The packed 4-bit W tile is read
// from global memory once per block tile and dequantized by all 256 threads straight into the
// LDS B tile: a' = fma(e4m3(c2), c1, mean) per (row, 64-block), w = bf16(cb[code] * a') with the
// 16 codewords read from a 64-byte LDS table (16 distinct words: no bank conflicts).
//  - forward: a thread owns one W row (one 64-block per step) and writes 8 x 16 bytes.
//  - backward: a thread owns an 8 x 8 (rows x cols) nibble block and writes its transpose,
//    8 reduction values per output column, so fragments stay contiguous along the reduction.

#include "common.h"
#include "launch.h"

namespace nf4k {

namespace {

constexpr int TM = 256;          // output rows per block tile
constexpr int TN = 256;          // output cols per block tile
constexpr int TK = 64;           // reduction per step (= one quantization block)
constexpr int LDSK = TK + 8;     // padded LDS row, bf16 elements (144 bytes)
constexpr int NTHREADS = 256;

struct GemmArgs {
    const uint16_t *A;       // [M, Kred] bf16
    const uint8_t *packed;   // W codes [wrows, wcols/2]
    const uint8_t *c2;       // E4M3 block constants
    const float *c1;         // 256-block multipliers
    const float *mean;       // [1]
    const uint16_t *Ae;      // [M, r] bf16 (extension A)
    const uint16_t *Be;      // [Nout, r] bf16 (extension B, row = output column)
    uint16_t *C;             // [M, Nout] bf16
    int64_t M, Nout, Kred;
    int64_t wrows, wcols;
    int32_t r;
    uint32_t accumulate;
    Codebook cb;
};

__device__ __forceinline__ u32x4 ldg16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Tile index -> (tm, tn), keeping each XCD (blockIdx % 8) on a contiguous run of tiles so that
// the tiles sharing A rows land on the same L2.
__device__ __forceinline__ void tile_coords(int ntm, int ntn, int &tm, int &tn) {
    const int nt = ntm * ntn;
    const int bid = blockIdx.x;
    const int q = nt / 8;
    int t = bid;
    if (bid < 8 * q) t = (bid % 8) * q + bid / 8;
    tm = t / ntn;
    tn = t % ntn;
}

template <bool BWD>
__global__ __launch_bounds__(NTHREADS, 1) void dqgemm_kernel(GemmArgs g) {
    extern __shared__ __align__(16) uint16_t smem[];
    uint16_t *As = smem;                              // [2][TM][LDSK]
    uint16_t *Bs = smem + 2 * TM * LDSK;              // [2][TN][LDSK]
    float *cbs = reinterpret_cast<float *>(smem + 2 * (TM + TN) * LDSK);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    if (tid < 16) cbs[tid] = g.cb.v[tid];

    const int ntm = (int)((g.M + TM - 1) / TM);
    const int ntn = (int)((g.Nout + TN - 1) / TN);
    int tm, tn;
    tile_coords(ntm, ntn, tm, tn);
    const int64_t m0 = (int64_t)tm * TM;
    const int64_t o0 = (int64_t)tn * TN;

    const int main_steps = (int)((g.Kred + TK - 1) / TK);
    const int ext_steps = (g.r + TK - 1) / TK;
    const int nsteps = main_steps + ext_steps;

    const float mean = g.mean[0];
    const int64_t wblk_per_row = g.wcols >> 6;

    // ---- register staging for one step ----
    // areg: A tile, 8 x 16 bytes per thread.
    // bbuf: extension B tile (8 x 16 bytes), or the packed W bytes and their block constants:
    //   forward  bbuf[0..1] = 32 packed bytes of one row, bbuf[2].x = E4M3 code, .y = c1 bits
    //   backward bbuf[0..1] = 8 rows x 4 packed bytes, bbuf[2..3] = 8 codes, bbuf[4..5] = 8 c1 bits
    u32x4 areg[8];
    u32x4 bbuf[8];

    auto gload = [&](int step) {
        const bool ext = step >= main_steps;
        // A operand: rows m0.., 64 reduction columns
        const uint16_t *Abase = ext ? g.Ae : g.A;
        const int64_t lda = ext ? (int64_t)g.r : g.Kred;
        const int64_t kcol0 = ext ? (int64_t)(step - main_steps) * TK : (int64_t)step * TK;
        const int64_t klim = ext ? (int64_t)g.r : g.Kred;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int c = tid + NTHREADS * q;
            const int row = c >> 3, seg = c & 7;
            const int64_t gm = m0 + row, gk = kcol0 + seg * 8;
            if (gm < g.M && gk < klim) areg[q] = ldg16(Abase + gm * lda + gk);
            else areg[q] = u32x4{0, 0, 0, 0};
        }
        if (ext) {
            // B extension rows are output columns, r-contiguous
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int c = tid + NTHREADS * q;
                const int row = c >> 3, seg = c & 7;
                const int64_t go = o0 + row, gk = kcol0 + seg * 8;
                if (go < g.Nout && gk < (int64_t)g.r) bbuf[q] = ldg16(g.Be + go * g.r + gk);
                else bbuf[q] = u32x4{0, 0, 0, 0};
            }
            return;
        }
        if (!BWD) {
            // thread owns W row n = o0 + tid, bytes [step*32, step*32+32)
            const int64_t n = o0 + tid;
            if (n < g.wrows) {
                const uint8_t *p = g.packed + n * (g.wcols >> 1) + (int64_t)step * 32;
                bbuf[0] = ldg16(p);
                bbuf[1] = ldg16(p + 16);
                const int64_t b = n * wblk_per_row + step;
                bbuf[2].x = g.c2[b];
                bbuf[2].y = __float_as_uint(g.c1[b >> 8]);
            } else {
                bbuf[0] = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
                bbuf[1] = bbuf[0];
                bbuf[2].x = 0;
                bbuf[2].y = 0;
            }
        } else {
            // thread owns rows n0+8*ng .. +7 (reduction) x cols k0+8*kg .. +7 (output)
            const int kg = tid >> 3, ng = tid & 7;
            const int64_t kcol = o0 + kg * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int64_t n = (int64_t)step * TK + ng * 8 + i;
                uint32_t wv = 0x77777777u, cv = 0, sv = 0;
                if (n < g.wrows && kcol < g.wcols) {
                    wv = *reinterpret_cast<const uint32_t *>(g.packed + n * (g.wcols >> 1) + (kcol >> 1));
                    const int64_t b = n * wblk_per_row + (kcol >> 6);
                    cv = g.c2[b];
                    sv = __float_as_uint(g.c1[b >> 8]);
                }
                bbuf[i >> 2][i & 3] = wv;
                bbuf[2 + (i >> 2)][i & 3] = cv;
                bbuf[4 + (i >> 2)][i & 3] = sv;
            }
        }
    };

    auto swrite = [&](int step, int st) {
        const bool ext = step >= main_steps;
        uint16_t *Ad = As + st * TM * LDSK;
        uint16_t *Bd = Bs + st * TN * LDSK;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int c = tid + NTHREADS * q;
            const int row = c >> 3, seg = c & 7;
            *reinterpret_cast<u32x4 *>(Ad + row * LDSK + seg * 8) = areg[q];
        }
        if (ext) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int c = tid + NTHREADS * q;
                const int row = c >> 3, seg = c & 7;
                *reinterpret_cast<u32x4 *>(Bd + row * LDSK + seg * 8) = bbuf[q];
            }
            return;
        }
        if (!BWD) {
            const float a = block_scale(bbuf[2].x, __uint_as_float(bbuf[2].y), mean);
            uint32_t words[8] = {bbuf[0].x, bbuf[0].y, bbuf[0].z, bbuf[0].w,
                                 bbuf[1].x, bbuf[1].y, bbuf[1].z, bbuf[1].w};
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const uint32_t w = words[d];
                u32x4 o;
                o.x = pack_bf16x2(cbs[w & 15u] * a, cbs[(w >> 4) & 15u] * a);
                o.y = pack_bf16x2(cbs[(w >> 8) & 15u] * a, cbs[(w >> 12) & 15u] * a);
                o.z = pack_bf16x2(cbs[(w >> 16) & 15u] * a, cbs[(w >> 20) & 15u] * a);
                o.w = pack_bf16x2(cbs[(w >> 24) & 15u] * a, cbs[(w >> 28) & 15u] * a);
                *reinterpret_cast<u32x4 *>(Bd + tid * LDSK + d * 8) = o;
            }
        } else {
            const int kg = tid >> 3, ng = tid & 7;
            float a[8];
            uint32_t wreg[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                a[i] = block_scale(bbuf[2 + (i >> 2)][i & 3], __uint_as_float(bbuf[4 + (i >> 2)][i & 3]), mean);
                wreg[i] = bbuf[i >> 2][i & 3];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int sh = 4 * j;
                u32x4 o;
                o.x = pack_bf16x2(cbs[(wreg[0] >> sh) & 15u] * a[0], cbs[(wreg[1] >> sh) & 15u] * a[1]);
                o.y = pack_bf16x2(cbs[(wreg[2] >> sh) & 15u] * a[2], cbs[(wreg[3] >> sh) & 15u] * a[3]);
                o.z = pack_bf16x2(cbs[(wreg[4] >> sh) & 15u] * a[4], cbs[(wreg[5] >> sh) & 15u] * a[5]);
                o.w = pack_bf16x2(cbs[(wreg[6] >> sh) & 15u] * a[6], cbs[(wreg[7] >> sh) & 15u] * a[7]);
                *reinterpret_cast<u32x4 *>(Bd + (kg * 8 + j) * LDSK + ng * 8) = o;
            }
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    auto compute = [&](int st) {
        const uint16_t *Asrc = As + st * TM * LDSK;
        const uint16_t *Bsrc = Bs + st * TN * LDSK;
        const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(Asrc + (wm * 128 + i * 32 + r32) * LDSK + s * 16 + h * 8);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8 *>(Bsrc + (wn * 128 + j * 32 + r32) * LDSK + s * 16 + h * 8);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);   // keep one sub-step of fragments live at a time
        }
    };

    __syncthreads();   // codebook table visible
    gload(0);
    swrite(0, 0);
    __syncthreads();
    for (int step = 0; step < nsteps; ++step) {
        const int st = step & 1;
        const bool more = step + 1 < nsteps;
        if (more) gload(step + 1);
        compute(st);
        if (more) swrite(step + 1, st ^ 1);
        __syncthreads();
    }

    // ---- epilogue: fp32 -> bf16, optional accumulate into C ----
    const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = o0 + wn * 128 + j * 32 + r32;
            if (col >= g.Nout) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + h * 4 + (v & 3);
                if (row < g.M) {
                    uint16_t *p = g.C + row * g.Nout + col;
                    float x = acc[i][j][v];
                    if (g.accumulate) x += bf16_to_f32(*p);
                    *p = (uint16_t)f32_to_bf16(x);
                }
            }
        }
    }
}

constexpr size_t kSmemBytes = (size_t)2 * (TM + TN) * LDSK * sizeof(uint16_t) + 16 * sizeof(float);

template <bool BWD>
hipError_t launch_impl(const GemmArgs &a, hipStream_t stream) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&dqgemm_kernel<BWD>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
    if (e != hipSuccess) return e;
    const int ntm = (int)((a.M + TM - 1) / TM);
    const int ntn = (int)((a.Nout + TN - 1) / TN);
    timing_before(stream, BWD ? 1 : 0);
    hipLaunchKernelGGL(dqgemm_kernel<BWD>, dim3(ntm * ntn), dim3(NTHREADS), kSmemBytes, stream, a);
    e = hipGetLastError();
    timing_after(stream);
    return e;
}

}  // namespace

hipError_t launch_dqgemm_fwd(const WeightView &w, const uint16_t *X, const uint16_t *sT,
                             const uint16_t *L2t, int32_t r, int64_t M, uint16_t *Y,
                             hipStream_t stream) {
    GemmArgs a;
    a.A = X;
    a.packed = w.packed; a.c2 = w.c2; a.c1 = w.c1; a.mean = w.mean;
    a.Ae = sT; a.Be = L2t; a.C = Y;
    a.M = M; a.Nout = w.rows; a.Kred = w.cols;
    a.wrows = w.rows; a.wcols = w.cols;
    a.r = r; a.accumulate = 0;
    for (int j = 0; j < 16; ++j) a.cb.v[j] = w.cb[j];
    return launch_impl<false>(a, stream);
}

hipError_t launch_dqgemm_bwd(const WeightView &w, const uint16_t *dY, const uint16_t *dT,
                             const uint16_t *L1, int32_t r, int64_t M, uint16_t *dX,
                             bool accumulate, hipStream_t stream) {
    GemmArgs a;
    a.A = dY;
    a.packed = w.packed; a.c2 = w.c2; a.c1 = w.c1; a.mean = w.mean;
    a.Ae = dT; a.Be = L1; a.C = dX;
    a.M = M; a.Nout = w.cols; a.Kred = w.rows;
    a.wrows = w.rows; a.wcols = w.cols;
    a.r = r; a.accumulate = accumulate ? 1u : 0u;
    for (int j = 0; j < 16; ++j) a.cb.v[j] = w.cb[j];
    return launch_impl<true>(a, stream);
}

}  // namespace nf4k
