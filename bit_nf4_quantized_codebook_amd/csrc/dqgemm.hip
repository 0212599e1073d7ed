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

// Buffer resource over [base, base + bytes): loads past the end return zeros, so tile edges need
// no branches (a branch that zero-fills a register with a load in flight forces a full wait).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int64_t clamped = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0LL ? 0x7FFFFFF0LL : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)clamped, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t bload1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
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

    const float mean = g.mean[0];
    const int64_t wblk_per_row = g.wcols >> 6;
    const int64_t wrow_bytes = g.wcols >> 1;

    // tile-relative buffer descriptors: reads past the end return zeros (no edge branches)
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A + m0 * g.Kred, (g.M - m0) * g.Kred * 2);
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(g.packed, g.wrows * wrow_bytes);
    const __amdgpu_buffer_rsrc_t rC2 = make_rsrc(g.c2, g.wrows * wblk_per_row);
    const __amdgpu_buffer_rsrc_t rC1 = make_rsrc(g.c1, ((g.wrows * wblk_per_row + 255) >> 8) * 4);

    // A tile: chunk q of this thread covers row (tid >> 3) + 32 q, 8 reduction elements at seg
    const int arow = tid >> 3, aseg = tid & 7;
    const uint32_t a_off0 = (uint32_t)((arow * g.Kred + aseg * 8) * 2);
    const uint32_t a_rowstep = (uint32_t)(32 * g.Kred * 2);
    const bool a_tail = (g.Kred % TK) != 0;     // only the backward reduction (N) can be ragged

    // W: forward thread owns row o0+tid; backward owns rows 8*ng.. x cols o0+8*kg..
    const int kg = tid >> 3, ng = tid & 7;
    int64_t w_row;            // forward: the W row; backward: the first reduction row of this thread
    uint32_t w_off0, c2_off0;
    if (!BWD) {
        w_row = o0 + tid;
        w_off0 = (uint32_t)(w_row * wrow_bytes);
        c2_off0 = (uint32_t)(w_row * wblk_per_row);
    } else {
        w_row = ng * 8;
        const int64_t kcol = o0 + kg * 8;
        w_off0 = (uint32_t)(w_row * wrow_bytes + (kcol >> 1));
        c2_off0 = (uint32_t)(w_row * wblk_per_row + (kcol >> 6));
    }

    struct Stage {
        u32x4 a[8];
        u32x4 w[2];        // forward: 32 packed bytes; backward: 8 rows x 4 bytes
        uint32_t c2[8];
        uint32_t c1[8];
    };

    // Loads of one step into a register stage.  Never behind a branch: a step past the end
    // (prefetch beyond the last step) reads out of range, i.e. zeros, so the memory-counter
    // waits stay exact across the software-pipelined loop.
    auto gload = [&](int step, Stage &sg) {
        const bool live = step < main_steps;
        const uint32_t kb = (uint32_t)step * TK * 2;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            uint32_t off = a_off0 + q * a_rowstep + kb;
            if (!live || (a_tail && (int64_t)step * TK + aseg * 8 >= g.Kred)) off = 0xFFFFFFF0u;
            sg.a[q] = bload16(rA, off);
        }
        if (!BWD) {
            const uint32_t off = live ? w_off0 + (uint32_t)step * 32 : 0xFFFFFFE0u;
            sg.w[0] = bload16(rW, off);
            sg.w[1] = bload16(rW, off + 16);
            const uint32_t b = live ? c2_off0 + (uint32_t)step : 0xFFFFFFF0u;
            sg.c2[0] = bload1(rC2, b);
            sg.c1[0] = bload4(rC1, live ? (b >> 8) * 4 : 0xFFFFFFF0u);
        } else {
            const uint32_t rstep = (uint32_t)((int64_t)step * TK * wrow_bytes);
            const uint32_t bstep = (uint32_t)((int64_t)step * TK * wblk_per_row);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t wo = w_off0 + rstep + (uint32_t)(i * wrow_bytes);
                sg.w[i >> 2][i & 3] = bload4(rW, live ? wo : 0xFFFFFFF0u);
                const uint32_t b = c2_off0 + bstep + (uint32_t)(i * wblk_per_row);
                sg.c2[i] = bload1(rC2, live ? b : 0xFFFFFFF0u);
                sg.c1[i] = bload4(rC1, live ? (b >> 8) * 4 : 0xFFFFFFF0u);
            }
        }
    };

    // part `part` (0..3) of writing a loaded step into LDS stage st: A chunks 2*part, 2*part+1
    // and a quarter of the dequantized B tile
    auto swrite_part = [&](int step, const Stage &sg, int st, int part, float *scl) {
        uint16_t *Ad = As + st * TM * LDSK;
        uint16_t *Bd = Bs + st * TN * LDSK;
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int q = part * 2 + qq;
            *reinterpret_cast<u32x4 *>(Ad + (arow + 32 * q) * LDSK + aseg * 8) = sg.a[q];
        }
        if (!BWD) {
            if (part == 0) scl[0] = block_scale(sg.c2[0], __uint_as_float(sg.c1[0]), mean);
            const float a = scl[0];
#pragma unroll
            for (int dd = 0; dd < 2; ++dd) {
                const int d = part * 2 + dd;
                const uint32_t w = sg.w[d >> 2][d & 3];
                u32x4 o;
                o.x = pack_bf16x2(cbs[w & 15u] * a, cbs[(w >> 4) & 15u] * a);
                o.y = pack_bf16x2(cbs[(w >> 8) & 15u] * a, cbs[(w >> 12) & 15u] * a);
                o.z = pack_bf16x2(cbs[(w >> 16) & 15u] * a, cbs[(w >> 20) & 15u] * a);
                o.w = pack_bf16x2(cbs[(w >> 24) & 15u] * a, cbs[(w >> 28) & 15u] * a);
                *reinterpret_cast<u32x4 *>(Bd + tid * LDSK + d * 8) = o;
            }
        } else {
            if (part == 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int64_t n = (int64_t)step * TK + w_row + i;
                    const float a = block_scale(sg.c2[i], __uint_as_float(sg.c1[i]), mean);
                    scl[i] = (n < g.wrows) ? a : 0.0f;     // reduction rows past N contribute 0
                }
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int j = part * 2 + jj;
                const int sh = 4 * j;
                u32x4 o;
                o.x = pack_bf16x2(cbs[(sg.w[0].x >> sh) & 15u] * scl[0], cbs[(sg.w[0].y >> sh) & 15u] * scl[1]);
                o.y = pack_bf16x2(cbs[(sg.w[0].z >> sh) & 15u] * scl[2], cbs[(sg.w[0].w >> sh) & 15u] * scl[3]);
                o.z = pack_bf16x2(cbs[(sg.w[1].x >> sh) & 15u] * scl[4], cbs[(sg.w[1].y >> sh) & 15u] * scl[5]);
                o.w = pack_bf16x2(cbs[(sg.w[1].z >> sh) & 15u] * scl[6], cbs[(sg.w[1].w >> sh) & 15u] * scl[7]);
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

    const int r32 = lane & 31, hh = lane >> 5;
    auto mfma_sub = [&](int st, int s) {
        const uint16_t *Asrc = As + st * TM * LDSK;
        const uint16_t *Bsrc = Bs + st * TN * LDSK;
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const bf16x8 *>(Asrc + (wm * 128 + i * 32 + r32) * LDSK + s * 16 + hh * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8 *>(Bsrc + (wn * 128 + j * 32 + r32) * LDSK + s * 16 + hh * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };

    // ---- main loop ----
    // LDS stages alternate per step.  Two register stages alternate too: the loads for step+2 are
    // issued at the start of step (a full step of latency to hide), while the data of step+1 is
    // dequantized into the other LDS stage in four parts interleaved with the four MFMA sub-steps.
    __syncthreads();   // codebook table visible
    float scl[8];
    Stage R0, R1;
    gload(0, R0);
#pragma unroll
    for (int part = 0; part < 4; ++part) swrite_part(0, R0, 0, part, scl);
    gload(1, R1);
    __syncthreads();
    int step = 0;
    for (; step + 1 < main_steps; step += 2) {
        // even step: compute LDS stage 0, fill stage 1 with step+1 from R1
        gload(step + 2, R0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            mfma_sub(0, s);
            swrite_part(step + 1, R1, 1, s, scl);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
        // odd step: compute stage 1, fill stage 0 with step+2 from R0 (zeros past the end;
        // stage 0 is only read again if step+2 is a real step)
        gload(step + 3, R1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            mfma_sub(1, s);
            swrite_part(step + 2, R0, 0, s, scl);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();
    }
    if (step < main_steps) {   // odd number of steps: the last one sits in stage 0
#pragma unroll
        for (int s = 0; s < 4; ++s) mfma_sub(0, s);
        __syncthreads();
    }

    // ---- LoRA extension: [A | Ae] . [B ; Be], r/64 more steps (operands zero padded) ----
    if (ext_steps > 0) {
        const __amdgpu_buffer_rsrc_t rAe = make_rsrc(g.Ae + m0 * g.r, (g.M - m0) * (int64_t)g.r * 2);
        const __amdgpu_buffer_rsrc_t rBe = make_rsrc(g.Be + o0 * g.r, (g.Nout - o0) * (int64_t)g.r * 2);
        for (int e = 0; e < ext_steps; ++e) {
            const int st = (main_steps + e) & 1;
            uint16_t *Ad = As + st * TM * LDSK;
            uint16_t *Bd = Bs + st * TN * LDSK;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int row = arow + 32 * q;
                const int64_t gk = (int64_t)e * TK + aseg * 8;
                const bool ok = gk < g.r;
                const u32x4 va = bload16(rAe, ok ? (uint32_t)((row * (int64_t)g.r + gk) * 2) : 0xFFFFFFF0u);
                const u32x4 vb = bload16(rBe, ok ? (uint32_t)((row * (int64_t)g.r + gk) * 2) : 0xFFFFFFF0u);
                *reinterpret_cast<u32x4 *>(Ad + row * LDSK + aseg * 8) = va;
                *reinterpret_cast<u32x4 *>(Bd + row * LDSK + aseg * 8) = vb;
            }
            __syncthreads();
#pragma unroll
            for (int s = 0; s < 4; ++s) mfma_sub(st, s);
            __syncthreads();
        }
    }

    // ---- epilogue: fp32 -> bf16, optional accumulate into C ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = o0 + wn * 128 + j * 32 + r32;
            if (col >= g.Nout) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm * 128 + i * 32 + (v >> 2) * 8 + hh * 4 + (v & 3);
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
