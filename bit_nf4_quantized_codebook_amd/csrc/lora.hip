// Low-rank (LoRA) side products of the QLoRA linear layer (gfx950).
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 4 eq. (3) (Y = XW + s X L1 L2) and section 3.5 (gradients for L1, L2 only).
//
// Each product is one streaming pass over an [M, K] or [M, N] activation with a rank-r (<= 128)
// partner, so the kernels are built for HBM bandwidth: a block tile is 64 x 64 outputs, the
// reduction is split over enough block tiles to fill the 256 CUs, every thread keeps four
// reduction steps of 16-byte loads in flight, and float32 partials are summed afterwards in a
// fixed order (deterministic).  Operands sit in LDS in their natural row-major layout; when the
// reduction runs along rows, fragments are read with ds_read_b64_tr_b16 (4 x 16 transposes per
// 16-lane group), so no operand is ever transposed in memory.
//   skinny_nt:  P[ks] = A[:, chunk ks] . B          A [M, Kred];  B = Bk [Kred, R] or Bt [R, Kred]
//   skinny_tn:  P[ms] = U[rows ms, :]^T . V[rows ms, :]    U [M, Pn], V [M, Qn]
// MFMA v_mfma_f32_32x32x16_bf16, 4 waves of 32 x 32.

#include "common.h"
#include "dqtile.h"
#include "launch.h"
#include "reduce.h"

namespace nf4k {

namespace {

constexpr int ST = 64;          // block tile (both output dims) and reduction step
constexpr int NSTAGE = 4;       // reduction steps in flight per block tile (skinny_nt)
// skinny_tn: two steps per tile and half the LDS, so four workgroups share a CU and fill each
// other's load waits (dL2 + dL1: 16.6 against 18.9 us at 4096 tokens; skinny_nt gained nothing)
constexpr int NSTAGE_TN = 2;
constexpr int ROWB = (ST + 8) * 2;   // padded LDS row, bytes (144: conflict-free 16-byte reads)


// 16-byte fragment of row `row` (the M/N index), reduction elements 16 s + 8 hh .. +7 of a tile
// stored [row][reduction]
__device__ __forceinline__ bf16x8 frag_rows(const uint8_t *t, int row, int s, int hh) {
    return *reinterpret_cast<const bf16x8 *>(t + row * ROWB + (s * 16 + hh * 8) * 2);
}
// same fragment from a tile stored [reduction][col]: two transposing reads
__device__ __forceinline__ bf16x8 frag_tr(const uint8_t *t, int col0, int s, int lane) {
    const int i16 = lane & 15, hh = lane >> 5, half = (lane >> 4) & 1;
    const int rowb = s * 16 + hh * 8 + (i16 >> 2);
    const uint8_t *base = t + (col0 + half * 16 + 4 * (i16 & 3)) * 2;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + rowb * ROWB));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(base + (rowb + 4) * ROWB));
    const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// Each thread moves 2 x 16 bytes of each 64 x 64 operand tile per step: tile row = tid/8 (+32),
// 16-byte chunk = tid%8.
struct TileLoad {
    u32x4 v[2];
};

// P[ks][m][j] = sum_{k in chunk ks} A[m][k] * B(k, j)
//   B_ROWS_K = true : B given as Bk [Kred, R] (row k), tile stored [k][j] -> transposing reads
//   B_ROWS_K = false: B given as Bt [R, Kred] (row j), tile stored [j][k] -> row reads
template <bool B_ROWS_K>
__global__ __launch_bounds__(256) void skinny_nt_kernel(const uint16_t *__restrict__ A,
                                                        const uint16_t *__restrict__ B,
                                                        float *__restrict__ P, int64_t M, int32_t R,
                                                        int64_t Kred, int64_t kchunk) {
    __shared__ __align__(16) uint8_t As[NSTAGE][ST * ROWB];
    __shared__ __align__(16) uint8_t Bs[NSTAGE][ST * ROWB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, r32 = lane & 31, hh = lane >> 5;
    const int64_t m0 = (int64_t)blockIdx.x * ST;
    const int j0 = blockIdx.y * ST;
    const int64_t kbeg = (int64_t)blockIdx.z * kchunk;
    const int64_t kend = (kbeg + kchunk < Kred) ? kbeg + kchunk : Kred;
    const int nsteps = kend > kbeg ? (int)((kend - kbeg + ST - 1) / ST) : 0;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(A + m0 * Kred, (M - m0) * Kred * 2);
    const __amdgpu_buffer_rsrc_t rB = B_ROWS_K ? make_rsrc(B, Kred * (int64_t)R * 2)
                                               : make_rsrc(B + (int64_t)j0 * Kred, ((int64_t)R - j0) * Kred * 2);
    const int trow = tid >> 3, tch = tid & 7;

    auto load = [&](int step, TileLoad &a, TileLoad &b) {
        const int64_t k0 = kbeg + (int64_t)step * ST;
        const bool live = step < nsteps;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = trow + 32 * h;
            // A: row m0+row, columns k0 + 8 tch; columns past the chunk end read zeros
            const int64_t ka = k0 + tch * 8;
            a.v[h] = bload16(rA, (live && ka < kend) ? (uint32_t)((row * Kred + ka) * 2) : 0xFFFFFFF0u);
            if (B_ROWS_K) {
                // B tile row = k0 + row, columns j0 + 8 tch (j < R)
                const int64_t kb = k0 + row;
                const bool ok = live && kb < kend && j0 + tch * 8 < R;
                b.v[h] = bload16(rB, ok ? (uint32_t)((kb * R + j0 + tch * 8) * 2) : 0xFFFFFFF0u);
            } else {
                // B tile row = j0 + row, columns k0 + 8 tch
                b.v[h] = bload16(rB, (live && ka < kend) ? (uint32_t)((row * Kred + ka) * 2) : 0xFFFFFFF0u);
            }
        }
    };
    auto store = [&](int slot, const TileLoad &a, const TileLoad &b) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = trow + 32 * h;
            *reinterpret_cast<u32x4 *>(&As[slot][row * ROWB + tch * 16]) = a.v[h];
            *reinterpret_cast<u32x4 *>(&Bs[slot][row * ROWB + tch * 16]) = b.v[h];
        }
    };

    f32x16 acc = {};
    TileLoad la[NSTAGE], lb[NSTAGE];
    for (int g0 = 0; g0 < nsteps; g0 += NSTAGE) {
#pragma unroll
        for (int u = 0; u < NSTAGE; ++u) load(g0 + u, la[u], lb[u]);
#pragma unroll
        for (int u = 0; u < NSTAGE; ++u) store(u, la[u], lb[u]);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NSTAGE; ++u) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 fa = frag_rows(As[u], wm * 32 + r32, s, hh);
                const bf16x8 fb = B_ROWS_K ? frag_tr(Bs[u], wn * 32, s, lane)
                                           : frag_rows(Bs[u], wn * 32 + r32, s, hh);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
            }
        }
        __syncthreads();
    }
    const int col = j0 + wn * 32 + r32;
    if (col < R) {
        float *Pk = P + (int64_t)blockIdx.z * M * R;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = m0 + wm * 32 + (v >> 2) * 8 + hh * 4 + (v & 3);
            if (row < M) Pk[row * R + col] = acc[v];
        }
    }
}

// P[ms][p][q] = sum_{m in chunk ms} U[m][p] * V[m][q];  U [M, Pn], V [M, Qn] (row-major).
// Both tiles are stored [m][p] / [m][q] and read with transposing fragment loads.
// One launch serves one or two independent products (the backward runs dL2 and dL1 together):
// blocks [0, nb0) take product 0, the rest product 1; within a product, block b is tile
// (b % tx, (b / tx) % ty) of reduction chunk b / (tx ty).
struct TnProb {
    const uint16_t *U, *V;
    float *P;
    uint16_t *out;           // unsplit: bf16(scale * product) here instead of P
    float scale;
    int64_t Pn, Qn, mchunk;
    int32_t tx, ty;
};
struct TnGroup {
    TnProb p[2];
    int64_t M;
    uint32_t nb0;
};
__global__ __launch_bounds__(256) void skinny_tn_kernel(TnGroup grp) {
    __shared__ __align__(16) uint8_t Us[NSTAGE_TN][ST * ROWB];
    __shared__ __align__(16) uint8_t Vs[NSTAGE_TN][ST * ROWB];
    const int second = blockIdx.x >= grp.nb0;
    const TnProb &pr = grp.p[second];
    const uint16_t *__restrict__ U = pr.U;
    const uint16_t *__restrict__ V = pr.V;
    float *__restrict__ P = pr.P;
    const int64_t M = grp.M, Pn = pr.Pn, Qn = pr.Qn, mchunk = pr.mchunk;
    const uint32_t b = blockIdx.x - (second ? grp.nb0 : 0u);
    const uint32_t bx = b % (uint32_t)pr.tx, by = (b / (uint32_t)pr.tx) % (uint32_t)pr.ty;
    const uint32_t bz = b / ((uint32_t)pr.tx * (uint32_t)pr.ty);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, r32 = lane & 31, hh = lane >> 5;
    const int64_t p0 = (int64_t)bx * ST;
    const int64_t q0 = (int64_t)by * ST;
    const int64_t mbeg = (int64_t)bz * mchunk;
    const int64_t mend = (mbeg + mchunk < M) ? mbeg + mchunk : M;
    const int nsteps = mend > mbeg ? (int)((mend - mbeg + ST - 1) / ST) : 0;
    const __amdgpu_buffer_rsrc_t rU = make_rsrc(U, M * Pn * 2);
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(V, M * Qn * 2);
    const int trow = tid >> 3, tch = tid & 7;
    const bool pok = p0 + tch * 8 < Pn, qok = q0 + tch * 8 < Qn;

    auto load = [&](int step, TileLoad &a, TileLoad &b) {
        const int64_t mm = mbeg + (int64_t)step * ST;
        const bool live = step < nsteps;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t gm = mm + trow + 32 * h;
            const bool ok = live && gm < mend;
            a.v[h] = bload16(rU, (ok && pok) ? (uint32_t)((gm * Pn + p0 + tch * 8) * 2) : 0xFFFFFFF0u);
            b.v[h] = bload16(rV, (ok && qok) ? (uint32_t)((gm * Qn + q0 + tch * 8) * 2) : 0xFFFFFFF0u);
        }
    };
    auto store = [&](int slot, const TileLoad &a, const TileLoad &b) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = trow + 32 * h;
            *reinterpret_cast<u32x4 *>(&Us[slot][row * ROWB + tch * 16]) = a.v[h];
            *reinterpret_cast<u32x4 *>(&Vs[slot][row * ROWB + tch * 16]) = b.v[h];
        }
    };

    f32x16 acc = {};
    TileLoad la[NSTAGE_TN], lb[NSTAGE_TN];
    for (int g0 = 0; g0 < nsteps; g0 += NSTAGE_TN) {
#pragma unroll
        for (int u = 0; u < NSTAGE_TN; ++u) load(g0 + u, la[u], lb[u]);
#pragma unroll
        for (int u = 0; u < NSTAGE_TN; ++u) store(u, la[u], lb[u]);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NSTAGE_TN; ++u) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 fa = frag_tr(Us[u], wm * 32, s, lane);
                const bf16x8 fb = frag_tr(Vs[u], wn * 32, s, lane);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb, acc, 0, 0, 0);
            }
        }
        __syncthreads();
    }
    const int64_t col = q0 + wn * 32 + r32;
    if (col < Qn && pr.out) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = p0 + wm * 32 + (v >> 2) * 8 + hh * 4 + (v & 3);
            if (row < Pn) pr.out[row * Qn + col] = (uint16_t)f32_to_bf16(pr.scale * acc[v]);
        }
    } else if (col < Qn) {
        float *Pk = P + (int64_t)bz * Pn * Qn;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = p0 + wm * 32 + (v >> 2) * 8 + hh * 4 + (v & 3);
            if (row < Pn) Pk[row * Qn + col] = acc[v];
        }
    }
}

// One launch serves one to three reductions: blocks [0, nb[0]) take the first, the next nb[1] the
// second, the rest the third.
struct RedGroup {
    RedProb p[3];
    uint32_t nb[3];
};
__global__ __launch_bounds__(256) void reduce_partials_kernel(RedGroup grp) {
    uint32_t b = blockIdx.x;
    const int i = b < grp.nb[0] ? 0 : (b < grp.nb[0] + grp.nb[1] ? 1 : 2);
    if (i >= 1) b -= grp.nb[0];
    if (i == 2) b -= grp.nb[1];
    reduce_partials_block(grp.p[i], b, grp.nb[i]);
}

}  // namespace

int choose_split(int64_t tiles, int64_t red_steps) {
    // aim for >= 512 block tiles in flight, each with >= 8 reduction steps
    int64_t s = (512 + tiles - 1) / tiles;
    if (s > red_steps / 8) s = red_steps / 8;
    if (s < 1) s = 1;
    if (s > 64) s = 64;
    return (int)s;
}

hipError_t launch_skinny_nt(const uint16_t *A, const uint16_t *B, bool b_rows_k, float *P, int64_t M,
                            int32_t R, int64_t Kred, int nsplit, hipStream_t stream) {
    const int64_t steps = (Kred + ST - 1) / ST;
    const int64_t per = (steps + nsplit - 1) / nsplit;
    dim3 grid((unsigned)((M + ST - 1) / ST), (unsigned)((R + ST - 1) / ST), (unsigned)nsplit);
    if (b_rows_k)
        hipLaunchKernelGGL(skinny_nt_kernel<true>, grid, dim3(256), 0, stream, A, B, P, M, R, Kred, per * ST);
    else
        hipLaunchKernelGGL(skinny_nt_kernel<false>, grid, dim3(256), 0, stream, A, B, P, M, R, Kred, per * ST);
    return hipGetLastError();
}

namespace {
TnProb tn_prob(const TnProduct &t, int64_t M, uint32_t &nblocks) {
    const int64_t steps = (M + ST - 1) / ST;
    const int64_t per = (steps + t.nsplit - 1) / t.nsplit;
    TnProb p;
    p.U = t.U; p.V = t.V; p.P = t.P; p.Pn = t.Pn; p.Qn = t.Qn; p.mchunk = per * ST;
    p.out = t.nsplit == 1 ? t.out : nullptr;
    p.scale = t.scale;
    p.tx = (int32_t)((t.Pn + ST - 1) / ST);
    p.ty = (int32_t)((t.Qn + ST - 1) / ST);
    nblocks = (uint32_t)p.tx * (uint32_t)p.ty * (uint32_t)t.nsplit;
    return p;
}
}  // namespace

RedProb red_prob(const Reduction &r, uint32_t &nblocks) {
    RedProb p;
    p.P = r.P; p.n = r.n; p.out = r.out; p.out2 = r.out2; p.s1 = r.s1; p.s2 = r.s2; p.nsplit = r.nsplit;
    p.stride = r.stride ? r.stride : r.n;
    p.accum = r.accum ? 1u : 0u;
    nblocks = reduce_blocks(r.n);
    return p;
}

SplitPlan gemm_split(int64_t tiles, int64_t steps, int quantum) {
    int64_t s = tiles > 0 ? 256 / tiles : 1;
    const int64_t smax = steps / quantum;
    if (s > smax) s = smax;
    if (s > 16) s = 16;
    if (s < 1) s = 1;
    int64_t per = (steps + s - 1) / s;
    per = (per + quantum - 1) / quantum * quantum;
    s = (steps + per - 1) / per;   // rounding per up may leave the last splits empty: drop them
    if (s <= 1) return SplitPlan{1, steps};
    return SplitPlan{(int)s, per};
}

hipError_t launch_skinny_tn(const TnProduct &a, const TnProduct *b, int64_t M, hipStream_t stream) {
    TnGroup g;
    uint32_t n0 = 0, n1 = 0;
    g.p[0] = tn_prob(a, M, n0);
    g.p[1] = b ? tn_prob(*b, M, n1) : g.p[0];
    g.M = M;
    g.nb0 = n0;
    hipLaunchKernelGGL(skinny_tn_kernel, dim3(n0 + (b ? n1 : 0u)), dim3(256), 0, stream, g);
    return hipGetLastError();
}

hipError_t launch_reduce_partials(const Reduction &a, const Reduction *b, hipStream_t stream, const Reduction *c) {
    RedGroup g;
    const Reduction *rs[3] = {&a, b, c};
    uint32_t total = 0;
    int used = 0;
    for (int i = 0; i < 3; ++i) {
        if (!rs[i]) continue;
        g.p[used] = red_prob(*rs[i], g.nb[used]);
        total += g.nb[used];
        ++used;
    }
    for (int i = used; i < 3; ++i) {
        g.p[i] = g.p[0];
        g.nb[i] = 0;
    }
    hipLaunchKernelGGL(reduce_partials_kernel, dim3(total), dim3(256), 0, stream, g);
    return hipGetLastError();
}

}  // namespace nf4k
