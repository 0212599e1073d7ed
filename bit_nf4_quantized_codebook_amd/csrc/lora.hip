// Low-rank (LoRA) side products of the QLoRA linear layer (gfx950).
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 4 eq. (3) (Y = XW + s X L1 L2) and section 3.5 (gradients for L1, L2 only).
//
// These are skinny products whose cost is one pass over an [M, K] or [M, N] activation:
//   skinny_nt:  P[ks] = A[:, chunk ks] . Bt[:, chunk ks]^T     (T = X L1, dT = s dY L2^T)
//   skinny_tn:  P[ms] = U[rows ms, :]^T . V[rows ms, :]        (dL2 = s T^T dY, dL1 = X^T dT)
// Both write float32 partials over a split of the reduction (enough block tiles to fill the
// 256 CUs), and reduce_partials sums them in a fixed order, scales, and rounds to bf16 once.
// MFMA v_mfma_f32_32x32x16_bf16 on 64 x 64 block tiles, 4 waves of 32 x 32.

#include "common.h"
#include "launch.h"

namespace nf4k {

namespace {

constexpr int ST = 64;          // block tile (both output dims) and reduction step
constexpr int LDP = ST + 8;     // padded LDS row (bf16)

__device__ __forceinline__ u32x4 ldg16z(const uint16_t *p, bool ok) {
    return ok ? *reinterpret_cast<const u32x4 *>(p) : u32x4{0, 0, 0, 0};
}

// P[ks][m][j] = sum_{k in chunk ks} A[m][k] * Bt[j][k];  A [M, Kred], Bt [R, Kred] (row-major)
__global__ __launch_bounds__(256) void skinny_nt_kernel(const uint16_t *__restrict__ A,
                                                        const uint16_t *__restrict__ Bt,
                                                        float *__restrict__ P, int64_t M, int32_t R,
                                                        int64_t Kred, int64_t kchunk) {
    __shared__ __align__(16) uint16_t As[ST * LDP];
    __shared__ __align__(16) uint16_t Bs[ST * LDP];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.x * ST;
    const int j0 = blockIdx.y * ST;
    const int ks = blockIdx.z;
    const int64_t kbeg = (int64_t)ks * kchunk;
    const int64_t kend = (kbeg + kchunk < Kred) ? kbeg + kchunk : Kred;
    f32x16 acc = {};
    const int r32 = lane & 31, h = lane >> 5;
    for (int64_t k0 = kbeg; k0 < kend; k0 += ST) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + 256 * q;
            const int row = c >> 3, seg = c & 7;
            const int64_t gk = k0 + seg * 8;
            const bool kin = gk < kend;
            u32x4 va = ldg16z(A + (m0 + row) * Kred + gk, kin && (m0 + row) < M);
            u32x4 vb = ldg16z(Bt + (int64_t)(j0 + row) * Kred + gk, kin && (j0 + row) < R);
            *reinterpret_cast<u32x4 *>(As + row * LDP + seg * 8) = va;
            *reinterpret_cast<u32x4 *>(Bs + row * LDP + seg * 8) = vb;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 a = *reinterpret_cast<const bf16x8 *>(As + (wm * 32 + r32) * LDP + s * 16 + h * 8);
            bf16x8 b = *reinterpret_cast<const bf16x8 *>(Bs + (wn * 32 + r32) * LDP + s * 16 + h * 8);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    const int col = j0 + wn * 32 + r32;
    if (col < R) {
        float *Pk = P + (int64_t)ks * M * R;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = m0 + wm * 32 + (v >> 2) * 8 + h * 4 + (v & 3);
            if (row < M) Pk[row * R + col] = acc[v];
        }
    }
}

// P[ms][p][q] = sum_{m in chunk ms} U[m][p] * V[m][q];  U [M, Pn], V [M, Qn] (row-major)
__global__ __launch_bounds__(256) void skinny_tn_kernel(const uint16_t *__restrict__ U,
                                                        const uint16_t *__restrict__ V,
                                                        float *__restrict__ P, int64_t M, int64_t Pn,
                                                        int64_t Qn, int64_t mchunk) {
    __shared__ __align__(16) uint16_t Us[ST * LDP];   // [p][m]
    __shared__ __align__(16) uint16_t Vs[ST * LDP];   // [q][m]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t p0 = (int64_t)blockIdx.x * ST;
    const int64_t q0 = (int64_t)blockIdx.y * ST;
    const int ms = blockIdx.z;
    const int64_t mbeg = (int64_t)ms * mchunk;
    const int64_t mend = (mbeg + mchunk < M) ? mbeg + mchunk : M;
    f32x16 acc = {};
    const int r32 = lane & 31, h = lane >> 5;
    for (int64_t mm = mbeg; mm < mend; mm += ST) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int c = tid + 256 * q;
            const int row = c >> 3, seg = c & 7;          // row = m offset, seg = 8 columns
            const int64_t gm = mm + row;
            const bool min_ = gm < mend;
            u32x4 vu = ldg16z(U + gm * Pn + p0 + seg * 8, min_ && (p0 + seg * 8) < Pn);
            u32x4 vv = ldg16z(V + gm * Qn + q0 + seg * 8, min_ && (q0 + seg * 8) < Qn);
            const uint32_t wu[4] = {vu.x, vu.y, vu.z, vu.w};
            const uint32_t wv[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Us[(seg * 8 + e) * LDP + row] = (uint16_t)(wu[e >> 1] >> (16 * (e & 1)));
                Vs[(seg * 8 + e) * LDP + row] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
            }
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 a = *reinterpret_cast<const bf16x8 *>(Us + (wm * 32 + r32) * LDP + s * 16 + h * 8);
            bf16x8 b = *reinterpret_cast<const bf16x8 *>(Vs + (wn * 32 + r32) * LDP + s * 16 + h * 8);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    const int64_t col = q0 + wn * 32 + r32;
    if (col < Qn) {
        float *Pk = P + (int64_t)ms * Pn * Qn;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int64_t row = p0 + wm * 32 + (v >> 2) * 8 + h * 4 + (v & 3);
            if (row < Pn) Pk[row * Qn + col] = acc[v];
        }
    }
}

// out[i] = bf16(s1 * sum_k P[k][i]) (k ascending); out2 (optional) = bf16(s2 * same sum)
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float *__restrict__ P, int nsplit,
                                                              int64_t n, float s1, uint16_t *__restrict__ out,
                                                              float s2, uint16_t *__restrict__ out2) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        float acc = P[i];
        for (int k = 1; k < nsplit; ++k) acc += P[(int64_t)k * n + i];
        if (out) out[i] = (uint16_t)f32_to_bf16(s1 * acc);
        if (out2) out2[i] = (uint16_t)f32_to_bf16(s2 * acc);
    }
}

// out[c][r] = in[r][c], bf16, via a 64 x 64 LDS tile
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t *__restrict__ in, int64_t R,
                                                        int64_t C, uint16_t *__restrict__ out) {
    __shared__ uint16_t t[64][65];
    const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int rr = e >> 6, cc = e & 63;
        const int64_t gr = r0 + rr, gc = c0 + cc;
        t[rr][cc] = (gr < R && gc < C) ? in[gr * C + gc] : (uint16_t)0;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int cc = e >> 6, rr = e & 63;
        const int64_t gr = r0 + rr, gc = c0 + cc;
        if (gr < R && gc < C) out[gc * R + gr] = t[rr][cc];
    }
}

}  // namespace

int choose_split(int64_t tiles, int64_t red_steps) {
    // aim for >= 512 block tiles in flight, each with >= 4 reduction steps
    int64_t s = (512 + tiles - 1) / tiles;
    if (s > red_steps / 4) s = red_steps / 4;
    if (s < 1) s = 1;
    if (s > 64) s = 64;
    return (int)s;
}

hipError_t launch_skinny_nt(const uint16_t *A, const uint16_t *Bt, float *P, int64_t M, int32_t R,
                            int64_t Kred, int nsplit, hipStream_t stream) {
    const int64_t steps = (Kred + ST - 1) / ST;
    const int64_t per = (steps + nsplit - 1) / nsplit;
    dim3 grid((unsigned)((M + ST - 1) / ST), (unsigned)((R + ST - 1) / ST), (unsigned)nsplit);
    hipLaunchKernelGGL(skinny_nt_kernel, grid, dim3(256), 0, stream, A, Bt, P, M, R, Kred, per * ST);
    return hipGetLastError();
}

hipError_t launch_skinny_tn(const uint16_t *U, const uint16_t *V, float *P, int64_t M, int64_t Pn,
                            int64_t Qn, int nsplit, hipStream_t stream) {
    const int64_t steps = (M + ST - 1) / ST;
    const int64_t per = (steps + nsplit - 1) / nsplit;
    dim3 grid((unsigned)((Pn + ST - 1) / ST), (unsigned)((Qn + ST - 1) / ST), (unsigned)nsplit);
    hipLaunchKernelGGL(skinny_tn_kernel, grid, dim3(256), 0, stream, U, V, P, M, Pn, Qn, per * ST);
    return hipGetLastError();
}

hipError_t launch_reduce_partials(const float *P, int nsplit, int64_t n, float s1, uint16_t *out,
                                  float s2, uint16_t *out2, hipStream_t stream) {
    int64_t g = (n + 255) / 256;
    if (g > 256 * 16) g = 256 * 16;
    if (g < 1) g = 1;
    hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)g), dim3(256), 0, stream, P, nsplit, n, s1,
                       out, s2, out2);
    return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t *in, int64_t R, int64_t C, uint16_t *out, hipStream_t stream) {
    dim3 grid((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64));
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, stream, in, R, C, out);
    return hipGetLastError();
}

}  // namespace nf4k
