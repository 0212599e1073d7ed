// SwiGLU glue between the gate/up and down linears of a gated MLP (not a step of the method):
//   h = silu(g) * u;  dg = dh * u * sig(g) * (1 + g (1 - sig(g)));  du = dh * g * sig(g)
// bf16 in/out, fp32 arithmetic, 8 elements (16 bytes) per thread per iteration.

#include "common.h"
#include "launch.h"

namespace nf4k {

namespace {

__device__ __forceinline__ float sigm(float x) { return swiglu_sig(x); }

__device__ __forceinline__ void unpack8(const u32x4 &v, float f[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
}

__device__ __forceinline__ u32x4 pack8(const float f[8]) {
    return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
}

__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint16_t *__restrict__ g,
                                                         const uint16_t *__restrict__ u,
                                                         uint16_t *__restrict__ h, int64_t n) {
    const int64_t nv = n >> 3;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv; i += (int64_t)gridDim.x * blockDim.x) {
        float fg[8], fu[8], fh[8];
        unpack8(reinterpret_cast<const u32x4 *>(g)[i], fg);
        unpack8(reinterpret_cast<const u32x4 *>(u)[i], fu);
#pragma unroll
        for (int k = 0; k < 8; ++k) fh[k] = swiglu_h(fg[k], fu[k]);
        reinterpret_cast<u32x4 *>(h)[i] = pack8(fh);
    }
    // scalar tail
    const int64_t t = (nv << 3) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n && t < (nv << 3) + 8) {
        const float x = bf16_to_f32(g[t]), y = bf16_to_f32(u[t]);
        h[t] = (uint16_t)f32_to_bf16(swiglu_h(x, y));
    }
}

__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t *__restrict__ dh,
                                                         const uint16_t *__restrict__ g,
                                                         const uint16_t *__restrict__ u,
                                                         uint16_t *__restrict__ dg,
                                                         uint16_t *__restrict__ du, int64_t n) {
    const int64_t nv = n >> 3;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv; i += (int64_t)gridDim.x * blockDim.x) {
        float fd[8], fg[8], fu[8], og[8], ou[8];
        unpack8(reinterpret_cast<const u32x4 *>(dh)[i], fd);
        unpack8(reinterpret_cast<const u32x4 *>(g)[i], fg);
        unpack8(reinterpret_cast<const u32x4 *>(u)[i], fu);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float s = sigm(fg[k]);
            ou[k] = fd[k] * fg[k] * s;
            og[k] = fd[k] * fu[k] * s * (1.0f + fg[k] * (1.0f - s));
        }
        reinterpret_cast<u32x4 *>(dg)[i] = pack8(og);
        reinterpret_cast<u32x4 *>(du)[i] = pack8(ou);
    }
    const int64_t t = (nv << 3) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n && t < (nv << 3) + 8) {
        const float d = bf16_to_f32(dh[t]), x = bf16_to_f32(g[t]), y = bf16_to_f32(u[t]);
        const float s = sigm(x);
        du[t] = (uint16_t)f32_to_bf16(d * x * s);
        dg[t] = (uint16_t)f32_to_bf16(d * y * s * (1.0f + x * (1.0f - s)));
    }
}

int grid_elems(int64_t n) {
    int64_t g = ((n >> 3) + 255) / 256;
    if (g > 256 * 8) g = 256 * 8;
    if (g < 1) g = 1;
    return (int)g;
}

}  // namespace

hipError_t launch_swiglu_fwd(const uint16_t *g, const uint16_t *u, uint16_t *h, int64_t n,
                             hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(grid_elems(n)), dim3(256), 0, stream, g, u, h, n);
    return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t *dh, const uint16_t *g, const uint16_t *u, uint16_t *dg,
                             uint16_t *du, int64_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid_elems(n)), dim3(256), 0, stream, dh, g, u, dg, du, n);
    return hipGetLastError();
}

}  // namespace nf4k
