// Level-1 quantization, double quantization and standalone double dequantization kernels.
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// sections 3.1 (block-wise quantization), 3.2 (NF4), 3.3 (double quantization), 3.5 (eq. 6).
//
// All three are HBM-streaming kernels: one pass over their input, coalesced 16-byte accesses,
// grid-stride loops sized to fill the 256 CUs.

#include "common.h"
#include "launch.h"

namespace nf4k {

// ------------------------------------------------------------------------------------------
// Level 1: one 64-block per group of 8 lanes; each lane owns 8 consecutive elements.
// Code = number of decision thresholds strictly below n, where thr[j] is the largest float
// not above the midpoint of codewords j and j+1 (so ties go to the lower index).
// ------------------------------------------------------------------------------------------
struct Thresholds {
    float t[15];
};

__device__ __forceinline__ uint32_t nearest_code(float n, const Thresholds &th) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < 15; ++j) c += (n > th.t[j]) ? 1u : 0u;
    return c;
}

__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ W, int64_t numel,
                                                       Thresholds th, uint32_t zero_code,
                                                       uint8_t *__restrict__ packed,
                                                       float *__restrict__ absmax) {
    const int lane8 = threadIdx.x & 7;
    const int64_t nblocks = (numel + 63) >> 6;
    const int64_t groups_per_grid = (int64_t)gridDim.x * (blockDim.x >> 3);
    for (int64_t b = (int64_t)blockIdx.x * (blockDim.x >> 3) + (threadIdx.x >> 3); b < nblocks;
         b += groups_per_grid) {
        const int64_t e0 = (b << 6) + lane8 * 8;
        float x[8];
        const bool full_block = ((b + 1) << 6) <= numel;
        if (full_block) {
            typedef float f4 __attribute__((ext_vector_type(4)));
            const f4 *p = reinterpret_cast<const f4 *>(W + e0);
            f4 v0 = __builtin_nontemporal_load(p);
            f4 v1 = __builtin_nontemporal_load(p + 1);
            x[0] = v0.x; x[1] = v0.y; x[2] = v0.z; x[3] = v0.w;
            x[4] = v1.x; x[5] = v1.y; x[6] = v1.z; x[7] = v1.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (e0 + i < numel) ? W[e0 + i] : 0.0f;
        }
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
        a = fmaxf(a, __shfl_xor(a, 1, 8));
        a = fmaxf(a, __shfl_xor(a, 2, 8));
        a = fmaxf(a, __shfl_xor(a, 4, 8));
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t c = zero_code;
            if (a != 0.0f) c = nearest_code(x[i] / a, th);
            if (e0 + i >= numel) c = zero_code;
            word |= c << (4 * i);
        }
        if (lane8 == 0) absmax[b] = a;
        if (full_block) {
            reinterpret_cast<uint32_t *>(packed)[e0 >> 3] = word;
        } else {
            const int64_t nbytes = (numel + 1) >> 1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t byte = (e0 >> 1) + i;
                if (byte < nbytes) packed[byte] = (uint8_t)(word >> (8 * i));
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Double quantization, phase 1: float64 sums of groups of 256 consecutive values, each summed
// sequentially in ascending order.  One wave per 64 groups: the wave stages its groups through
// LDS with coalesced loads, then each lane runs the sequential sum of one group.
// ------------------------------------------------------------------------------------------
template <typename Tin>
__global__ __launch_bounds__(64) void group_sum_kernel(const Tin *__restrict__ in, int64_t n,
                                                       double *__restrict__ out) {
    __shared__ Tin tile[64][257];
    const int lane = threadIdx.x;
    const int64_t g0 = (int64_t)blockIdx.x * 64;
    const int64_t ngroups = (n + 255) >> 8;
    for (int g = 0; g < 64; ++g) {
        const int64_t base = (g0 + g) << 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t idx = base + i * 64 + lane;
            tile[g][i * 64 + lane] = (idx < n) ? in[idx] : (Tin)0;
        }
    }
    __syncthreads();
    const int64_t g = g0 + lane;
    if (g < ngroups) {
        const int64_t base = g << 8;
        const int cnt = (int)((n - base) < 256 ? (n - base) : 256);
        double s = 0.0;
        for (int i = 0; i < cnt; ++i) s += (double)tile[lane][i];
        out[g] = s;
    }
}

// Phase 2: per 256-block of constants, centre by the mean, scale by max|y|/448 and encode E4M3
// (section 3.3), or with int8 set scale by max|y|/127 and round to an integer (eq. (1) at 8 bits).
__global__ __launch_bounds__(64) void dq_encode_kernel(const float *__restrict__ absmax, int64_t nb,
                                                       const double *__restrict__ total,
                                                       uint8_t *__restrict__ codes,
                                                       float *__restrict__ scales,
                                                       float *__restrict__ mean_out, uint32_t int8) {
    const int lane = threadIdx.x;
    const float mu = (float)(total[0] / (double)nb);
    const int64_t ng = (nb + 255) >> 8;
    for (int64_t g = blockIdx.x; g < ng; g += gridDim.x) {
        const int64_t i0 = (g << 8) + lane * 4;
        float y[4];
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            y[k] = (i0 + k < nb) ? (absmax[i0 + k] - mu) : 0.0f;
            m = fmaxf(m, fabsf(y[k]));
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        const float s = int8 ? m / 127.0f : m / 448.0f;
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t c = 0;
            if (s != 0.0f) {
                float t = y[k] / s;
                if (int8) {
                    t = fminf(fmaxf(__builtin_rintf(t), -127.0f), 127.0f);
                    c = (uint32_t)(int32_t)t & 0xFFu;
                } else {
                    t = fminf(fmaxf(t, -448.0f), 448.0f);
                    c = f32_to_e4m3(t);
                }
            }
            word |= c << (8 * k);
        }
        if (i0 + 3 < nb) {
            reinterpret_cast<uint32_t *>(codes)[i0 >> 2] = word;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (i0 + k < nb) codes[i0 + k] = (uint8_t)(word >> (8 * k));
        }
        if (lane == 0) scales[g] = s;
        if (lane == 0 && g == 0) mean_out[0] = mu;
    }
}

// ------------------------------------------------------------------------------------------
// Standalone dequantization: one packed dword (8 weights) per lane.  Double dequantization
// (eq. 6) when absmax_plain is NULL; otherwise eq. (2) at one level, the block constant taken
// from the float32 absmax array as stored by the first quantization level.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ packed,
                                                      const uint8_t *__restrict__ absmax_q,
                                                      const float *__restrict__ absmax_scale,
                                                      const float *__restrict__ absmax_mean,
                                                      const float *__restrict__ absmax_plain,
                                                      int64_t numel, Codebook cbk, uint32_t dq_int8,
                                                      uint16_t *__restrict__ out) {
    __shared__ float cb[16];
    if (threadIdx.x < 16) cb[threadIdx.x] = cbk.v[threadIdx.x];
    __syncthreads();
    const bool plain = absmax_plain != nullptr;
    const float mean = plain ? 0.0f : absmax_mean[0];
    const int64_t nwords = (numel + 7) >> 3;
    for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
         w += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e0 = w << 3;
        const int64_t b = e0 >> 6;
        const float a = plain ? absmax_plain[b] : block_scale(absmax_q[b], absmax_scale[b >> 8], mean, dq_int8 != 0);
        uint32_t word;
        if (e0 + 8 <= numel) {
            word = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(packed) + w);
        } else {
            word = 0;
            for (int i = 0; i < 4; ++i)
                if (2 * i < numel - e0) word |= (uint32_t)packed[(e0 >> 1) + i] << (8 * i);
        }
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = cb[(word >> (8 * i)) & 15u] * a;
            const float hi = cb[(word >> (8 * i + 4)) & 15u] * a;
            o[i] = pack_bf16x2(lo, hi);
        }
        if (e0 + 8 <= numel) {
            u32x4 v = {o[0], o[1], o[2], o[3]};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(out + e0));
        } else {
            for (int i = 0; i < 8; ++i)
                if (e0 + i < numel) out[e0 + i] = (uint16_t)(o[i >> 1] >> (16 * (i & 1)));
        }
    }
}

// ------------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------------
static int grid_for(int64_t items, int per_block, int max_blocks) {
    int64_t g = (items + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > max_blocks) g = max_blocks;
    return (int)g;
}

hipError_t launch_quantize(const float *W, int64_t numel, const float thr[15], uint32_t zero_code,
                           uint8_t *packed, float *absmax, hipStream_t stream) {
    if (numel == 0) return hipSuccess;
    Thresholds th;
    for (int j = 0; j < 15; ++j) th.t[j] = thr[j];
    const int64_t nblocks = (numel + 63) >> 6;
    const int grid = grid_for(nblocks, 32, 256 * 64);
    hipLaunchKernelGGL(quantize_kernel, dim3(grid), dim3(256), 0, stream, W, numel, th, zero_code,
                       packed, absmax);
    return hipGetLastError();
}

size_t double_quant_ws(int64_t nb) {
    // one float64 per 256-group at each level, levels laid out back to back
    int64_t len = (nb + 255) / 256;
    size_t total = (size_t)len;
    while (len > 1) {
        len = (len + 255) / 256;
        total += (size_t)len;
    }
    return (total + 1) * sizeof(double);
}

hipError_t launch_double_quant(const float *absmax, int64_t nb, uint8_t *codes, float *scales,
                               float *mean, void *ws, bool int8, hipStream_t stream) {
    double *buf = reinterpret_cast<double *>(ws);
    double *level = buf;
    // level 0: floats -> doubles
    int64_t len = (nb + 255) / 256;
    hipLaunchKernelGGL(group_sum_kernel<float>, dim3(grid_for(len, 64, 1 << 30)), dim3(64), 0,
                       stream, absmax, nb, level);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    while (len > 1) {
        double *next = level + len;
        const int64_t nlen = (len + 255) / 256;
        hipLaunchKernelGGL(group_sum_kernel<double>, dim3(grid_for(nlen, 64, 1 << 30)), dim3(64), 0,
                           stream, level, len, next);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        level = next;
        len = nlen;
    }
    const int64_t ng = (nb + 255) / 256;
    hipLaunchKernelGGL(dq_encode_kernel, dim3(grid_for(ng, 1, 256 * 32)), dim3(64), 0, stream,
                       absmax, nb, level, codes, scales, mean, int8 ? 1u : 0u);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t *packed, const uint8_t *absmax_q, const float *absmax_scale,
                          const float *absmax_mean, const float *absmax_plain, uint32_t dq_int8,
                          int64_t numel, const float cb[16], uint16_t *out, hipStream_t stream) {
    if (numel == 0) return hipSuccess;
    Codebook c;
    for (int j = 0; j < 16; ++j) c.v[j] = cb[j];
    const int64_t nwords = (numel + 7) >> 3;
    hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(nwords, 256, 256 * 32)), dim3(256), 0, stream,
                       packed, absmax_q, absmax_scale, absmax_mean, absmax_plain, numel, c, dq_int8, out);
    return hipGetLastError();
}

}  // namespace nf4k
