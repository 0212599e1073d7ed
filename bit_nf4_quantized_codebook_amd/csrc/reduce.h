// Fixed-order sum of split-reduction partials, shared by the launches that carry it: its own
// launch (one to three reductions) and, at large token counts, extra workgroups of the weight
// expansion launch.
//   out[i] = bf16(s1 * sum_k P[k stride + i]) (k ascending); out2 (optional) = bf16(s2 * the same
//   sum); with accum, out[i] = bf16(s1 * sum + out[i]) (the product added to what out holds).
// Four elements per thread (n and stride are multiples of 4 for every caller: r % 8 == 0, and the
// split GEMMs' output widths are multiples of 8).
#pragma once

#include "common.h"

namespace nf4k {

struct RedProb {
    const float *P;
    int64_t n, stride;
    uint16_t *out, *out2;
    float s1, s2;
    int32_t nsplit;
    uint32_t accum;
};

// workgroup `blk` of `nblk` workgroups (256 threads) covering one reduction
__device__ __forceinline__ void reduce_partials_block(const RedProb &pr, int64_t blk, int64_t nblk) {
    typedef float f32v4 __attribute__((ext_vector_type(4)));
    const float *__restrict__ P = pr.P;
    uint16_t *__restrict__ out = pr.out;
    uint16_t *__restrict__ out2 = pr.out2;
    const int64_t n = pr.n, stride = pr.stride;
    const int nsplit = pr.nsplit;
    const float s1 = pr.s1, s2 = pr.s2;
    const int64_t n4 = n >> 2;
    for (int64_t i = blk * 256 + threadIdx.x; i < n4; i += nblk * 256) {
        f32v4 acc = reinterpret_cast<const f32v4 *>(P)[i];
        // the partials' loads go out eight at a time (one after another, each waiting for the
        // last, a 32-way sum took 10 us for 1024 elements); the adds keep ascending k
        for (int k0 = 1; k0 < nsplit; k0 += 8) {
            f32v4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (k0 + u < nsplit) v[u] = reinterpret_cast<const f32v4 *>(P + (int64_t)(k0 + u) * stride)[i];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (k0 + u < nsplit) acc += v[u];
        }
        if (out && pr.accum) {
            const uint2 old = reinterpret_cast<const uint2 *>(out)[i];
            const uint2 o = {pack_bf16x2(s1 * acc.x + bf16_to_f32(old.x & 0xFFFFu), s1 * acc.y + bf16_to_f32(old.x >> 16)),
                             pack_bf16x2(s1 * acc.z + bf16_to_f32(old.y & 0xFFFFu), s1 * acc.w + bf16_to_f32(old.y >> 16))};
            reinterpret_cast<uint2 *>(out)[i] = o;
        } else if (out) {
            uint2 o = {pack_bf16x2(s1 * acc.x, s1 * acc.y), pack_bf16x2(s1 * acc.z, s1 * acc.w)};
            reinterpret_cast<uint2 *>(out)[i] = o;
        }
        if (out2) {
            uint2 o = {pack_bf16x2(s2 * acc.x, s2 * acc.y), pack_bf16x2(s2 * acc.z, s2 * acc.w)};
            reinterpret_cast<uint2 *>(out2)[i] = o;
        }
    }
}

// workgroups for one reduction: one per 256 x 4 elements, at most 2048
inline uint32_t reduce_blocks(int64_t n) {
    int64_t g = ((n >> 2) + 255) / 256;
    if (g > 256 * 8) g = 256 * 8;
    if (g < 1) g = 1;
    return (uint32_t)g;
}

}  // namespace nf4k
