// Fixed-order sum of split-reduction partials, shared by the launches that carry it: its own
// launch (one or two reductions) and, at large token counts, extra workgroups of the weight
// expansion launch.
//   out[i] = bf16(s1 * sum_k P[k][i]) (k ascending); out2 (optional) = bf16(s2 * the same sum).
// Four elements per thread (n is a multiple of 4 for every caller: r % 8 == 0).
#pragma once

#include "common.h"

namespace nf4k {

struct RedProb {
    const float *P;
    int64_t n;
    uint16_t *out, *out2;
    float s1, s2;
    int32_t nsplit;
};

// workgroup `blk` of `nblk` workgroups (256 threads) covering one reduction
__device__ __forceinline__ void reduce_partials_block(const RedProb &pr, int64_t blk, int64_t nblk) {
    typedef float f32v4 __attribute__((ext_vector_type(4)));
    const float *__restrict__ P = pr.P;
    uint16_t *__restrict__ out = pr.out;
    uint16_t *__restrict__ out2 = pr.out2;
    const int64_t n = pr.n;
    const int nsplit = pr.nsplit;
    const float s1 = pr.s1, s2 = pr.s2;
    const int64_t n4 = n >> 2;
    for (int64_t i = blk * 256 + threadIdx.x; i < n4; i += nblk * 256) {
        f32v4 acc = reinterpret_cast<const f32v4 *>(P)[i];
        for (int k = 1; k < nsplit; ++k) acc += reinterpret_cast<const f32v4 *>(P + (int64_t)k * n)[i];
        if (out) {
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
