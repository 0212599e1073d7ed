// Shared device helpers for the gfx950 kernels (bf16/E4M3 bit manipulation, MFMA vector types).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4k {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Codebook {
    float v[16];
};

// bf16 (as raw bits) -> float, exact.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32; subnormals kept).
__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    __bf16 h = (__bf16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Two floats -> packed bf16 pair (lo in bits 0-15).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// OCP FP8 E4M3 -> float (exact; codes 0x7F/0xFF are NaN and never produced here).
// Branch-free: |v| = (8 [e > 0] + m) * 2^(max(e, 1) - 10), which covers subnormals (e = 0).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const uint32_t sig = m | (min(e, 1u) << 3);
    const float mag = __builtin_amdgcn_ldexpf((float)sig, (int)max(e, 1u) - 10);
    return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// float in [-448, 448] -> E4M3, round to nearest even, sign kept.
__device__ __forceinline__ uint32_t f32_to_e4m3(float t) {
    const uint32_t u = __float_as_uint(t);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (__uint_as_float(a) < 0.015625f) {
        // below the smallest normal 2^-6: multiples of 2^-9 (the scaling is exact)
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        // keep 3 mantissa bits, ties to even; a carry rolls into the exponent
        uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - ((127u - 7u) << 3);
    }
    return sign | code;
}

// Rebuilt first-level block constant (eq. 6 inner dequant): one rounding.  The 8-bit code is
// OCP E4M3 (the 8-bit float of section 3.3) or, when int8 is set, a two's complement integer
// (eq. (1) at 8 bits applied to the centred constants).
__device__ __forceinline__ float block_scale(uint32_t code, float s2, float mean, bool int8) {
    const float v = int8 ? (float)((int32_t)(code << 24) >> 24) : e4m3_to_f32(code);
    return __builtin_fmaf(v, s2, mean);
}

// SwiGLU glue of the gated MLP (not a step of the method), fp32: h = silu(g) u, silu(g) = g sig(g).
// One definition for the glue kernels and the gated GEMM's epilogue, so both give the same bits.
// sig uses the hardware reciprocal (v_rcp_f32, about 1 ulp) rather than a division: the results
// are rounded to bf16, and in the GEMM epilogue the division's dozen instructions per element
// were exposed.
__device__ __forceinline__ float swiglu_sig(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float swiglu_h(float g, float u) { return g * swiglu_sig(g) * u; }

}  // namespace nf4k
