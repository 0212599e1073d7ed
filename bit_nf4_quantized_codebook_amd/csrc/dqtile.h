// Device helpers shared by the kernels (gfx950): buffer descriptors and loads, the XCD-aware tile
// order, and the per-block 16-entry bf16 table with its v_perm_b32 lookups.
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// section 3.5 eq. (6): each weight element is cb[code] * a' rounded once to bf16, with
// a' = fma(e4m3(c2), c1, mean) the rebuilt block constant.
#pragma once

#include "common.h"

namespace nf4k {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;

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

// Tile index bid (blockIdx.x, or its tile part when a product's reduction is split) -> (tm, tn),
// keeping each XCD (bid % 8) on a contiguous run of tiles so that the tiles sharing A rows land on
// the same L2.
__device__ __forceinline__ void tile_coords(int ntm, int ntn, int bid, int &tm, int &tn) {
    const int nt = ntm * ntn;
    const int q = nt / 8;
    int t = bid;
    if (bid < 8 * q) t = (bid % 8) * q + bid / 8;
    tm = t / ntn;
    tn = t % ntn;
}

// Tile index -> (tm, tn) for the bf16 GEMM: each XCD takes a contiguous run of tile indices (as
// above), and the run is walked in groups of GM tile rows, column by column within a group, so
// that the 32 tiles an XCD runs at once form a GM x (32 / GM) block: they share GM tile rows of A
// and 32 / GM tile columns of B in that XCD's L2.
template <int GM>
__device__ __forceinline__ void tile_coords_grouped(int ntm, int ntn, int bid, int &tm, int &tn) {
    const int nt = ntm * ntn;
    const int q = nt / 8;
    int t = bid;
    if (bid < 8 * q) t = (bid % 8) * q + bid / 8;
    const int per_group = GM * ntn;
    const int grp = t / per_group;
    const int first = grp * GM;
    const int gsize = min(ntm - first, GM);
    const int in = t - grp * per_group;
    tm = first + in % gsize;
    tn = in / gsize;
}

// ---- the 16-entry bf16 table of one quantization block, as byte planes ----
struct Lut {
    uint32_t la0, la1, lb0, lb1;   // low bytes of entries 0-3, 4-7, 8-11, 12-15
    uint32_t ha0, ha1, hb0, hb1;   // high bytes
};

__device__ __forceinline__ Lut make_lut(const Codebook &cb, float a) {
    uint32_t p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = pack_bf16x2(cb.v[2 * j] * a, cb.v[2 * j + 1] * a);
    Lut t;
    t.la0 = __builtin_amdgcn_perm(p[1], p[0], 0x06040200u);
    t.ha0 = __builtin_amdgcn_perm(p[1], p[0], 0x07050301u);
    t.la1 = __builtin_amdgcn_perm(p[3], p[2], 0x06040200u);
    t.ha1 = __builtin_amdgcn_perm(p[3], p[2], 0x07050301u);
    t.lb0 = __builtin_amdgcn_perm(p[5], p[4], 0x06040200u);
    t.hb0 = __builtin_amdgcn_perm(p[5], p[4], 0x07050301u);
    t.lb1 = __builtin_amdgcn_perm(p[7], p[6], 0x06040200u);
    t.hb1 = __builtin_amdgcn_perm(p[7], p[6], 0x07050301u);
    return t;
}

// Look up 4 codes (one per byte of x, each 0..15): returns low and high bytes of the 4 entries.
__device__ __forceinline__ void lut4(const Lut &t, uint32_t x, uint32_t &lo, uint32_t &hi) {
    // v_perm selector 0..7 picks a byte of the 8-byte pair; 8..12 give 0 when both sources are
    // 0 and >= 13 gives 0xFF: so perm(0, 0, x + 5) is 0xFF exactly where x >= 8.
    const uint32_t m = __builtin_amdgcn_perm(0u, 0u, x + 0x05050505u);
    const uint32_t xb = x ^ 0x08080808u;
    const uint32_t la = __builtin_amdgcn_perm(t.la1, t.la0, x);
    const uint32_t lb = __builtin_amdgcn_perm(t.lb1, t.lb0, xb);
    const uint32_t ha = __builtin_amdgcn_perm(t.ha1, t.ha0, x);
    const uint32_t hb = __builtin_amdgcn_perm(t.hb1, t.hb0, xb);
    lo = (m & lb) | (~m & la);
    hi = (m & hb) | (~m & ha);
}

// 8 packed codes (element i in bits 4i..4i+3) -> 8 bf16 in element order (4 dwords)
__device__ __forceinline__ u32x4 dequant8(const Lut &t, uint32_t w) {
    uint32_t le, he, lo, ho;
    lut4(t, w & 0x0F0F0F0Fu, le, he);           // elements 0, 2, 4, 6
    lut4(t, (w >> 4) & 0x0F0F0F0Fu, lo, ho);    // elements 1, 3, 5, 7
    const uint32_t p0 = __builtin_amdgcn_perm(lo, le, 0x05010400u);
    const uint32_t q0 = __builtin_amdgcn_perm(ho, he, 0x05010400u);
    const uint32_t p1 = __builtin_amdgcn_perm(lo, le, 0x07030602u);
    const uint32_t q1 = __builtin_amdgcn_perm(ho, he, 0x07030602u);
    u32x4 o;
    o.x = __builtin_amdgcn_perm(q0, p0, 0x05010400u);
    o.y = __builtin_amdgcn_perm(q0, p0, 0x07030602u);
    o.z = __builtin_amdgcn_perm(q1, p1, 0x05010400u);
    o.w = __builtin_amdgcn_perm(q1, p1, 0x07030602u);
    return o;
}

// Same 8 codes in "planar" order (elements 0, 2, 4, 6, 1, 3, 5, 7): 4 byte-interleaves fewer.
// Used where the 8 values land on output columns (backward), which the epilogue permutes back.
__device__ __forceinline__ u32x4 dequant8_planar(const Lut &t, uint32_t w) {
    uint32_t le, he, lo, ho;
    lut4(t, w & 0x0F0F0F0Fu, le, he);
    lut4(t, (w >> 4) & 0x0F0F0F0Fu, lo, ho);
    u32x4 o;
    o.x = __builtin_amdgcn_perm(he, le, 0x05010400u);   // elements 0, 2
    o.y = __builtin_amdgcn_perm(he, le, 0x07030602u);   // elements 4, 6
    o.z = __builtin_amdgcn_perm(ho, lo, 0x05010400u);   // elements 1, 3
    o.w = __builtin_amdgcn_perm(ho, lo, 0x07030602u);   // elements 5, 7
    return o;
}

// column held at position p (0..7) of an 8-column group after dequant8_planar
__device__ __forceinline__ int planar_col(int p) { return ((p & 3) << 1) | (p >> 2); }

}  // namespace nf4k
