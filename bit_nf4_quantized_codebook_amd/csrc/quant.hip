// Level-1 quantization, double quantization and standalone double dequantization kernels.
//
// Page: "QLoRA: Efficient Finetuning of Quantized LLMs" study notes (gitcode.csdn.net),
// sections 3.1 (block-wise quantization), 3.2 (NF4), 3.3 (double quantization), 3.5 (eq. 6).
//
// All three are HBM-streaming kernels: one pass over their input, coalesced 16-byte accesses,
// grid-stride loops sized to fill the 256 CUs.

#include <cmath>
#include <cstring>

#include "common.h"
#include "launch.h"

namespace nf4k {

// ------------------------------------------------------------------------------------------
// Level 1.  A wave takes 8 consecutive 64-blocks (512 floats) per iteration with two fully
// contiguous 1 KB loads: lane l reads elements 256 q + 4 l .. +3 (q = 0, 1), so block 4 q + l / 16
// is held by 16 lanes, 4 elements each, and its absmax is a 16-lane max.  Code = number of
// decision thresholds strictly below n, where thr[j] is the largest float not above the midpoint
// of codewords j and j+1 (so ties go to the lower index).  Each lane writes its 4 codes as 2 bytes
// (128 contiguous bytes per wave and q).
//
// n = fp32(x / a) without a division per element: with r = fp32(1 / a) (one IEEE division per
// block and lane), q0 = fp32(x r) is within an ulp of x / a, the remainder x - a q0 is exact in
// one fma, and fp32(q0 + (x - a q0) r) is the correctly rounded quotient (Markstein's correction
// step) as long as that remainder stays in the normal range.  With a in [2^-60, 2^100] it does
// for every quotient of magnitude 2^-40 or more; below that the result may differ from x / a in
// its last bits, which decides no code as long as every threshold is at least 2^-39 away from
// zero (the host checks; otherwise, and for blocks outside that range, the kernel divides).  A
// CPU run over 4e8 random and boundary cases (all-ones significands, quotients next to the
// thresholds) found no difference at or above 2^-40.
// The code, the number of thresholds below n, comes from a 256-bucket table over [-1, 1]: bucket
// i = trunc(fp32(n * 127.5 + 128)) (one fma, a clamp, a conversion) holds the count of thresholds
// below the bucket and the one threshold inside it (or +inf), so the code is that count plus one
// compare.  The host builds the table and checks that it decides every code as the count would:
// each bucket widened by 2^-12 of its width on both sides (far more than the fma's rounding
// moves n across a bucket edge) holds at most one threshold, and none lies below the first
// bucket (a NaN quotient takes bucket 0 and code 0, as the count gives).  Codebooks that fail the
// check (two codewords closer than a bucket, as in a table with two zeros) take a binary search
// instead, one bit per level: 4 compares, the last three levels' thresholds read from LDS.
// ------------------------------------------------------------------------------------------
struct Thresholds {
    float t[15];
};

constexpr int QT_BUCKETS = 256;
struct QTable {
    uint32_t thr[QT_BUCKETS];    // bits of the threshold inside the bucket, +inf if none
    uint8_t below[QT_BUCKETS];   // thresholds below the bucket
};

__device__ __forceinline__ uint32_t table_code(float n, const uint2 *tab) {
    // med3 clamps into [0, 255] (a NaN quotient gives 0); the conversion truncates
    const uint32_t i = (uint32_t)__builtin_amdgcn_fmed3f(__builtin_fmaf(n, 127.5f, 128.0f), 0.0f, 255.0f);
    const uint2 e = tab[i];
    return e.y + (n > __uint_as_float(e.x) ? 1u : 0u);
}

// v moved by the DPP control CTRL within 16-lane rows (every source lane inside the row)
template <int CTRL>
__device__ __forceinline__ float row_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// t7: the middle threshold; ts: the 15 thresholds in LDS
__device__ __forceinline__ uint32_t nearest_code(float n, float t7, const float *ts) {
    uint32_t c = n > t7 ? 1u : 0u;                        // c = b3
    c = 2 * c + (n > ts[8 * c + 3] ? 1u : 0u);            // t[3] or t[11]; c = 2 b3 + b2
    c = 2 * c + (n > ts[4 * c + 1] ? 1u : 0u);            // t[1], t[5], t[9] or t[13]
    return 2 * c + (n > ts[2 * c] ? 1u : 0u);             // t[0], t[2], ..., t[14]
}

template <bool TABLE>
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ W, int64_t numel,
                                                       Thresholds th, QTable qt, uint32_t zero_code,
                                                       uint32_t fast_div, uint8_t *__restrict__ packed,
                                                       float *__restrict__ absmax) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x & 63;
    __shared__ float ts[16];
    __shared__ uint2 tab[TABLE ? QT_BUCKETS : 1];
    if (TABLE) tab[threadIdx.x] = make_uint2(qt.thr[threadIdx.x], qt.below[threadIdx.x]);   // 256 threads
    else if (threadIdx.x < 15) ts[threadIdx.x] = th.t[threadIdx.x];
    __syncthreads();
    const int64_t nblocks = (numel + 63) >> 6;
    const int64_t nchunks = (numel + 511) >> 9;                      // 512-element wave chunks
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t nbytes = (numel + 1) >> 1;
    for (int64_t ch = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); ch < nchunks; ch += waves) {
        const int64_t base = ch << 9;
        const bool full = base + 512 <= numel;
        float x[2][4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t e0 = base + 256 * q + 4 * lane;
            if (full) {
                const f4 v = __builtin_nontemporal_load(reinterpret_cast<const f4 *>(W + e0));
                x[q][0] = v.x; x[q][1] = v.y; x[q][2] = v.z; x[q][3] = v.w;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) x[q][i] = (e0 + i < numel) ? W[e0 + i] : 0.0f;
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int64_t e0 = base + 256 * q + 4 * lane;
            const int64_t b = e0 >> 6;
            float a = fmaxf(fmaxf(fabsf(x[q][0]), fabsf(x[q][1])), fmaxf(fabsf(x[q][2]), fabsf(x[q][3])));
            // max over the block's 16 lanes with DPP row moves (no LDS round trips): lane ^ 1,
            // lane ^ 2 (quad permutes), then the mirror within each 8 and within the 16
            a = fmaxf(a, row_move<0xB1>(a));
            a = fmaxf(a, row_move<0x4E>(a));
            a = fmaxf(a, row_move<0x141>(a));
            a = fmaxf(a, row_move<0x140>(a));
            float n[4];
            if (fast_div && a >= 0x1p-60f && a <= 0x1p100f) {   // uniform per block
                const float r = 1.0f / a;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float q0 = x[q][i] * r;
                    n[i] = __builtin_fmaf(__builtin_fmaf(-a, q0, x[q][i]), r, q0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) n[i] = x[q][i] / a;   // a == 0: masked below
            }
            // every element is coded, then the zero code is selected for an all-zero block and
            // for padding elements past the end: no branch per element
            uint32_t word = 0;
            if (TABLE) {
#pragma unroll
                for (int i = 0; i < 4; ++i) word |= table_code(n[i], tab) << (4 * i);
                if (!full) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (e0 + i >= numel) word = (word & ~(15u << (4 * i))) | (zero_code << (4 * i));
                }
                if (a == 0.0f) word = zero_code * 0x1111u;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool valid = a != 0.0f && e0 + i < numel;
                    const uint32_t c = nearest_code(valid ? n[i] : 0.0f, th.t[7], ts);
                    word |= (valid ? c : zero_code) << (4 * i);
                }
            }
            if ((lane & 15) == 0 && b < nblocks) absmax[b] = a;
            const int64_t byte = e0 >> 1;
            if (full) {
                *reinterpret_cast<uint16_t *>(packed + byte) = (uint16_t)word;
            } else {
                if (byte < nbytes) packed[byte] = (uint8_t)word;
                if (byte + 1 < nbytes) packed[byte + 1] = (uint8_t)(word >> 8);
            }
        }
    }
}

// ------------------------------------------------------------------------------------------
// Double quantization, phase 1: the float64 sum behind the mean, taken as a 256-ary tree (groups
// of 256 consecutive values, each summed sequentially in ascending order, level after level).
// group_sum_kernel: one level, GPW groups per workgroup.  Its four waves stage the groups in LDS
// with coalesced 16-byte loads (rows padded to 257 elements, so that lane i reading element k of
// row i hits bank (i + k) mod 64), then one wave runs the GPW sequential sums, a group per lane.
// The first level (11008 groups for a 22016 x 8192 weight) takes 16 groups per workgroup, so that
// every CU stages a share (64 per workgroup left 84 CUs idle and took 8.4 us).
// ------------------------------------------------------------------------------------------
template <typename Tin, int GPW>
__global__ __launch_bounds__(256) void group_sum_kernel(const Tin *__restrict__ in, int64_t n,
                                                        double *__restrict__ out) {
    constexpr int ROW = 257;
    constexpr int PER16 = 16 / (int)sizeof(Tin);            // elements per 16-byte load
    __shared__ Tin tile[GPW * ROW];
    const int tid = threadIdx.x;
    const int64_t e0 = (int64_t)blockIdx.x * (GPW * 256);    // first element of the workgroup
    typedef Tin v16 __attribute__((ext_vector_type(PER16)));
    constexpr int LOADS = GPW * 256 / (256 * PER16);
    static_assert(LOADS >= 1 && GPW <= 64, "groups per workgroup");
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
        const int e = (q * 256 + tid) * PER16;                // element within the workgroup's run
        Tin v[PER16];
        if (e0 + e + PER16 <= n) {
            const v16 x = *reinterpret_cast<const v16 *>(in + e0 + e);
#pragma unroll
            for (int k = 0; k < PER16; ++k) v[k] = x[k];
        } else {
#pragma unroll
            for (int k = 0; k < PER16; ++k) v[k] = (e0 + e + k < n) ? in[e0 + e + k] : (Tin)0;
        }
#pragma unroll
        for (int k = 0; k < PER16; ++k) tile[((e + k) >> 8) * ROW + ((e + k) & 255)] = v[k];
    }
    __syncthreads();
    if (tid >= GPW) return;
    const int64_t g = (int64_t)blockIdx.x * GPW + tid;
    const int64_t base = g << 8;
    if (base >= n) return;
    const int cnt = (int)((n - base) < 256 ? (n - base) : 256);
    const Tin *row = tile + tid * ROW;
    double s = 0.0;
    if (cnt == 256) {
#pragma unroll 16
        for (int i = 0; i < 256; ++i) s += (double)row[i];
    } else {
        for (int i = 0; i < cnt; ++i) s += (double)row[i];
    }
    out[g] = s;
}

// The last levels in one workgroup: up to TAIL_MAX float64 values are staged in LDS (one pad slot
// per 256, so lanes summing neighbouring groups fall on different banks), then each level's
// groups are summed sequentially, a group per lane, until one value is left.
constexpr int TAIL_MAX = 16384;
__global__ __launch_bounds__(1024) void group_sum_tail_kernel(const double *__restrict__ in, int64_t n,
                                                              double *__restrict__ total) {
    __shared__ double v[TAIL_MAX + TAIL_MAX / 256];
    const int tid = threadIdx.x;
    {
        // every load in flight before the first LDS store
        double r[TAIL_MAX / 1024];
#pragma unroll
        for (int q = 0; q < TAIL_MAX / 1024; ++q) {
            const int e = tid + 1024 * q;
            r[q] = e < (int)n ? in[e] : 0.0;
        }
#pragma unroll
        for (int q = 0; q < TAIL_MAX / 1024; ++q) {
            const int e = tid + 1024 * q;
            if (e < (int)n) v[e + (e >> 8)] = r[q];
        }
    }
    __syncthreads();
    int len = (int)n;
    while (len > 1) {
        const int ng = (len + 255) >> 8;
        double s = 0.0;
        if (tid < ng) {
            // group tid: values 256 tid .. , stored from 257 tid (one pad slot per 256 before it)
            const double *g = v + 257 * tid;
            const int cnt = (len - 256 * tid) < 256 ? (len - 256 * tid) : 256;
            if (cnt == 256) {
#pragma unroll 16
                for (int i = 0; i < 256; ++i) s += g[i];
            } else {
                for (int i = 0; i < cnt; ++i) s += g[i];
            }
        }
        __syncthreads();
        if (tid < ng) v[tid + (tid >> 8)] = s;       // value tid of the next level
        __syncthreads();
        len = ng;
    }
    if (tid == 0) total[0] = v[0];
}

// Phase 2: per 256-block of constants, centre by the mean, scale by max|y|/448 and encode E4M3
// (section 3.3), or with int8 set scale by max|y|/127 and round to an integer (eq. (1) at 8 bits).
__global__ __launch_bounds__(64) void dq_encode_kernel(const float *__restrict__ absmax, int64_t nb,
                                                       const double *__restrict__ total,
                                                       uint8_t *__restrict__ codes,
                                                       float *__restrict__ scales,
                                                       float *__restrict__ mean_out, uint32_t int8) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const int lane = threadIdx.x;
    const float mu = (float)(total[0] / (double)nb);
    const int64_t ng = (nb + 255) >> 8;
    // y = absmax - mean of the group's 4 values of this lane (0 past the end)
    auto load = [&](int64_t g, float (&y)[4]) {
        const int64_t i0 = (g << 8) + lane * 4;
        if (g < ng && i0 + 3 < nb) {
            const f4 a = *reinterpret_cast<const f4 *>(absmax + i0);
            y[0] = a.x - mu; y[1] = a.y - mu; y[2] = a.z - mu; y[3] = a.w - mu;
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = (g < ng && i0 + k < nb) ? (absmax[i0 + k] - mu) : 0.0f;
        }
    };
    // the next group's loads go out before this group's arithmetic
    float y[4];
    load(blockIdx.x, y);
    for (int64_t g = blockIdx.x; g < ng; g += gridDim.x) {
        float yn[4];
        load(g + gridDim.x, yn);
        const int64_t i0 = (g << 8) + lane * 4;
        // from 0: a NaN constant is passed over, as fmaxf does (the lane's value is never NaN)
        float m = fmaxf(fmaxf(fmaxf(0.0f, fabsf(y[0])), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
        // max over the wave: within each 16-lane row by DPP moves (lane ^ 1, lane ^ 2, the mirror
        // within 8, the mirror within 16), then the four rows' maxima
        m = fmaxf(m, row_move<0xB1>(m));
        m = fmaxf(m, row_move<0x4E>(m));
        m = fmaxf(m, row_move<0x141>(m));
        m = fmaxf(m, row_move<0x140>(m));
        const int mi = __float_as_int(m);
        m = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(mi, 0)), __int_as_float(__builtin_amdgcn_readlane(mi, 16))),
                  fmaxf(__int_as_float(__builtin_amdgcn_readlane(mi, 32)), __int_as_float(__builtin_amdgcn_readlane(mi, 48))));
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
#pragma unroll
        for (int k = 0; k < 4; ++k) y[k] = yn[k];
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

// The bucket table of the level-1 kernel; false where a widened bucket holds two thresholds or a
// threshold lies below the first bucket (the kernel then searches).  Bucket i takes the quotients
// n whose fp32(n * 127.5 + 128) truncates to i: n in [(i - 128) / 127.5, (i - 127) / 127.5), up to
// the fma's rounding (2^-17 in units of the bucket), well inside the 2^-12 margin checked here.
bool build_quant_table(const float thr[15], QTable &q) {
    for (int i = 0; i < QT_BUCKETS; ++i) {
        const double lo = ((double)i - 128.0 - 0x1p-12) / 127.5;
        const double hi = ((double)i - 127.0 + 0x1p-12) / 127.5;
        int below = 0, inside = 0;
        float t_in = INFINITY;
        for (int j = 0; j < 15; ++j) {
            const double t = (double)thr[j];
            if (!(t == t)) return false;
            if (t < lo) {
                ++below;
            } else if (t <= hi) {
                ++inside;
                t_in = thr[j];
            }
        }
        if (inside > 1 || (i == 0 && below != 0)) return false;
        std::memcpy(&q.thr[i], &t_in, 4);
        q.below[i] = (uint8_t)below;
    }
    return true;
}

hipError_t launch_quantize(const float *W, int64_t numel, const float thr[15], uint32_t zero_code,
                           uint8_t *packed, float *absmax, hipStream_t stream) {
    if (numel == 0) return hipSuccess;
    Thresholds th;
    // the reciprocal form of the division decides every code as the division would when no
    // threshold lies within 2^-39 of zero (see the kernel)
    uint32_t fast_div = 1;
    for (int j = 0; j < 15; ++j) {
        th.t[j] = thr[j];
        if (!(std::fabs(thr[j]) >= 0x1p-39f)) fast_div = 0;   // also a NaN threshold
    }
    static_assert(sizeof(QTable) + sizeof(Thresholds) + 64 <= 4096, "kernel arguments");
    QTable qt;
    const bool table = build_quant_table(thr, qt);
    const int64_t nchunks = (numel + 511) >> 9;
    const int grid = grid_for(nchunks, 4, 256 * 32);
    if (table)
        hipLaunchKernelGGL(quantize_kernel<true>, dim3(grid), dim3(256), 0, stream, W, numel, th, qt, zero_code,
                           fast_div, packed, absmax);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, dim3(grid), dim3(256), 0, stream, W, numel, th, qt, zero_code,
                           fast_div, packed, absmax);
    return hipGetLastError();
}

// Level arrays of the tree sum, back to back, each padded to an even length so that every array
// starts 16-byte aligned (its kernel reads it with 16-byte loads); the total follows the last one.
static int64_t padded(int64_t len) { return (len + 1) & ~(int64_t)1; }

size_t double_quant_ws(int64_t nb) {
    // one float64 per 256-group at each level
    int64_t len = (nb + 255) / 256;
    size_t total = (size_t)padded(len);
    while (len > 1) {
        len = (len + 255) / 256;
        total += (size_t)padded(len);
    }
    return (total + 2) * sizeof(double);
}

hipError_t launch_double_quant(const float *absmax, int64_t nb, uint8_t *codes, float *scales,
                               float *mean, void *ws, bool int8, hipStream_t stream) {
    double *buf = reinterpret_cast<double *>(ws);
    double *level = buf;
    // level 1: floats -> float64 group sums
    int64_t len = (nb + 255) / 256;
    hipLaunchKernelGGL((group_sum_kernel<float, 16>), dim3(grid_for(len, 16, 1 << 30)), dim3(256), 0,
                       stream, absmax, nb, level);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // middle levels while more than one workgroup's LDS holds
    while (len > TAIL_MAX) {
        double *next = level + padded(len);
        const int64_t nlen = (len + 255) / 256;
        hipLaunchKernelGGL((group_sum_kernel<double, 64>), dim3(grid_for(nlen, 64, 1 << 30)), dim3(256), 0,
                           stream, level, len, next);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        level = next;
        len = nlen;
    }
    // the remaining levels, and the total after the level arrays
    double *total = level + padded(len);
    hipLaunchKernelGGL(group_sum_tail_kernel, dim3(1), dim3(1024), 0, stream, level, len, total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ng = (nb + 255) / 256;
    // (two groups per wave, a workgroup per group, or four one-group waves per workgroup: each
    // measured slower, 8.6-9.2 us against 7.9 us at 11008 groups, when the wave's max still went
    // through LDS shuffles)
    hipLaunchKernelGGL(dq_encode_kernel, dim3(grid_for(ng, 1, 256 * 32)), dim3(64), 0, stream,
                       absmax, nb, total, codes, scales, mean, int8 ? 1u : 0u);
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
