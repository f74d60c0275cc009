// Device helpers shared by the bandwidth-bound quantisation kernels of
// libi8mm (quant_kernels.hip, variant_kernels.hip): packed 16-bit integer
// operations on pairs of fp16 values, per-chunk row work on 16-byte chunks
// of 8 fp16 values, and block-wide prefix counts of the outlier mask.
//
// Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for
// Transformers at Scale" (paper-graph-ui digest); [TM] transformer-math
// LLM.int8() tutorial (aicassindra.com).
#pragma once

#include "device_common.h"

#include <cmath>

namespace i8mm {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_sub_u16(uint32_t a, uint32_t b) {   // lane-wise, modulo 2^16
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) - __builtin_bit_cast(u16x2, b));
}

constexpr uint32_t kAbs2 = 0x7fff7fffu;     // clears the sign bits of both fp16 halves
constexpr uint32_t kInfBits = 0x7c00u;      // +inf; larger |x| patterns are NaN

__device__ __forceinline__ uint32_t word_of(const uint4& v, int k) {
    return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Per-chunk row work ([DIGEST] Step 4; [TM] "Absmax INT8 quantization from
// first principles").

// The chunk with the values whose bit in `bits` is set replaced by +0.
__device__ __forceinline__ uint4 chunk_clear(const uint4& v, uint32_t bits) {
    auto keep = [&](int k) {
        const uint32_t lo = (bits >> (2 * k)) & 1u ? 0u : 0x0000ffffu;
        const uint32_t hi = (bits >> (2 * k + 1)) & 1u ? 0u : 0xffff0000u;
        return lo | hi;
    };
    return make_uint4(v.x & keep(0), v.y & keep(1), v.z & keep(2), v.w & keep(3));
}

// Running packed maximum of the |x| bit patterns of a chunk.
__device__ __forceinline__ uint32_t chunk_absmax_fold(const uint4& v, uint32_t m2) {
    return pk_max_u16(pk_max_u16(m2, v.x & kAbs2),
                      pk_max_u16(pk_max_u16(v.y & kAbs2, v.z & kAbs2), v.w & kAbs2));
}

// The larger of the two halves of a packed maximum, as a float.
__device__ __forceinline__ float absmax_value(uint32_t m2) {
    const uint32_t a = m2 & 0xffffu, b = m2 >> 16;
    return half_bits_to_float(a > b ? a : b);
}

// fl32(x c) for the fp16 value x in the low (HI = false) or high half of
// word w: v_fma_mix_f32 widens the half exactly and rounds x c + 0 once,
// which is the rounded product except that a zero product comes out +0
// (round_code maps both zeros to code 0), in one instruction.
template <bool HI>
__device__ __forceinline__ float mul_half(uint32_t w, float c) {
    float r;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(c));
    else
        asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(c));
    return r;
}

// round half away from zero of v = fl32(x c), as in quantize_one
__device__ __forceinline__ int round_code(float v) {
    return static_cast<int>(__fadd_rn(v, copysignf(0.49999997f, v)));
}

// The 8 quantised values of a chunk (quantize_one of each), packed bytewise.
__device__ __forceinline__ uint2 chunk_quantize(const uint4& v, float sc) {
    int q[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        q[2 * k] = round_code(mul_half<false>(word_of(v, k), sc));
        q[2 * k + 1] = round_code(mul_half<true>(word_of(v, k), sc));
    }
    return make_uint2(pack_bytes(q[0], q[1], q[2], q[3]), pack_bytes(q[4], q[5], q[6], q[7]));
}

// ---------------------------------------------------------------------------
// Outlier test ([DIGEST] "The Full LLM.int8() Algorithm", Step 1: column j
// is an outlier iff some |X_ij| >= alpha). With thr = the smallest fp16 bit
// pattern in [0, inf] whose value is >= alpha, |x| >= alpha holds iff
// thr <= bits(|x|) <= inf (NaN fails both tests), i.e. iff
// (bits(|x|) - thr) mod 2^16 <= inf - thr. A column's flag is therefore the
// running minimum of that difference over the rows, tested once at the end.
struct Threshold {
    uint32_t thr2;    // thr in both halves
    uint32_t span;    // inf - thr
};

__device__ __forceinline__ void detect_fold(uint4& d, const uint4& v, uint32_t thr2) {
    d.x = pk_min_u16(d.x, pk_sub_u16(v.x & kAbs2, thr2));
    d.y = pk_min_u16(d.y, pk_sub_u16(v.y & kAbs2, thr2));
    d.z = pk_min_u16(d.z, pk_sub_u16(v.z & kAbs2, thr2));
    d.w = pk_min_u16(d.w, pk_sub_u16(v.w & kAbs2, thr2));
}

__device__ __forceinline__ uint4 detect_init() { return make_uint4(~0u, ~0u, ~0u, ~0u); }

// Bit e set iff column e of the chunk is flagged.
__device__ __forceinline__ uint32_t detect_flags(const uint4& d, uint32_t span) {
    uint32_t f = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) f |= (((word_of(d, e >> 1) >> ((e & 1) * 16)) & 0xffffu) <= span ? 1u : 0u) << e;
    return f;
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero, so a ragged or absent row needs no branch around its loads (and
// waits on later loads stay countable).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                             0x00020000);
}

__device__ __forceinline__ uint4 load_chunk_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ uint4 load_chunk(const uint16_t* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// Exclusive prefix sum of the popcounts of mask words [0, nw) into pre[]
// (LDS), for a block of `nthr` threads; returns |O|.
__device__ __forceinline__ int block_mask_prefix(const uint32_t* smask, int* pre, int nw, int* wsum, int nthr) {
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6, nwav = nthr / 64;
    const int per = (nw + nthr - 1) / nthr;
    const int w0 = t * per;
    const int w1 = w0 + per < nw ? w0 + per : nw;
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(smask[w]);
    const int incl = wave_inclusive_scan(cnt, lane);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    if (wid == 0) {
        int v = lane < nwav ? wsum[lane] : 0;
        v = wave_inclusive_scan(v, lane);
        if (lane < nwav) wsum[lane] = v;
    }
    __syncthreads();
    int run = (wid > 0 ? wsum[wid - 1] : 0) + incl - cnt;
    for (int w = w0; w < w1; ++w) {
        pre[w] = run;
        run += __popc(smask[w]);
    }
    const int n = wsum[nwav - 1];
    __syncthreads();
    return n;
}

// Writes mask[], idx[0 .. n) and n_out from the LDS mask and its prefix.
__device__ __forceinline__ void emit_outlier_set(const uint32_t* smask, const int* pre, int nw, int n,
                                                 uint32_t* __restrict__ mask, int32_t* __restrict__ idx,
                                                 int32_t* __restrict__ n_out, int nthr) {
    for (int w = threadIdx.x; w < nw; w += nthr) {
        uint32_t bits = smask[w];
        if (mask) mask[w] = bits;
        int r = pre[w];
        while (bits) {
            idx[r++] = w * 32 + (__ffs(bits) - 1);
            bits &= bits - 1u;
        }
    }
    if (threadIdx.x == 0) n_out[0] = n;
}

// Rank of outlier column j (bit j set) among the outlier columns.
__device__ __forceinline__ int outlier_rank(const uint32_t* smask, const int* pre, int j) {
    return pre[j >> 5] + __popc(smask[j >> 5] & ((1u << (j & 31)) - 1u));
}

// Host side of the outlier test.
// Exact fp16 value of a bit pattern in [0, 0x7c00].
inline float half_value(uint32_t b) {
    const int e = static_cast<int>(b >> 10), m = static_cast<int>(b & 0x3ffu);
    if (e == 31) return INFINITY;
    return e == 0 ? std::ldexp(static_cast<float>(m), -24) : std::ldexp(static_cast<float>(m + 1024), e - 25);
}

// The smallest fp16 bit pattern in [0, inf] whose value is >= alpha (alpha
// >= 0, not NaN); the values of [0, inf] increase with their patterns.
inline Threshold make_threshold(float alpha) {
    uint32_t lo = 0, hi = kInfBits;
    while (lo < hi) {
        const uint32_t mid = (lo + hi) / 2;
        if (half_value(mid) >= alpha) hi = mid;
        else lo = mid + 1;
    }
    return Threshold{lo | (lo << 16), kInfBits - lo};
}

}  // namespace
}  // namespace i8mm
