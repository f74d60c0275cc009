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

// The 8 quantised values of a chunk, packed bytewise.
__device__ __forceinline__ uint2 chunk_quantize(const uint4& v, float sc) {
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int q = quantize_one(half_bits_to_float((word_of(v, e >> 1) >> ((e & 1) * 16)) & 0xffffu), sc);
        packed[e >> 2] |= (static_cast<uint32_t>(q) & 0xffu) << ((e & 3) * 8);
    }
    return make_uint2(packed[0], packed[1]);
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

}  // namespace
}  // namespace i8mm
