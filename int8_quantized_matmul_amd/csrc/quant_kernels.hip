// Bandwidth-bound kernels of the LLM.int8() path for gfx950: outlier-column
// detection, stream compaction of the outlier set, row-wise absmax
// quantisation with the outlier gather, and load-time column-wise weight
// quantisation.
//
// Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for
// Transformers at Scale" (paper-graph-ui digest); [TM] transformer-math
// LLM.int8() tutorial (aicassindra.com).

#include "device_common.h"
#include "launch.h"

namespace i8mm {
namespace {

// ---------------------------------------------------------------------------
// Fill a uint32 array (used to clear the outlier mask before detection; a
// kernel rather than a memset so that the sequence is graph-capture safe).
__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// Outlier-column detection ([DIGEST] "The Full LLM.int8() Algorithm", Step 1).
//
// Block = 256 threads covering 2048 columns (8 fp16 = 16 bytes per thread,
// so one wavefront reads 1 KiB contiguous per row) and `rows` rows. Each
// thread ORs its 8 per-column flags over its rows in a register; the four
// threads of a 32-column mask word meet in LDS through atomicOr, and each
// non-zero word reaches the global mask with one global atomicOr. The mask
// must be zero beforehand.
constexpr int kDetectCols = 2048;

__global__ __launch_bounds__(256) void k_detect(const uint16_t* __restrict__ X, int64_t s, int64_t h,
                                                float alpha, int rows, int64_t n_col_blocks,
                                                uint32_t* __restrict__ mask) {
    __shared__ uint32_t lmask[kDetectCols / 32];
    const int t = threadIdx.x;
    if (t < kDetectCols / 32) lmask[t] = 0u;
    __syncthreads();

    const int64_t cb = static_cast<int64_t>(blockIdx.x) % n_col_blocks;
    const int64_t rb = static_cast<int64_t>(blockIdx.x) / n_col_blocks;
    const int64_t col0 = cb * kDetectCols + static_cast<int64_t>(t) * 8;
    uint32_t flags = 0;
    if (col0 < h) {
        const int64_t r0 = rb * rows;
        const int64_t r1 = r0 + rows < s ? r0 + rows : s;
        const uint16_t* p = X + r0 * h + col0;
        int64_t r = r0;
        for (; r + 4 <= r1; r += 4, p += 4 * h) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const uint4*>(p + u * h);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = half_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
                    flags |= (fabsf(x) >= alpha ? 1u : 0u) << e;
                }
            }
        }
        for (; r < r1; ++r, p += h) {
            uint4 v = *reinterpret_cast<const uint4*>(p);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = half_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
                flags |= (fabsf(x) >= alpha ? 1u : 0u) << e;
            }
        }
    }
    if (flags) atomicOr(&lmask[t >> 2], flags << ((t & 3) * 8));
    __syncthreads();
    if (t < kDetectCols / 32) {
        uint32_t wbits = lmask[t];
        if (wbits) atomicOr(&mask[cb * (kDetectCols / 32) + t], wbits);
    }
}

// ---------------------------------------------------------------------------
// Stream compaction of the mask into the ascending index list idx[0..|O|)
// and |O|. One block of 1024 threads: per-thread popcounts over a run of
// mask words, a block-wide exclusive scan, then each thread writes the
// indices of its set bits in order.
__global__ __launch_bounds__(1024) void k_compact(const uint32_t* __restrict__ mask, int nw,
                                                  int32_t* __restrict__ idx, int32_t* __restrict__ n_out) {
    __shared__ int wsum[16];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int per = (nw + 1023) / 1024;
    const int w0 = t * per;
    const int w1 = w0 + per < nw ? w0 + per : nw;
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(mask[w]);
    const int incl = wave_inclusive_scan(cnt, lane);
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    if (wid == 0) {
        // LDS operations of one wavefront execute in order: every lane reads
        // before any lane writes.
        int v = lane < 16 ? wsum[lane] : 0;
        v = wave_inclusive_scan(v, lane);
        if (lane < 16) wsum[lane] = v;
    }
    __syncthreads();
    int base = (wid > 0 ? wsum[wid - 1] : 0) + incl - cnt;
    for (int w = w0; w < w1; ++w) {
        uint32_t bits = mask[w];
        while (bits) {
            const int b = __ffs(bits) - 1;
            idx[base++] = w * 32 + b;
            bits &= bits - 1u;
        }
    }
    if (t == 0) n_out[0] = wsum[15];
}

// Block-wide max of the per-thread partial absmax (256 threads), then the
// row scale fl32(127 / m).
__device__ __forceinline__ float block_absmax_scale(float m, float* red, int lane, int wid) {
    m = wave_max(m);
    if (lane == 0) red[wid] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return absmax_scale(m);
}

// ---------------------------------------------------------------------------
// Row-wise absmax quantisation over the non-outlier columns plus the gather
// of the outlier columns ([DIGEST] "The Full LLM.int8() Algorithm", Steps 2
// and 4; [TM] "Absmax INT8 quantization from first principles").
//
// One 256-thread block per row. Each thread owns 8-column chunks
// c = t, t + 256, ...; with CPT > 0 the row stays in registers between the
// absmax pass and the quantise pass (CPT chunks per thread), otherwise the
// second pass re-reads the row (an L2 hit).
template <int CPT>
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ X, int64_t h,
                                                    const uint32_t* __restrict__ mask,
                                                    const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ n_out,
                                                    int8_t* __restrict__ Xq, float* __restrict__ c_x,
                                                    uint16_t* __restrict__ X_O, int64_t ldo) {
    __shared__ float red[4];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int64_t i = blockIdx.x;
    const uint16_t* xr = X + i * h;
    const int64_t nch = h / 8;

    float m = 0.0f;
    auto absmax_chunk = [&](const uint4& v, int64_t c) {
        const uint32_t bits = (mask[c >> 2] >> ((c & 3) * 8)) & 0xffu;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = fabsf(half_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
            if (!((bits >> e) & 1u)) m = fmaxf(m, x);
        }
    };
    int8_t* qr = Xq + i * h;
    auto quantize_chunk = [&](const uint4& v, int64_t c, float sc) {
        const uint32_t bits = (mask[c >> 2] >> ((c & 3) * 8)) & 0xffu;
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = half_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
            int q = ((bits >> e) & 1u) ? 0 : quantize_one(x, sc);
            packed[e >> 2] |= (static_cast<uint32_t>(q) & 0xffu) << ((e & 3) * 8);
        }
        *reinterpret_cast<uint2*>(qr + c * 8) = make_uint2(packed[0], packed[1]);
    };

    if constexpr (CPT > 0) {
        uint4 cache[CPT];
#pragma unroll
        for (int p = 0; p < CPT; ++p) {
            const int64_t c = t + 256 * p;
            if (c < nch) cache[p] = *reinterpret_cast<const uint4*>(xr + c * 8);
        }
#pragma unroll
        for (int p = 0; p < CPT; ++p) {
            const int64_t c = t + 256 * p;
            if (c < nch) absmax_chunk(cache[p], c);
        }
        const float sc = block_absmax_scale(m, red, lane, wid);
        if (t == 0) c_x[i] = sc;
#pragma unroll
        for (int p = 0; p < CPT; ++p) {
            const int64_t c = t + 256 * p;
            if (c < nch) quantize_chunk(cache[p], c, sc);
        }
    } else {
        for (int64_t c = t; c < nch; c += 256) absmax_chunk(*reinterpret_cast<const uint4*>(xr + c * 8), c);
        const float sc = block_absmax_scale(m, red, lane, wid);
        if (t == 0) c_x[i] = sc;
        for (int64_t c = t; c < nch; c += 256) quantize_chunk(*reinterpret_cast<const uint4*>(xr + c * 8), c, sc);
    }

    // Gather X_O[i, k] = X[i, idx[k]], zero-padded to a multiple of 32.
    const int n = n_out[0];
    const int npad = (n + 31) & ~31;
    uint16_t* orow = X_O + i * ldo;
    for (int k = t; k < npad; k += 256) orow[k] = k < n ? xr[idx[k]] : static_cast<uint16_t>(0);
}

// ---------------------------------------------------------------------------
// Forward-path variants. The detection kernel ORs into a mask accumulator
// (kept zero between forwards; the product kernel clears it again), and the
// quantise kernel below works from that accumulator directly: the rank of an
// outlier column j in O is the number of set mask bits below j, so each
// block writes X_O straight from the registers holding its row, and block 0
// also emits the mask, the ascending index list and |O|. This replaces the
// separate clear and compaction launches of the standalone entry points.

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
        mask[w] = bits;
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

// One 256-thread block per row (as k_quant_rows), mask from the accumulator.
// Dynamic LDS: nw mask words + nw prefix counts.
template <int CPT>
__global__ __launch_bounds__(256) void k_quant_rows_acc(const uint16_t* __restrict__ X, int64_t h,
                                                        const uint32_t* __restrict__ acc,
                                                        uint32_t* __restrict__ mask, int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ n_out,
                                                        int8_t* __restrict__ Xq, float* __restrict__ c_x,
                                                        uint16_t* __restrict__ X_O, int64_t ldo) {
    extern __shared__ uint32_t dyn[];
    __shared__ float red[4];
    __shared__ int wsum[4];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int nw = static_cast<int>(h / 32);
    uint32_t* smask = dyn;
    int* pre = reinterpret_cast<int*>(dyn + nw);
    const int64_t i = blockIdx.x;
    const uint16_t* xr = X + i * h;
    const int64_t nch = h / 8;

    uint4 cache[CPT > 0 ? CPT : 1];
    if constexpr (CPT > 0) {
#pragma unroll
        for (int p = 0; p < CPT; ++p) {
            const int64_t c = t + 256 * p;
            if (c < nch) cache[p] = *reinterpret_cast<const uint4*>(xr + c * 8);
        }
    }
    for (int w = t; w < nw; w += 256) smask[w] = acc[w];
    __syncthreads();
    const int n = block_mask_prefix(smask, pre, nw, wsum, 256);

    float m = 0.0f;
    auto chunk_bits = [&](int64_t c) { return (smask[c >> 2] >> ((c & 3) * 8)) & 0xffu; };
    auto absmax_chunk = [&](const uint4& v, int64_t c) {
        const uint32_t bits = chunk_bits(c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float x = fabsf(half_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
            if (!((bits >> e) & 1u)) m = fmaxf(m, x);
        }
    };
    int8_t* qr = Xq + i * h;
    uint16_t* orow = X_O + i * ldo;
    auto quantize_chunk = [&](const uint4& v, int64_t c, float sc) {
        const uint32_t bits = chunk_bits(c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t xb = (w[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
            const bool out = (bits >> e) & 1u;
            int q = out ? 0 : quantize_one(half_bits_to_float(xb), sc);
            packed[e >> 2] |= (static_cast<uint32_t>(q) & 0xffu) << ((e & 3) * 8);
            if (out) orow[outlier_rank(smask, pre, static_cast<int>(c * 8 + e))] = static_cast<uint16_t>(xb);
        }
        *reinterpret_cast<uint2*>(qr + c * 8) = make_uint2(packed[0], packed[1]);
    };

    if constexpr (CPT > 0) {
#pragma unroll
        for (int p = 0; p < CPT; ++p) {
            const int64_t c = t + 256 * p;
            if (c < nch) absmax_chunk(cache[p], c);
        }
        const float sc = block_absmax_scale(m, red, lane, wid);
        if (t == 0) c_x[i] = sc;
#pragma unroll
        for (int p = 0; p < CPT; ++p) {
            const int64_t c = t + 256 * p;
            if (c < nch) quantize_chunk(cache[p], c, sc);
        }
    } else {
        for (int64_t c = t; c < nch; c += 256) absmax_chunk(*reinterpret_cast<const uint4*>(xr + c * 8), c);
        const float sc = block_absmax_scale(m, red, lane, wid);
        if (t == 0) c_x[i] = sc;
        for (int64_t c = t; c < nch; c += 256) quantize_chunk(*reinterpret_cast<const uint4*>(xr + c * 8), c, sc);
    }
    const int npad = (n + 31) & ~31;
    for (int k = n + t; k < npad; k += 256) orow[k] = 0;
    if (i == 0) emit_outlier_set(smask, pre, nw, n, mask, idx, n_out, 256);
}

// Small inputs (s <= 16 rows, s * ceil(h / 8192) <= 16): detection,
// compaction and row quantisation in one 1024-thread block. Thread t owns
// the 8-column chunks t and t + 1024 of every row and keeps them in
// registers (at most 16 chunks); column flags are ORed over the rows in a
// register and meet in an LDS mask through atomicOr, per-row maxima are
// reduced across each wavefront and combined with an integer atomicMax on
// the float bits (non-negative floats order like their bit patterns).
constexpr int kSmallThreads = 1024;
constexpr int kSmallMaxRows = 16;       // per-row LDS tables below hold 16 rows

template <int CC>   // column chunks per thread (1: h <= 8192, 2: h <= 16384)
__global__ __launch_bounds__(kSmallThreads) void k_prologue_small(const uint16_t* __restrict__ X, int s, int h,
                                                                  float alpha, uint32_t* __restrict__ mask,
                                                                  int32_t* __restrict__ idx,
                                                                  int32_t* __restrict__ n_out,
                                                                  int8_t* __restrict__ Xq, float* __restrict__ c_x,
                                                                  uint16_t* __restrict__ X_O, int64_t ldo) {
    constexpr int R = kSmallMaxRows / CC;   // rows held per column chunk
    extern __shared__ uint32_t dyn[];
    __shared__ int wsum[kSmallThreads / 64];
    __shared__ uint32_t rmax[kSmallMaxRows];
    __shared__ float rscale[kSmallMaxRows];
    if (s > R || h > CC * kSmallThreads * 8) return;   // the launcher never sends these
    const int t = threadIdx.x, lane = t & 63;
    const int nw = h / 32;
    const int nch_row = h / 8;
    uint32_t* smask = dyn;
    int* pre = reinterpret_cast<int*>(dyn + nw);

    for (int w = t; w < nw; w += kSmallThreads) smask[w] = 0u;
    if (t < kSmallMaxRows) rmax[t] = 0u;
    uint4 v[CC][R];
#pragma unroll
    for (int cc = 0; cc < CC; ++cc) {
        const int c = t + kSmallThreads * cc;
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (c < nch_row && r < s) v[cc][r] = *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(r) * h + c * 8);
    }
    __syncthreads();
    // Step 1: column flags, ORed over the rows first.
#pragma unroll
    for (int cc = 0; cc < CC; ++cc) {
        const int c = t + kSmallThreads * cc;
        uint32_t flags = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (c < nch_row && r < s) {
                const uint32_t w[4] = {v[cc][r].x, v[cc][r].y, v[cc][r].z, v[cc][r].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = half_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
                    flags |= (fabsf(x) >= alpha ? 1u : 0u) << e;
                }
            }
        }
        if (flags) atomicOr(&smask[c >> 2], flags << ((c & 3) * 8));
    }
    __syncthreads();
    const int n = block_mask_prefix(smask, pre, nw, wsum, kSmallThreads);
    // Row absmax over the non-outlier columns.
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < s) {
            float m = 0.0f;
#pragma unroll
            for (int cc = 0; cc < CC; ++cc) {
                const int c = t + kSmallThreads * cc;
                if (c < nch_row) {
                    const uint32_t bits = (smask[c >> 2] >> ((c & 3) * 8)) & 0xffu;
                    const uint32_t w[4] = {v[cc][r].x, v[cc][r].y, v[cc][r].z, v[cc][r].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float x = fabsf(half_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu));
                        if (!((bits >> e) & 1u)) m = fmaxf(m, x);
                    }
                }
            }
            m = wave_max(m);
            if (lane == 0 && m > 0.0f) atomicMax(&rmax[r], __float_as_uint(m));
        }
    }
    __syncthreads();
    if (t < s) {
        const float sc = absmax_scale(__uint_as_float(rmax[t]));
        rscale[t] = sc;
        c_x[t] = sc;
    }
    __syncthreads();
    // Quantise, gather the outlier columns by rank, pad X_O rows.
#pragma unroll
    for (int cc = 0; cc < CC; ++cc) {
        const int c = t + kSmallThreads * cc;
        if (c < nch_row) {
            const uint32_t bits = (smask[c >> 2] >> ((c & 3) * 8)) & 0xffu;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (r < s) {
                    const uint32_t w[4] = {v[cc][r].x, v[cc][r].y, v[cc][r].z, v[cc][r].w};
                    const float sc = rscale[r];
                    uint32_t packed[2] = {0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const uint32_t xb = (w[e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                        const bool out = (bits >> e) & 1u;
                        int qv = out ? 0 : quantize_one(half_bits_to_float(xb), sc);
                        packed[e >> 2] |= (static_cast<uint32_t>(qv) & 0xffu) << ((e & 3) * 8);
                        if (out) X_O[r * ldo + outlier_rank(smask, pre, c * 8 + e)] = static_cast<uint16_t>(xb);
                    }
                    *reinterpret_cast<uint2*>(Xq + static_cast<int64_t>(r) * h + c * 8) = make_uint2(packed[0], packed[1]);
                }
            }
        }
    }
    const int npad = (n + 31) & ~31;
    for (int r = 0; r < s; ++r)
        for (int k = n + t; k < npad; k += kSmallThreads) X_O[r * ldo + k] = 0;
    emit_outlier_set(smask, pre, nw, n, mask, idx, n_out, kSmallThreads);
}

// ---------------------------------------------------------------------------
// Load-time column-wise quantisation of W [h, o] into Wq_t [o, h]
// ([DIGEST] "The Full LLM.int8() Algorithm", Step 4; "Why vector-wise
// rather than row-wise": constants computed once at load time).
//
// One 256-thread block per 64-column strip. Pass 1: per-column absmax over
// all h rows (thread = 8 columns x every 32nd row; one wavefront reads 8
// rows x 128 bytes). Pass 2: 64x64 tiles are quantised, transposed through
// LDS and written as 16-byte runs of Wq_t rows.
__global__ __launch_bounds__(256) void k_quant_cols(const uint16_t* __restrict__ W, int64_t h, int64_t o,
                                                    int8_t* __restrict__ Wq_t, float* __restrict__ c_w) {
    __shared__ float red[32][65];
    __shared__ float scale[64];
    __shared__ __attribute__((aligned(16))) int8_t tile[64][80];
    const int t = threadIdx.x;
    const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int cc = t & 7, rg = t >> 3;

    float m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = 0.0f;
    for (int64_t r = rg; r < h; r += 32) {
        uint4 v = *reinterpret_cast<const uint4*>(W + r * o + j0 + cc * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            m[e] = fmaxf(m[e], fabsf(half_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu)));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg][cc * 8 + e] = m[e];
    __syncthreads();
    if (t < 64) {
        float mm = 0.0f;
        for (int g = 0; g < 32; ++g) mm = fmaxf(mm, red[g][t]);
        const float sc = absmax_scale(mm);
        scale[t] = sc;
        c_w[j0 + t] = sc;
    }
    __syncthreads();

    for (int64_t r0 = 0; r0 < h; r0 += 64) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int q = t + 256 * p;
            const int row = q >> 3, ch = q & 7;
            uint4 v = *reinterpret_cast<const uint4*>(W + (r0 + row) * o + j0 + ch * 8);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = half_bits_to_float((w[e >> 1] >> ((e & 1) * 16)) & 0xffffu);
                tile[ch * 8 + e][row] = static_cast<int8_t>(quantize_one(x, scale[ch * 8 + e]));
            }
        }
        __syncthreads();
        const int col = t >> 2, seg = t & 3;
        *reinterpret_cast<uint4*>(Wq_t + (j0 + col) * h + r0 + seg * 16) =
            *reinterpret_cast<const uint4*>(&tile[col][seg * 16]);
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_detect(const uint16_t* X, int64_t s, int64_t h, float alpha,
                         uint32_t* mask, int32_t* idx, int32_t* n_out, hipStream_t stream) {
    const int64_t nw = (h + 31) / 32;
    hipLaunchKernelGGL(k_fill_u32, dim3(static_cast<unsigned>((nw + 255) / 256)), dim3(256), 0, stream,
                       mask, nw, 0u);
    const int64_t n_cb = (h + kDetectCols - 1) / kDetectCols;
    // Aim for about 2048 blocks; at least 4 rows per thread for load overlap.
    int64_t rows = (s * n_cb + 2047) / 2048;
    if (rows < 4) rows = 4;
    const int64_t n_rb = (s + rows - 1) / rows;
    hipLaunchKernelGGL(k_detect, dim3(static_cast<unsigned>(n_cb * n_rb)), dim3(256), 0, stream,
                       X, s, h, alpha, static_cast<int>(rows), n_cb, mask);
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, stream, mask, static_cast<int>(nw), idx, n_out);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* X, int64_t s, int64_t h,
                                const uint32_t* mask, const int32_t* idx, const int32_t* n_out,
                                int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo,
                                hipStream_t stream) {
    const int64_t nch = h / 8;
    const dim3 grid(static_cast<unsigned>(s)), block(256);
    if (nch <= 256)
        hipLaunchKernelGGL(k_quant_rows<1>, grid, block, 0, stream, X, h, mask, idx, n_out, Xq, c_x, X_O, ldo);
    else if (nch <= 512)
        hipLaunchKernelGGL(k_quant_rows<2>, grid, block, 0, stream, X, h, mask, idx, n_out, Xq, c_x, X_O, ldo);
    else if (nch <= 1024)
        hipLaunchKernelGGL(k_quant_rows<4>, grid, block, 0, stream, X, h, mask, idx, n_out, Xq, c_x, X_O, ldo);
    else if (nch <= 2048)
        hipLaunchKernelGGL(k_quant_rows<8>, grid, block, 0, stream, X, h, mask, idx, n_out, Xq, c_x, X_O, ldo);
    else
        hipLaunchKernelGGL(k_quant_rows<0>, grid, block, 0, stream, X, h, mask, idx, n_out, Xq, c_x, X_O, ldo);
    return hipGetLastError();
}

hipError_t launch_forward_prologue(const uint16_t* X, int64_t s, int64_t h, float alpha, uint32_t* acc,
                                   uint32_t* mask, int32_t* idx, int32_t* n_out, int8_t* Xq, float* c_x,
                                   uint16_t* X_O, int64_t ldo, hipStream_t stream, bool* acc_used) {
    const int64_t nw = h / 32;
    const size_t dyn = static_cast<size_t>(2 * nw * 4);
    const int64_t cc = (h + 8 * kSmallThreads - 1) / (8 * kSmallThreads);   // column chunks per thread
    if (cc <= 2 && s * cc <= kSmallMaxRows) {
        *acc_used = false;
        if (cc == 1)
            hipLaunchKernelGGL(k_prologue_small<1>, dim3(1), dim3(kSmallThreads), dyn, stream, X, static_cast<int>(s),
                               static_cast<int>(h), alpha, mask, idx, n_out, Xq, c_x, X_O, ldo);
        else
            hipLaunchKernelGGL(k_prologue_small<2>, dim3(1), dim3(kSmallThreads), dyn, stream, X, static_cast<int>(s),
                               static_cast<int>(h), alpha, mask, idx, n_out, Xq, c_x, X_O, ldo);
        return hipGetLastError();
    }
    *acc_used = true;
    const int64_t n_cb = (h + kDetectCols - 1) / kDetectCols;
    int64_t rows = (s * n_cb + 2047) / 2048;
    if (rows < 4) rows = 4;
    const int64_t n_rb = (s + rows - 1) / rows;
    hipLaunchKernelGGL(k_detect, dim3(static_cast<unsigned>(n_cb * n_rb)), dim3(256), 0, stream,
                       X, s, h, alpha, static_cast<int>(rows), n_cb, acc);
    const int64_t nch = h / 8;
    const dim3 grid(static_cast<unsigned>(s)), block(256);
    if (nch <= 256)
        hipLaunchKernelGGL(k_quant_rows_acc<1>, grid, block, dyn, stream, X, h, acc, mask, idx, n_out, Xq, c_x, X_O, ldo);
    else if (nch <= 512)
        hipLaunchKernelGGL(k_quant_rows_acc<2>, grid, block, dyn, stream, X, h, acc, mask, idx, n_out, Xq, c_x, X_O, ldo);
    else if (nch <= 1024)
        hipLaunchKernelGGL(k_quant_rows_acc<4>, grid, block, dyn, stream, X, h, acc, mask, idx, n_out, Xq, c_x, X_O, ldo);
    else if (nch <= 2048)
        hipLaunchKernelGGL(k_quant_rows_acc<8>, grid, block, dyn, stream, X, h, acc, mask, idx, n_out, Xq, c_x, X_O, ldo);
    else
        hipLaunchKernelGGL(k_quant_rows_acc<0>, grid, block, dyn, stream, X, h, acc, mask, idx, n_out, Xq, c_x, X_O, ldo);
    return hipGetLastError();
}

hipError_t launch_quantize_cols(const uint16_t* W, int64_t h, int64_t o,
                                int8_t* Wq_t, float* c_w, hipStream_t stream) {
    hipLaunchKernelGGL(k_quant_cols, dim3(static_cast<unsigned>(o / 64)), dim3(256), 0, stream,
                       W, h, o, Wq_t, c_w);
    return hipGetLastError();
}

}  // namespace i8mm
