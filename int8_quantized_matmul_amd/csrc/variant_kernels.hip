// Zeropoint (asymmetric) quantisation kernels for gfx950: the quantiser the
// pages compare with absmax before choosing absmax for the int8 path.
//
// Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for
// Transformers at Scale" (paper-graph-ui digest), "Quantization Primitives:
// Absmax and Zeropoint Quantization" (nd = 2 * 127 / (max - min), a zero
// point, the four-term product) and "Vector-wise Quantization" (Table 1's
// zeropoint vector-wise row); [PY] "LLM.int8() 完全拆解" (pinghaoyang.com.cn),
// "量化为什么会崩：一个尺度统治全局" (the zero point and the four-term product).
//
// Each row of X (over the columns not in O) and each column of W gets
//   nd = fl32(254 / fl32(max - min))   (1 when max == min),
//   zp = round(fl32(nd * min)) + 127,
//   q  = clamp(round(fl32(nd * x)) - zp, -127, 127),
// rounding half away from zero, so that q + zp approximates nd * x: the
// form in which the product adds the zero points back,
//   C'_ij = sum over k not in O of (q_x,ik + zp_x,i)(q_w,kj + zp_w,j),
// evaluated by the product kernel from the int8 product and the code sums
// written here (rowsum_x, colsum_w). The pages print the zero point as a
// product of X and its minimum, a garble; the formula above is the reading
// under which the codes fill [-127, 127] and the four-term product holds.

#include "device_common.h"
#include "launch.h"
#include "quant_common.h"

namespace i8mm {
namespace {

// round half away from zero of an fp32 value v with |v| < 2^31: adding the
// largest float below 1/2 with v's sign, then truncating (the conversion
// truncates), moves exactly the ties and everything above them to the next
// integer, for every magnitude (below 2^22 the sum rounds to the integer
// below or above as the fraction is < or >= 1/2; above, v is already a
// multiple of 1/2).
__device__ __forceinline__ int round_half_away_int(float v) {
    return static_cast<int>(__fadd_rn(v, copysignf(0.49999997f, v)));
}

struct ZeroPoint {
    float nd;
    int zp;
};

__device__ __forceinline__ ZeroPoint zeropoint_of(float lo, float hi) {
    const float span = __fsub_rn(hi, lo);
    const float nd = span > 0.0f ? __fdiv_rn(254.0f, span) : 1.0f;
    return ZeroPoint{nd, round_half_away_int(__fmul_rn(nd, lo)) + 127};
}

__device__ __forceinline__ int zeropoint_code(float x, const ZeroPoint& z) {
    const int q = round_half_away_int(__fmul_rn(x, z.nd)) - z.zp;
    return q < -127 ? -127 : (q > 127 ? 127 : q);
}

__device__ __forceinline__ float half_at(const uint4& v, int e) {
    return half_bits_to_float((word_of(v, e >> 1) >> ((e & 1) * 16)) & 0xffffu);
}

// ---------------------------------------------------------------------------
// Rows of X: one wavefront per row, four rows per block sharing an LDS copy
// of the mask and its prefix counts. Pass 1 sends the outlier values to X_O
// at their rank and takes min and max over the other values; pass 2
// re-reads the row (an L2 hit), writes the codes (0 in the outlier columns)
// and sums them. Dynamic LDS: nw mask words + nw prefix counts.
__global__ __launch_bounds__(256) void k_quant_rows_zp(const uint16_t* __restrict__ X, int64_t s, int64_t h,
                                                       const uint32_t* __restrict__ mask, int8_t* __restrict__ Xq,
                                                       float* __restrict__ nd_x, int32_t* __restrict__ zp_x,
                                                       int32_t* __restrict__ rowsum_x, uint16_t* __restrict__ X_O,
                                                       int64_t ldo, uint32_t* __restrict__ mask_out,
                                                       int32_t* __restrict__ idx, int32_t* __restrict__ n_out) {
    extern __shared__ uint32_t dyn[];
    __shared__ int wsum[4];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int nw = static_cast<int>(h / 32);
    uint32_t* smask = dyn;
    int* pre = reinterpret_cast<int*>(dyn + nw);
    for (int w = t; w < nw; w += 256) smask[w] = mask[w];
    __syncthreads();
    const int n = block_mask_prefix(smask, pre, nw, wsum, 256);
    if (blockIdx.x == 0 && idx != nullptr) emit_outlier_set(smask, pre, nw, n, mask_out, idx, n_out, 256);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 4 + wid;
    if (i >= s) return;

    const uint16_t* xr = X + i * h;
    uint16_t* orow = X_O + i * ldo;
    const int64_t nch = h / 8;
    auto bits_of = [&](int64_t c) { return (smask[c >> 2] >> ((c & 3) * 8)) & 0xffu; };
    float lo = INFINITY, hi = -INFINITY;
    for (int64_t c = lane; c < nch; c += 64) {
        const uint4 v = load_chunk(xr + c * 8);
        const uint32_t bits = bits_of(c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if ((bits >> e) & 1u) {
                orow[outlier_rank(smask, pre, static_cast<int>(c * 8 + e))] =
                    static_cast<uint16_t>(word_of(v, e >> 1) >> ((e & 1) * 16));
            } else {
                const float x = half_at(v, e);
                lo = fminf(lo, x);
                hi = fmaxf(hi, x);
            }
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
    }
    if (lo > hi) lo = hi = 0.0f;   // every column is an outlier
    const ZeroPoint z = zeropoint_of(lo, hi);

    int8_t* qr = Xq + i * h;
    int sum = 0;
    for (int64_t c = lane; c < nch; c += 64) {
        const uint4 v = load_chunk(xr + c * 8);
        const uint32_t bits = bits_of(c);
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int q = (bits >> e) & 1u ? 0 : zeropoint_code(half_at(v, e), z);
            sum += q;
            packed[e >> 2] |= (static_cast<uint32_t>(q) & 0xffu) << ((e & 3) * 8);
        }
        *reinterpret_cast<uint2*>(qr + c * 8) = make_uint2(packed[0], packed[1]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
    if (lane == 0) {
        nd_x[i] = z.nd;
        zp_x[i] = z.zp;
        rowsum_x[i] = sum;
    }
    const int npad = (n + 31) & ~31;
    for (int k = n + lane; k < npad; k += 64) orow[k] = 0;
}

// ---------------------------------------------------------------------------
// The same with the row held in registers and split over WPR wavefronts
// (4 / WPR rows per block; part q of a row owns its 8-column chunks
// 64 (WPR p + q) + lane, p < CPL), as the absmax row quantiser does: X is
// read once, the outlier values go to X_O straight from the registers, min
// and max exclude the outlier columns, and the parts of a row meet in LDS
// for min, max and the code sum. The codes are those of k_quant_rows_zp
// (same zeropoint_of / zeropoint_code). If idx is non-null, block 0 also
// writes the index list and |O| (and the mask to mask_out if that is
// non-null), as the absmax row quantiser does. Dynamic LDS: nw mask words +
// nw prefix counts.
template <int CPL, int WPR>
__global__ __launch_bounds__(256) void k_quant_rows_zp_reg(const uint16_t* __restrict__ X, int64_t s, int64_t h,
                                                           const uint32_t* __restrict__ mask,
                                                           int8_t* __restrict__ Xq, float* __restrict__ nd_x,
                                                           int32_t* __restrict__ zp_x, int32_t* __restrict__ rowsum_x,
                                                           uint16_t* __restrict__ X_O, int64_t ldo,
                                                           uint32_t* __restrict__ mask_out, int32_t* __restrict__ idx,
                                                           int32_t* __restrict__ n_out) {
    extern __shared__ uint32_t dyn[];
    __shared__ int wsum[4];
    __shared__ float part_lo[4], part_hi[4];
    __shared__ int part_sum[4];
    // wavefront index in a scalar register (uniform row descriptor)
    const int t = threadIdx.x, lane = t & 63, wid = __builtin_amdgcn_readfirstlane(t >> 6);
    const int part = wid % WPR;
    const int nw = static_cast<int>(h / 32);
    uint32_t* smask = dyn;
    int* pre = reinterpret_cast<int*>(dyn + nw);
    const int64_t i = static_cast<int64_t>(blockIdx.x) * (4 / WPR) + wid / WPR;
    const bool live = i < s;
    const uint16_t* xr = X + (live ? i : 0) * h;
    const int64_t nch = h / 8;
    auto chunk_of = [&](int p) -> int64_t { return 64 * (WPR * p + part) + lane; };

    // mask words first, then the row (chunks past the row, and every chunk
    // of a row past s, read zero)
    uint32_t mw = 0u;
    if (t < nw) mw = mask[t];
    const __amdgpu_buffer_rsrc_t rrow = range_rsrc(xr, live ? static_cast<uint32_t>(2 * h) : 0u);
    uint4 cache[CPL];
#pragma unroll
    for (int p = 0; p < CPL; ++p) cache[p] = load_chunk_rsrc(rrow, static_cast<uint32_t>(chunk_of(p) * 16));
    if (t < nw) smask[t] = mw;
    for (int w = t + 256; w < nw; w += 256) smask[w] = mask[w];   // h > 8192
    __syncthreads();
    const int n = block_mask_prefix(smask, pre, nw, wsum, 256);
    if (blockIdx.x == 0 && idx != nullptr) emit_outlier_set(smask, pre, nw, n, mask_out, idx, n_out, 256);

    uint16_t* orow = X_O + i * ldo;
    auto bits_of = [&](int64_t c) { return (smask[c >> 2] >> ((c & 3) * 8)) & 0xffu; };
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int p = 0; p < CPL; ++p) {
        const int64_t c = chunk_of(p);
        if (c >= nch) continue;
        const uint32_t bits = bits_of(c);
        if (bits && live) {
            const int w = static_cast<int>(c >> 2), sh = static_cast<int>(c & 3) * 8;
            int rank = pre[w] + __popc(smask[w] & ((1u << sh) - 1u));
            for (uint32_t b = bits; b; b &= b - 1u) {
                const int e = __ffs(b) - 1;
                orow[rank++] = static_cast<uint16_t>(word_of(cache[p], e >> 1) >> ((e & 1) * 16));
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!((bits >> e) & 1u)) {
                const float x = half_at(cache[p], e);
                lo = fminf(lo, x);
                hi = fmaxf(hi, x);
            }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, off, kWave));
        hi = fmaxf(hi, __shfl_xor(hi, off, kWave));
    }
    if constexpr (WPR > 1) {
        if (lane == 0) {
            part_lo[wid] = lo;
            part_hi[wid] = hi;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < WPR; ++q) {
            lo = fminf(lo, part_lo[wid - part + q]);
            hi = fmaxf(hi, part_hi[wid - part + q]);
        }
    }
    if (lo > hi) lo = hi = 0.0f;   // every column is an outlier
    const ZeroPoint z = zeropoint_of(lo, hi);

    int8_t* qr = Xq + i * h;
    int sum = 0;
#pragma unroll
    for (int p = 0; p < CPL; ++p) {
        const int64_t c = chunk_of(p);
        if (c >= nch) continue;
        const uint32_t bits = bits_of(c);
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int q = (bits >> e) & 1u ? 0 : zeropoint_code(half_at(cache[p], e), z);
            sum += q;
            packed[e >> 2] |= (static_cast<uint32_t>(q) & 0xffu) << ((e & 3) * 8);
        }
        if (live) *reinterpret_cast<uint2*>(qr + c * 8) = make_uint2(packed[0], packed[1]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
    if constexpr (WPR > 1) {
        if (lane == 0) part_sum[wid] = sum;
        __syncthreads();
        sum = 0;
#pragma unroll
        for (int q = 0; q < WPR; ++q) sum += part_sum[wid - part + q];
    }
    if (!live) return;
    if (lane == 0 && part == 0) {
        nd_x[i] = z.nd;
        zp_x[i] = z.zp;
        rowsum_x[i] = sum;
    }
    const int npad = (n + 31) & ~31;
    if (part == 0)
        for (int k = n + lane; k < npad; k += 64) orow[k] = 0;
}

// ---------------------------------------------------------------------------
// Columns of W (load time) into the panel layout Wq [h / 64][o][64], as
// k_quant_cols does for absmax: one 256-thread block per 64-column strip;
// pass 1 takes min and max per column over all h rows, pass 2 quantises
// 64 x 64 tiles, transposes them through LDS into the strip's 4 KiB of each
// panel, and sums each column's codes.
__global__ __launch_bounds__(256) void k_quant_cols_zp(const uint16_t* __restrict__ W, int64_t h, int64_t o,
                                                       int8_t* __restrict__ Wq, float* __restrict__ nd_w,
                                                       int32_t* __restrict__ zp_w, int32_t* __restrict__ colsum_w) {
    __shared__ float rlo[32][65];
    __shared__ float rhi[32][65];
    __shared__ int rsum[32][65];
    __shared__ ZeroPoint zps[64];
    __shared__ __attribute__((aligned(16))) int8_t tile[64][80];
    const int t = threadIdx.x;
    const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int cc = t & 7, rg = t >> 3;

    float lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] = INFINITY;
        hi[e] = -INFINITY;
    }
    for (int64_t r = rg; r < h; r += 32) {
        const uint4 v = load_chunk(W + r * o + j0 + cc * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = half_at(v, e);
            lo[e] = fminf(lo[e], x);
            hi[e] = fmaxf(hi[e], x);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        rlo[rg][cc * 8 + e] = lo[e];
        rhi[rg][cc * 8 + e] = hi[e];
    }
    __syncthreads();
    if (t < 64) {
        float l = INFINITY, u = -INFINITY;
        for (int g = 0; g < 32; ++g) {
            l = fminf(l, rlo[g][t]);
            u = fmaxf(u, rhi[g][t]);
        }
        const ZeroPoint z = zeropoint_of(l, u);
        zps[t] = z;
        nd_w[j0 + t] = z.nd;
        zp_w[j0 + t] = z.zp;
    }
    __syncthreads();

    // Thread t always handles the 8 columns (t % 8) * 8 .. + 7.
    int csum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int64_t r0 = 0; r0 < h; r0 += 64) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int q = t + 256 * p;
            const int row = q >> 3, ch = q & 7;
            const uint4 v = load_chunk(W + (r0 + row) * o + j0 + ch * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int code = zeropoint_code(half_at(v, e), zps[ch * 8 + e]);
                csum[e] += code;
                tile[ch * 8 + e][row] = static_cast<int8_t>(code);
            }
        }
        __syncthreads();
        const int col = t >> 2, seg = t & 3;
        *reinterpret_cast<uint4*>(Wq + (r0 / 64) * o * 64 + (j0 + col) * 64 + seg * 16) =
            *reinterpret_cast<const uint4*>(&tile[col][seg * 16]);
        __syncthreads();
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) rsum[rg][cc * 8 + e] = csum[e];
    __syncthreads();
    if (t < 64) {
        int sum = 0;
        for (int g = 0; g < 32; ++g) sum += rsum[g][t];
        colsum_w[j0 + t] = sum;
    }
}

}  // namespace

hipError_t launch_quantize_rows_zp(const uint16_t* X, int64_t s, int64_t h, const uint32_t* mask, int8_t* Xq,
                                   float* nd_x, int32_t* zp_x, int32_t* rowsum_x, uint16_t* X_O, int64_t ldo,
                                   hipStream_t stream, uint32_t* mask_out, int32_t* idx, int32_t* n_out) {
    const size_t dyn = static_cast<size_t>(2 * (h / 32) * 4);
    // Wavefronts per row as for the absmax row quantiser: ~4096 wavefronts
    // in all while each holds at most 16 chunks of its row.
    const int64_t nch = h / 8;
    int wpr = s >= 4096 ? 1 : s >= 2048 ? 2 : 4;
    while (wpr > 1 && (nch + 64 * wpr - 1) / (64 * wpr) > 16) wpr = wpr == 4 ? 1 : 4;
    const int64_t per_lane = (nch + 64 * wpr - 1) / (64 * wpr);
    if (per_lane > 16) {
        // long rows: one wavefront per row reading it twice
        hipLaunchKernelGGL(k_quant_rows_zp, dim3(static_cast<unsigned>((s + 3) / 4)), dim3(256), dyn, stream, X, s,
                           h, mask, Xq, nd_x, zp_x, rowsum_x, X_O, ldo, mask_out, idx, n_out);
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>((s + 4 / wpr - 1) / (4 / wpr))), block(256);
#define I8MM_ZPROWS(CPL, W)                                                                                      \
    hipLaunchKernelGGL((k_quant_rows_zp_reg<CPL, W>), grid, block, dyn, stream, X, s, h, mask, Xq, nd_x, zp_x,    \
                       rowsum_x, X_O, ldo, mask_out, idx, n_out)
#define I8MM_ZPROWS_W(W)                                 \
    if (per_lane <= 2) I8MM_ZPROWS(2, W);                \
    else if (per_lane <= 4) I8MM_ZPROWS(4, W);           \
    else if (per_lane <= 8) I8MM_ZPROWS(8, W);           \
    else I8MM_ZPROWS(16, W);
    if (wpr == 4) {
        I8MM_ZPROWS_W(4)
    } else if (wpr == 2) {
        I8MM_ZPROWS_W(2)
    } else {
        I8MM_ZPROWS_W(1)
    }
#undef I8MM_ZPROWS_W
#undef I8MM_ZPROWS
    return hipGetLastError();
}

hipError_t launch_quantize_cols_zp(const uint16_t* W, int64_t h, int64_t o, int8_t* Wq, float* nd_w, int32_t* zp_w,
                                   int32_t* colsum_w, hipStream_t stream) {
    hipLaunchKernelGGL(k_quant_cols_zp, dim3(static_cast<unsigned>(o / 64)), dim3(256), 0, stream, W, h, o, Wq, nd_w,
                       zp_w, colsum_w);
    return hipGetLastError();
}

}  // namespace i8mm
