// Bandwidth-bound kernels of the LLM.int8() path for gfx950: outlier-column
// detection, the index list of the outlier set, row-wise absmax quantisation
// with the outlier gather, and load-time column-wise weight quantisation.
//
// Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for
// Transformers at Scale" (paper-graph-ui digest); [TM] transformer-math
// LLM.int8() tutorial (aicassindra.com).
//
// X is read as 16-byte chunks of 8 fp16 values and handled two values per
// 32-bit word with packed 16-bit integer operations where the result is
// exact: for non-NaN fp16 values, the bit patterns of |x| (sign bit
// cleared) order like the values, so maxima and threshold tests run on
// them directly.

#include "device_common.h"
#include "launch.h"
#include "quant_common.h"

#include <cmath>

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
// Outlier-column detection into a mask. One block per (512-column strip,
// 32-row block): wavefront w folds rows 8 w .. 8 w + 7 of the block into
// its lanes' detection state (each lane owns 8 columns and keeps its 8 row
// loads in flight at once), the 4 lanes of a mask word combine through
// shuffles, the 4 wavefronts meet in LDS, and each non-zero word of the
// strip reaches the mask with one atomicOr per block (the mask must be zero
// beforehand). Same-address global atomics serialise, so the per-block
// merge keeps their count per word at s / 32.
constexpr int kDetRows = 32;

__global__ __launch_bounds__(256) void k_detect(const uint16_t* __restrict__ X, int64_t s, int64_t h,
                                                Threshold th, int64_t n_strips, uint32_t* __restrict__ mask) {
    __shared__ uint32_t words[16];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    if (t < 16) words[t] = 0u;
    // 32-bit division (the grid is 32-bit): short ahead of the loads
    const uint32_t ns32 = static_cast<uint32_t>(n_strips);
    const int64_t strip = blockIdx.x % ns32, rb = blockIdx.x / ns32;
    const int64_t col = strip * 512 + lane * 8;
    const int64_t r0 = rb * kDetRows + wid * 8;
    uint32_t flags = 0;
    if (col < h) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = r0 + u < s ? load_chunk(X + (r0 + u) * h + col) : make_uint4(0, 0, 0, 0);
        uint4 d = detect_init();
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (r0 + u < s) detect_fold(d, v[u], th.thr2);
        flags = detect_flags(d, th.span);
    }
    uint32_t word = flags << ((lane & 3) * 8);
    word |= __shfl_xor(word, 1, kWave);
    word |= __shfl_xor(word, 2, kWave);
    __syncthreads();
    if ((lane & 3) == 0 && word != 0u) atomicOr(&words[lane >> 2], word);
    __syncthreads();
    if (t < 16 && words[t] != 0u) atomicOr(&mask[strip * 16 + t], words[t]);
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

// ---------------------------------------------------------------------------
// Row-wise absmax quantisation over the non-outlier columns plus the gather
// of the outlier columns ([DIGEST] "The Full LLM.int8() Algorithm", Steps 2
// and 4; [TM] "Absmax INT8 quantization from first principles").
//
// One wavefront per row, four rows per block sharing an LDS copy of the
// mask (read from `src_mask`) and its prefix counts, so that the rank of an
// outlier column in O (the number of set mask bits below it) places it in
// X_O straight from the registers. Lane l owns the 8-column chunks
// l, l + 64, ...: chunks holding outlier columns first send those values to
// X_O and replace them by +0, after which the absmax and the quantisation
// run over whole chunks (a zero neither raises the maximum nor yields a
// non-zero code). With CPL > 0 the row stays in registers (CPL chunks per
// lane), otherwise the second pass re-reads it (an L2 hit). If idx is
// non-null, block 0 also writes the index list and |O| (and the mask to
// `mask_out` if that is non-null).
// SC selects where the scale comes from: Absmax (the row's own, written to
// c_x), MaxOnly (only the row's absmax over the non-outlier columns is
// written, as a float, to c_x; nothing else), or Given (c_x[i] already holds
// the scale, e.g. one constant for the whole tensor, and is only read).
// Dynamic LDS: nw mask words + nw prefix counts.
enum class RowScale { Absmax, MaxOnly, Given };

// WPR wavefronts share a row (4 / WPR rows per block; wavefront part q of a
// row owns its chunks 64 (WPR p + q) + lane) and meet in LDS for the row
// maximum, so that few rows still give the GPU enough wavefronts; WPR > 1
// only with the row held in registers.
template <int CPL, RowScale SC = RowScale::Absmax, int WPR = 1>
__global__ __launch_bounds__(256) void k_quant_rows(const uint16_t* __restrict__ X, int64_t s, int64_t h,
                                                    const uint32_t* __restrict__ src_mask,
                                                    uint32_t* __restrict__ mask_out, int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ n_out,
                                                    int8_t* __restrict__ Xq, float* __restrict__ c_x,
                                                    uint16_t* __restrict__ X_O, int64_t ldo) {
    static_assert(WPR == 1 || CPL > 0, "row split needs the row in registers");
    extern __shared__ uint32_t dyn[];
    __shared__ int wsum[4];
    __shared__ uint32_t part_max[4];
    // wavefront index in a scalar register: the row's buffer descriptor is
    // then known to be uniform (in vector registers it costs a loop around
    // every load)
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

    // The mask words are loaded before the row, so that the prefix counts
    // below wait only for them (vector-memory waits are in issue order) and
    // run while the row is still in flight.
    uint32_t mw = 0u;
    if (t < nw) mw = src_mask[t];
    uint4 cache[CPL > 0 ? CPL : 1];
    if constexpr (CPL > 0) {
        // chunks past the row, and every chunk of a row past s, read zero
        const __amdgpu_buffer_rsrc_t rrow = range_rsrc(xr, live ? static_cast<uint32_t>(2 * h) : 0u);
#pragma unroll
        for (int p = 0; p < CPL; ++p) cache[p] = load_chunk_rsrc(rrow, static_cast<uint32_t>(chunk_of(p) * 16));
    }
    if (t < nw) smask[t] = mw;
    for (int w = t + 256; w < nw; w += 256) smask[w] = src_mask[w];   // h > 8192
    __syncthreads();
    const int n = block_mask_prefix(smask, pre, nw, wsum, 256);
    if (blockIdx.x == 0 && idx != nullptr) emit_outlier_set(smask, pre, nw, n, mask_out, idx, n_out, 256);
    if constexpr (WPR == 1) {
        if (!live) return;
    }

    uint16_t* orow = X_O + i * ldo;
    auto bits_of = [&](int64_t c) { return (smask[c >> 2] >> ((c & 3) * 8)) & 0xffu; };
    // Outlier values to X_O; the chunk comes back with them cleared. The
    // chunk's first outlier column takes rank pre[word] plus the set bits
    // below it in its word, the next ones follow in order; the loop runs
    // once per outlier column in the chunk (usually none).
    auto split = [&](const uint4& v, int64_t c) {
        const uint32_t bits = bits_of(c);
        if (!bits || !live) return v;   // a row past s holds zeros (WPR > 1 only)
        if constexpr (SC == RowScale::MaxOnly) return chunk_clear(v, bits);
        const int w = static_cast<int>(c >> 2), sh = static_cast<int>(c & 3) * 8;
        int rank = pre[w] + __popc(smask[w] & ((1u << sh) - 1u));
        for (uint32_t b = bits; b; b &= b - 1u) {
            const int e = __ffs(b) - 1;
            orow[rank++] = static_cast<uint16_t>(word_of(v, e >> 1) >> ((e & 1) * 16));
        }
        return chunk_clear(v, bits);
    };
    uint32_t m2 = 0;
    if constexpr (CPL > 0) {
#pragma unroll
        for (int p = 0; p < CPL; ++p) {
            const int64_t c = chunk_of(p);
            if (c < nch) {
                cache[p] = split(cache[p], c);
                m2 = chunk_absmax_fold(cache[p], m2);
            }
        }
    } else {
        for (int64_t c = lane; c < nch; c += 64) m2 = chunk_absmax_fold(split(load_chunk(xr + c * 8), c), m2);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m2 = pk_max_u16(m2, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m2), off, kWave)));
    if constexpr (WPR > 1) {
        if (lane == 0) part_max[wid] = m2;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < WPR; ++q) m2 = pk_max_u16(m2, part_max[wid - part + q]);
        if (!live) return;
    }
    if constexpr (SC == RowScale::MaxOnly) {
        if (lane == 0 && part == 0) c_x[i] = absmax_value(m2);
        return;
    }
    float sc;
    if constexpr (SC == RowScale::Given) {
        sc = c_x[i];
    } else {
        sc = absmax_scale(absmax_value(m2));
        if (lane == 0 && part == 0) c_x[i] = sc;
    }

    // Xq null: the codes are made later, inside the product (c_x, X_O and
    // the outlier set are still written here).
    int8_t* qr = Xq != nullptr ? Xq + i * h : nullptr;
    if constexpr (CPL > 0) {
#pragma unroll
        for (int p = 0; p < CPL; ++p) {
            const int64_t c = chunk_of(p);
            if (qr != nullptr && c < nch) *reinterpret_cast<uint2*>(qr + c * 8) = chunk_quantize(cache[p], sc);
        }
    } else if (qr != nullptr) {
        for (int64_t c = lane; c < nch; c += 64)
            *reinterpret_cast<uint2*>(qr + c * 8) =
                chunk_quantize(chunk_clear(load_chunk(xr + c * 8), bits_of(c)), sc);
    }
    const int npad = (n + 31) & ~31;
    if (part == 0)
        for (int k = n + lane; k < npad; k += 64) orow[k] = 0;
}

// ---------------------------------------------------------------------------
// Forward path for few rows (the one-call forward takes it for s <= 8 when
// X is larger than kOneLaunchBytes, the kernels hold up to 16 RG rows):
// blocks of 256 threads on 128-column
// slabs, thread t on the 8-column chunk t % 16 of rows t / 16 + 16 g,
// g < RG. A block of k_small_detect sees every row of its
// slab, so it writes the slab's mask words itself and folds the per-row
// maxima over its non-outlier columns into `rowmax` with an integer
// atomicMax on the float bits (non-negative floats order like their bit
// patterns); k_small_quant then quantises with the finished row maxima.
// rowmax must be zero beforehand.
constexpr int kSlabCols = 128;
// Up to 8 rows the slab pair and detection + row pass take the same time
// on 12288 columns (~94 us per decode forward); from 16 rows on, detection
// + row pass is 2.6-7.4 us faster per forward (16-64 rows).
constexpr int kSmallRowsMax = 8;
// Up to 8 rows and this many bytes of X, the one-launch prologue
// (k_small_prologue) replaces the slab pair. Measured per forward: 1-8 rows
// on 256 x 512, 10.4-12.4 us against 13.1-14.1; 1-2 rows on 4096 x 16384,
// 17.0-17.2 against 18.0-18.1; one row on 12288 x 49152, 93.2 against 95.5.
// With more of X each block's scan costs more than the second launch (8
// rows on 12288 x 49152: 95.2 against 94.7), and from 9 rows on it lost on
// every width measured (256-12288 columns).
constexpr int64_t kOneLaunchBytes = 24576;

template <int RG>
__global__ __launch_bounds__(256) void k_small_detect(const uint16_t* __restrict__ X, int s, int h, Threshold th,
                                                      uint32_t* __restrict__ mask, uint32_t* __restrict__ rowmax) {
    __shared__ uint32_t smask[kSlabCols / 32];
    const int t = threadIdx.x, c = t & 15, r = t >> 4;
    const int64_t col = static_cast<int64_t>(blockIdx.x) * kSlabCols + c * 8;
    const bool cok = col < h;
    if (t < kSlabCols / 32) smask[t] = 0u;
    // rows past s fall past the resource and read zero; columns past h are
    // sent out of range
    const __amdgpu_buffer_rsrc_t rX = range_rsrc(X, static_cast<uint32_t>(2 * static_cast<int64_t>(s) * h));
    uint4 v[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g)
        v[g] = load_chunk_rsrc(rX, cok ? static_cast<uint32_t>(2 * (static_cast<int64_t>(r + 16 * g) * h + col))
                                       : 0x80000000u);
    uint4 d = detect_init();
#pragma unroll
    for (int g = 0; g < RG; ++g)
        if (cok && r + 16 * g < s) detect_fold(d, v[g], th.thr2);
    const uint32_t flags = detect_flags(d, th.span);
    __syncthreads();
    if (flags) atomicOr(&smask[c >> 2], flags << ((c & 3) * 8));
    __syncthreads();
    const int64_t w0 = static_cast<int64_t>(blockIdx.x) * (kSlabCols / 32);
    if (t < kSlabCols / 32 && w0 + t < h / 32) mask[w0 + t] = smask[t];
    const uint32_t bits = (smask[c >> 2] >> ((c & 3) * 8)) & 0xffu;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int row = r + 16 * g;
        uint32_t m2 = chunk_absmax_fold(chunk_clear(v[g], bits), 0u);
        // the 16 lanes of one row are lanes 16 k .. 16 k + 15 of the wavefront
#pragma unroll
        for (int off = 8; off > 0; off >>= 1)
            m2 = pk_max_u16(m2, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m2), off, kWave)));
        const float m = absmax_value(m2);
        if (c == 0 && row < s && m > 0.0f) atomicMax(&rowmax[row], __float_as_uint(m));
    }
}

template <int RG>
__global__ __launch_bounds__(256) void k_small_quant(const uint16_t* __restrict__ X, int s, int h,
                                                     const uint32_t* __restrict__ mask,
                                                     const uint32_t* __restrict__ rowmax,
                                                     int32_t* __restrict__ idx, int32_t* __restrict__ n_out,
                                                     int8_t* __restrict__ Xq, float* __restrict__ c_x,
                                                     uint16_t* __restrict__ X_O, int64_t ldo) {
    __shared__ int part[2][4];
    __shared__ float rscale[16 * RG];
    __shared__ uint32_t slab[kSlabCols / 32];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6, c = t & 15, r = t >> 4;
    const int nw = h / 32;
    const int w0 = static_cast<int>(blockIdx.x) * (kSlabCols / 32);
    const int64_t col = static_cast<int64_t>(blockIdx.x) * kSlabCols + c * 8;
    const bool cok = col < h;
    // The mask words (the first 512 into registers) and row maxima are
    // loaded before the rows, so that waiting for them does not wait for
    // the rows (vector-memory waits are in issue order).
    const uint32_t mwa = t < nw ? mask[t] : 0u;
    const uint32_t mwb = t + 256 < nw ? mask[t + 256] : 0u;
    const uint32_t rm = t < s ? rowmax[t] : 0u;
    const __amdgpu_buffer_rsrc_t rX = range_rsrc(X, static_cast<uint32_t>(2 * static_cast<int64_t>(s) * h));
    uint4 v[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g)
        v[g] = load_chunk_rsrc(rX, cok ? static_cast<uint32_t>(2 * (static_cast<int64_t>(r + 16 * g) * h + col))
                                       : 0x80000000u);
    // Outlier columns before this slab and in total; this slab's own words
    // go to LDS for the ranks below.
    int before = 0, total = 0;
    auto count = [&](int w, uint32_t word) {
        const int p = __popc(word);
        total += p;
        before += w < w0 ? p : 0;
        if (w >= w0 && w < w0 + kSlabCols / 32) slab[w - w0] = word;
    };
    if (t < nw) count(t, mwa);
    if (t + 256 < nw) count(t + 256, mwb);
    for (int w = t + 512; w < nw; w += 256) count(w, mask[w]);   // h > 16384
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        before += __shfl_xor(before, off, kWave);
        total += __shfl_xor(total, off, kWave);
    }
    if (lane == 0) {
        part[0][wid] = before;
        part[1][wid] = total;
    }
    if (t < s) rscale[t] = absmax_scale(__uint_as_float(rm));
    __syncthreads();
    before = part[0][0] + part[0][1] + part[0][2] + part[0][3];
    total = part[1][0] + part[1][1] + part[1][2] + part[1][3];

    // Rank of this chunk's first outlier column: the slab's words below it,
    // then the bits below it in its own word.
    const int q = c >> 2;
    int rank = before;
    uint32_t word = 0u;
    for (int j = 0; j <= q; ++j) {
        word = w0 + j < nw ? slab[j] : 0u;
        if (j < q) rank += __popc(word);
    }
    rank += __popc(word & ((1u << ((c & 3) * 8)) - 1u));
    const uint32_t bits = (word >> ((c & 3) * 8)) & 0xffu;

#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int row = r + 16 * g;
        if (cok && row < s) {
            if (bits) {
                int k = rank;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if ((bits >> e) & 1u)
                        X_O[row * ldo + k++] = static_cast<uint16_t>(word_of(v[g], e >> 1) >> ((e & 1) * 16));
            }
            *reinterpret_cast<uint2*>(Xq + static_cast<int64_t>(row) * h + col) =
                chunk_quantize(chunk_clear(v[g], bits), rscale[row]);
        }
    }
    if (r == 0 && cok && bits) {
        int k = rank;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((bits >> e) & 1u) idx[k++] = static_cast<int32_t>(col + e);
    }
    if (blockIdx.x == 0) {
        if (t < s) c_x[t] = rscale[t];
        if (t == 0) n_out[0] = total;
        const int pad = ((total + 31) & ~31) - total;
        for (int e = t; e < s * pad; e += 256) X_O[(e / pad) * ldo + total + e % pad] = 0;
    }
}

// ---------------------------------------------------------------------------
// Forward prologue for few rows and small X in one launch: outlier columns,
// row-wise absmax scales over the other columns, codes and the outlier
// gather ([DIGEST] "The Full LLM.int8() Algorithm", Steps 1, 2 and 4; [TM]
// "Absmax INT8 quantization from first principles"). Every block of
// 1024 threads scans all of X (at most R rows): a thread takes 8-column
// chunks with all their rows, so it knows a chunk's outlier flags at once
// and folds the rows' maxima over the non-outlier columns in the same pass.
// The block thus holds the whole mask and the finished row maxima without
// waiting for any other block, and quantises the rows of its own 128-column
// slab as k_small_quant does. Blocks start their scans at staggered chunks,
// so that the blocks sharing an L2 fetch different lines of X first. Max
// and OR do not depend on the order, so the results equal the two-launch
// pair's bit for bit. Each block reads all of X, so this pays only while X
// is small (see kOneLaunchBytes).
template <int R>
__global__ __launch_bounds__(1024) void k_small_prologue(const uint16_t* __restrict__ X, int s, int h, Threshold th,
                                                         uint32_t* __restrict__ mask, int32_t* __restrict__ idx,
                                                         int32_t* __restrict__ n_out, int8_t* __restrict__ Xq,
                                                         float* __restrict__ c_x, uint16_t* __restrict__ X_O,
                                                         int64_t ldo) {
    constexpr int kSlabChunks = kSlabCols / 8;   // 8-column chunks per slab row
    static_assert(R >= 1 && R <= 16 && 16 * kSlabChunks <= 1024, "launch shape");
    extern __shared__ uint32_t smask[];   // h / 32 words
    __shared__ uint32_t pmax[16][R];
    __shared__ int part[2][16];
    __shared__ float rscale[R];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int nw = h / 32, nch = h / 8;
    const __amdgpu_buffer_rsrc_t rX = range_rsrc(X, static_cast<uint32_t>(2 * static_cast<int64_t>(s) * h));

    // This block's slab first, so that its loads are in flight during the scan.
    const int sc = t % kSlabChunks, sr = t / kSlabChunks;
    const int scol = static_cast<int>(blockIdx.x) * kSlabChunks * 8 + sc * 8;
    const bool sok = t < 16 * kSlabChunks && sr < s && scol < h;
    const uint4 sv = load_chunk_rsrc(rX, sok ? static_cast<uint32_t>(2 * (sr * h + scol)) : 0x80000000u);

    // The scan. Four aligned lanes hold the four chunks of one mask word
    // (the start is a multiple of 4 chunks, and so is h / 8).
    const int start = static_cast<int>((static_cast<int64_t>(blockIdx.x) * (nch / 4)) / gridDim.x) * 4;
    uint32_t m2[R];
#pragma unroll
    for (int r = 0; r < R; ++r) m2[r] = 0u;
    for (int base = 0; base < nch; base += 1024) {
        const bool ok = base + t < nch;
        int c = start + base + t;
        if (c >= nch) c -= nch;
        uint4 v[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            v[r] = load_chunk_rsrc(rX, ok ? static_cast<uint32_t>(2 * (r * h + c * 8)) : 0x80000000u);
        uint4 d = detect_init();
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (r < s) detect_fold(d, v[r], th.thr2);
        const uint32_t flags = ok ? detect_flags(d, th.span) : 0u;
#pragma unroll
        for (int r = 0; r < R; ++r) m2[r] = chunk_absmax_fold(chunk_clear(v[r], flags), m2[r]);
        uint32_t word = flags << ((c & 3) * 8);
        word |= __shfl_xor(word, 1, kWave);
        word |= __shfl_xor(word, 2, kWave);
        if (ok && (lane & 3) == 0) smask[c >> 2] = word;
    }
    // The rows' reductions are independent: each level's shuffles issue
    // together (one LDS round trip per level, not one per row and level).
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t o2[R];
#pragma unroll
        for (int r = 0; r < R; ++r) o2[r] = static_cast<uint32_t>(__shfl_xor(static_cast<int>(m2[r]), off, kWave));
#pragma unroll
        for (int r = 0; r < R; ++r) m2[r] = pk_max_u16(m2[r], o2[r]);
    }
    if (lane == 0)
#pragma unroll
        for (int r = 0; r < R; ++r) pmax[wid][r] = m2[r];
    __syncthreads();

    // Outlier columns before this slab and in total; row scales.
    const int w0 = static_cast<int>(blockIdx.x) * (kSlabChunks / 4);
    int before = 0, total = 0;
    for (int w = t; w < nw; w += 1024) {
        const int p = __popc(smask[w]);
        total += p;
        before += w < w0 ? p : 0;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        before += __shfl_xor(before, off, kWave);
        total += __shfl_xor(total, off, kWave);
    }
    if (lane == 0) {
        part[0][wid] = before;
        part[1][wid] = total;
    }
    if (t < R) {
        uint32_t m = 0u;
#pragma unroll
        for (int w = 0; w < 16; ++w) m = pk_max_u16(m, pmax[w][t]);
        rscale[t] = absmax_scale(absmax_value(m));
    }
    __syncthreads();
    before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        before += part[0][w];
        total += part[1][w];
    }

    // Rank of the chunk's first outlier column: the slab's words below it,
    // then the bits below it in its own word.
    const int q = sc >> 2;
    int rank = before;
    uint32_t word = 0u;
    for (int j = 0; j <= q; ++j) {
        word = w0 + j < nw ? smask[w0 + j] : 0u;
        if (j < q) rank += __popc(word);
    }
    rank += __popc(word & ((1u << ((sc & 3) * 8)) - 1u));
    const uint32_t bits = (word >> ((sc & 3) * 8)) & 0xffu;
    if (sok) {
        if (bits) {
            int k = rank;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if ((bits >> e) & 1u) X_O[sr * ldo + k++] = static_cast<uint16_t>(word_of(sv, e >> 1) >> ((e & 1) * 16));
        }
        *reinterpret_cast<uint2*>(Xq + static_cast<int64_t>(sr) * h + scol) =
            chunk_quantize(chunk_clear(sv, bits), rscale[sr]);
    }
    if (t < 16 * kSlabChunks && sr == 0 && scol < h && bits) {
        int k = rank;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((bits >> e) & 1u) idx[k++] = scol + e;
    }
    if (t < kSlabChunks / 4 && w0 + t < nw) mask[w0 + t] = smask[w0 + t];
    if (blockIdx.x == 0) {
        if (t < s) c_x[t] = rscale[t];
        if (t == 0) n_out[0] = total;
        const int pad = ((total + 31) & ~31) - total;
        for (int e = t; e < s * pad; e += 1024) X_O[(e / pad) * ldo + total + e % pad] = 0;
    }
}

// ---------------------------------------------------------------------------
// One absmax constant for a whole tensor ([DIGEST] "Quantization Primitives":
// tensor-wise absmax, 127 over the tensor's largest magnitude) from the
// per-row (or per-column) maxima m[0 .. n): c = fl32(127 / max m) (1 when
// the max is 0) is written over m[0 .. n), so that a per-row (per-column)
// quantiser reading its own entry applies the one constant. One block.
__global__ __launch_bounds__(1024) void k_tensor_scale(float* __restrict__ m, int64_t n) {
    __shared__ float wmax[16];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    float v = 0.0f;
    for (int64_t i = t; i < n; i += 1024) v = fmaxf(v, m[i]);
    v = wave_max(v);
    if (lane == 0) wmax[wid] = v;
    __syncthreads();
    float mx = 0.0f;
#pragma unroll
    for (int w = 0; w < 16; ++w) mx = fmaxf(mx, wmax[w]);
    const float c = absmax_scale(mx);
    for (int64_t i = t; i < n; i += 1024) m[i] = c;
}

// ---------------------------------------------------------------------------
// Load-time column-wise quantisation of W [h, o] into the panel layout
// Wq [h / 64][o][64] (W_i8[k, j] at (k / 64) o 64 + 64 j + k % 64)
// ([DIGEST] "The Full LLM.int8() Algorithm", Step 4; "Why vector-wise
// rather than row-wise": constants computed once at load time), in three
// launches that each cover the whole matrix with many blocks:
//   1. k_col_absmax_part: the largest |W_ij| of each column over each chunk
//      of kColRows rows, as fp16 bit patterns (the patterns of |x| order
//      like the values), into a small array of partial maxima;
//   2. k_col_absmax_reduce: one thread per column takes the largest of its
//      partial maxima and writes c_w_j = fl32(127 / m_j) (MaxOnly: m_j);
//   3. k_quant_panels: one block per 64-row panel and 512 columns quantises
//      the panel with the column constants and writes the columns' 64-code
//      runs, which lie contiguous in the panel.
// The partial maxima live in the Wq buffer itself (h / kColRows rows of o
// patterns, far smaller than h o bytes): the last launch overwrites them
// after the reduction has read them (same stream).
constexpr int kColRows = 256;

__global__ __launch_bounds__(256) void k_col_absmax_part(const uint16_t* __restrict__ W, int64_t h, int64_t o,
                                                         uint16_t* __restrict__ part) {
    __shared__ uint4 red[4][64];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 512 + lane * 8;   // the lane's 8 columns
    const int64_t r0 = static_cast<int64_t>(blockIdx.y) * kColRows;
    const int64_t nrows = h - r0 < kColRows ? h - r0 : kColRows;           // a multiple of 64
    uint32_t m[4] = {0u, 0u, 0u, 0u};
    if (j0 < o) {
        const uint16_t* src = W + r0 * o + j0;
        // wavefront wid reads rows wid, wid + 4, ...: one KiB of one row per
        // load, 16 loads in flight per lane (nrows is a multiple of 64)
        for (int64_t i0 = wid; i0 < nrows; i0 += 64) {
            uint4 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = load_chunk(src + (i0 + 4 * u) * o);
#pragma unroll
            for (int u = 0; u < 16; ++u)
#pragma unroll
                for (int k = 0; k < 4; ++k) m[k] = pk_max_u16(m[k], word_of(v[u], k) & kAbs2);
        }
    }
    red[wid][lane] = make_uint4(m[0], m[1], m[2], m[3]);
    __syncthreads();
    if (wid == 0 && j0 < o) {
        uint4 r = red[0][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const uint4 q = red[w][lane];
            r = make_uint4(pk_max_u16(r.x, q.x), pk_max_u16(r.y, q.y), pk_max_u16(r.z, q.z), pk_max_u16(r.w, q.w));
        }
        *reinterpret_cast<uint4*>(part + static_cast<int64_t>(blockIdx.y) * o + j0) = r;
    }
}

template <RowScale SC>
__global__ __launch_bounds__(256) void k_col_absmax_reduce(const uint16_t* __restrict__ part, int nparts, int64_t o,
                                                           float* __restrict__ c_w) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (j >= o) return;
    uint32_t m = 0;
#pragma unroll 8
    for (int r = 0; r < nparts; ++r) {
        const uint32_t v = part[r * o + j];
        m = v > m ? v : m;
    }
    const float mx = half_bits_to_float(m);
    c_w[j] = SC == RowScale::MaxOnly ? mx : absmax_scale(mx);
}

// Panel quantisation: block = one 64-row panel x 512 columns; wavefront w
// quantises rows 16 w .. 16 w + 15, lane l the 8 columns 8 l .. 8 l + 7
// (one 16-byte load per row: a wavefront reads one KiB of a row at once).
// Each column's 16 codes go to LDS as one 16-byte write at the column's
// 64-byte run; the block then writes its 512 runs (32 KiB, contiguous in
// the panel) with 16-byte stores, one KiB per wavefront store. LDS keeps
// 16 bytes of padding after every 8 columns, so both the 16-byte writes
// (lanes 8 columns apart) and the read-back (4 lanes per column) fill the
// banks without conflicts beyond the passes a 16-byte access needs.
constexpr int kPanelCols = 512;

__device__ __forceinline__ int panel_lds_offset(int col, int seg) { return col * 64 + (col >> 3) * 16 + seg * 16; }

__global__ __launch_bounds__(256) void k_quant_panels(const uint16_t* __restrict__ W, int64_t o,
                                                      const float* __restrict__ c_w, int8_t* __restrict__ Wq) {
    __shared__ __attribute__((aligned(16))) int8_t tile[kPanelCols * 64 + kPanelCols / 8 * 16];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int64_t p = blockIdx.y;                                        // rows 64 p .. 64 p + 63
    const int64_t jb = static_cast<int64_t>(blockIdx.x) * kPanelCols;    // the block's first column
    const int64_t ncols = o - jb < kPanelCols ? o - jb : kPanelCols;     // a multiple of 64
    const int64_t j0 = jb + 8 * lane;
    if (8 * lane < ncols) {
        const uint4 s0 = *reinterpret_cast<const uint4*>(c_w + j0);
        const uint4 s1 = *reinterpret_cast<const uint4*>(c_w + j0 + 4);
        const float sc[8] = {__builtin_bit_cast(float, s0.x), __builtin_bit_cast(float, s0.y),
                             __builtin_bit_cast(float, s0.z), __builtin_bit_cast(float, s0.w),
                             __builtin_bit_cast(float, s1.x), __builtin_bit_cast(float, s1.y),
                             __builtin_bit_cast(float, s1.z), __builtin_bit_cast(float, s1.w)};
        const uint16_t* src = W + (p * 64 + 16 * wid) * o + j0;
        uint4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = load_chunk(src + i * o);
        // codes of column 8 lane + e for the wavefront's 16 rows, 4 rows per word
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t q[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                int c[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t wd = word_of(v[4 * k + r], e >> 1);
                    c[r] = round_code((e & 1) ? mul_half<true>(wd, sc[e]) : mul_half<false>(wd, sc[e]));
                }
                q[k] = pack_bytes(c[0], c[1], c[2], c[3]);
            }
            *reinterpret_cast<uint4*>(tile + panel_lds_offset(8 * lane + e, wid)) = make_uint4(q[0], q[1], q[2], q[3]);
        }
    }
    __syncthreads();
    // the block's runs: bytes 16 i .. 16 i + 15 of the 64 ncols contiguous bytes
    int8_t* dst = Wq + p * o * 64 + jb * 64;
    const int nchunks = static_cast<int>(ncols * 4);
#pragma unroll
    for (int k = 0; k < kPanelCols * 4 / 256; ++k) {
        const int i = t + 256 * k;
        if (i < nchunks)
            *reinterpret_cast<uint4*>(dst + 16 * i) = *reinterpret_cast<const uint4*>(tile + panel_lds_offset(i >> 2, i & 3));
    }
}

// ---------------------------------------------------------------------------
// Load-time packing of fp16 W [h, o] for the dense fp16 product into the
// fp16 panel layout Wp [h / 32][o][32] (W[k, j] at element
// (k / 32) o 32 + 32 j + k % 32): the same 64-byte run per column and panel
// as the int8 layout, holding 32 reduction rows. One block per (64-column
// strip, 32-row panel); the 32 x 64 tile is transposed through LDS and
// written as the strip's contiguous 4 KiB of the panel.
__global__ __launch_bounds__(256) void k_pack_fp16_panels(const uint16_t* __restrict__ W, int64_t o,
                                                          uint16_t* __restrict__ Wp) {
    __shared__ __attribute__((aligned(16))) uint16_t tile[64][40];   // [column][row], rows padded to 80 bytes
    const int t = threadIdx.x;
    const int64_t j0 = static_cast<int64_t>(blockIdx.x) * 64;
    const int64_t p = blockIdx.y;
    const int row = t >> 3, ch = t & 7;
    const uint4 v = load_chunk(W + (p * 32 + row) * o + j0 + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        tile[ch * 8 + e][row] = static_cast<uint16_t>(word_of(v, e >> 1) >> ((e & 1) * 16));
    __syncthreads();
    const int col = t >> 2, seg = t & 3;
    *reinterpret_cast<uint4*>(Wp + (p * o + j0 + col) * 32 + seg * 8) =
        *reinterpret_cast<const uint4*>(&tile[col][seg * 8]);
}

}  // namespace

namespace {

hipError_t launch_detect_into(const uint16_t* X, int64_t s, int64_t h, float alpha, uint32_t* mask,
                              hipStream_t stream) {
    const int64_t n_strips = (h + 511) / 512;
    const int64_t blocks = n_strips * ((s + kDetRows - 1) / kDetRows);
    hipLaunchKernelGGL(k_detect, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       X, s, h, make_threshold(alpha), n_strips, mask);
    return hipGetLastError();
}

hipError_t launch_rows(const uint16_t* X, int64_t s, int64_t h, const uint32_t* src_mask, uint32_t* mask_out,
                       int32_t* idx, int32_t* n_out, int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo,
                       hipStream_t stream) {
    // Wavefronts per row: enough for ~4096 wavefronts in all (4 per SIMD),
    // and more while a lane would hold over 8 chunks of its row (long rows:
    // at 4096 x 12288 four wavefronts per row took the prologue from 54 to
    // 42 us), as long as each still holds its part of the row in registers;
    // rows too long even for four (over 32768 columns) take one wavefront
    // per row that re-reads the row.
    const int64_t nch = h / 8;
    auto per_lane_of = [&](int w) { return (nch + 64 * w - 1) / (64 * w); };
    int wpr = s >= 4096 ? 1 : s >= 2048 ? 2 : 4;
    while (wpr < 4 && per_lane_of(wpr) > 8) wpr *= 2;
    if (per_lane_of(wpr) > 16) wpr = 1;
    const int64_t per_lane = per_lane_of(wpr);
    const dim3 grid(static_cast<unsigned>((s + 4 / wpr - 1) / (4 / wpr))), block(256);
    const size_t dyn = static_cast<size_t>(2 * (h / 32) * 4);
#define I8MM_QROWS(CPL, W)                                                                                     \
    hipLaunchKernelGGL((k_quant_rows<CPL, RowScale::Absmax, W>), grid, block, dyn, stream, X, s, h, src_mask,   \
                       mask_out, idx, n_out, Xq, c_x, X_O, ldo)
#define I8MM_QROWS_W(W)                                  \
    if (per_lane <= 2) I8MM_QROWS(2, W);                 \
    else if (per_lane <= 4) I8MM_QROWS(4, W);            \
    else I8MM_QROWS(8, W);
    if (wpr == 4) {
        if (per_lane <= 8) { I8MM_QROWS_W(4) }
        else I8MM_QROWS(16, 4);
    } else if (wpr == 2) {
        I8MM_QROWS_W(2)
    } else if (per_lane <= 8) {
        I8MM_QROWS_W(1)
    } else {
        I8MM_QROWS(0, 1);
    }
#undef I8MM_QROWS_W
#undef I8MM_QROWS
    return hipGetLastError();
}

}  // namespace

hipError_t launch_detect(const uint16_t* X, int64_t s, int64_t h, float alpha,
                         uint32_t* mask, int32_t* idx, int32_t* n_out, hipStream_t stream) {
    const int64_t nw = (h + 31) / 32;
    hipLaunchKernelGGL(k_fill_u32, dim3(static_cast<unsigned>((nw + 255) / 256)), dim3(256), 0, stream,
                       mask, nw, 0u);
    hipError_t e = launch_detect_into(X, s, h, alpha, mask, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, stream, mask, static_cast<int>(nw), idx, n_out);
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream) {
    hipLaunchKernelGGL(k_fill_u32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, p, n, v);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* X, int64_t s, int64_t h,
                                const uint32_t* mask, const int32_t* idx, const int32_t* n_out,
                                int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo,
                                hipStream_t stream) {
    // The index list and |O| are re-derived from the mask on the device (the
    // caller's copies are read-only here and equal by construction).
    (void)idx;
    (void)n_out;
    return launch_rows(X, s, h, mask, nullptr, nullptr, nullptr, Xq, c_x, X_O, ldo, stream);
}

hipError_t launch_forward_prologue(const uint16_t* X, int64_t s, int64_t h, float alpha, uint32_t* acc,
                                   uint32_t* mask, int32_t* idx, int32_t* n_out, int8_t* Xq, float* c_x,
                                   uint16_t* X_O, int64_t ldo, hipStream_t stream, int* clear_words) {
    if (s <= kSmallRowsMax && 2 * s * h <= kOneLaunchBytes) {
        // no accumulator: every block finds the mask and the row maxima itself
        *clear_words = 0;
        const dim3 grid(static_cast<unsigned>((h + kSlabCols - 1) / kSlabCols)), block(1024);
        const size_t lds = static_cast<size_t>(h / 32) * sizeof(uint32_t);
        const int si = static_cast<int>(s), hi = static_cast<int>(h);
        const Threshold th = make_threshold(alpha);
#define I8MM_ONE(R)                                                                                          \
    hipLaunchKernelGGL(k_small_prologue<R>, grid, block, lds, stream, X, si, hi, th, mask, idx, n_out, Xq, c_x, \
                       X_O, ldo)
        if (s <= 1)
            I8MM_ONE(1);
        else if (s <= 2)
            I8MM_ONE(2);
        else if (s <= 4)
            I8MM_ONE(4);
        else
            I8MM_ONE(8);
#undef I8MM_ONE
        return hipGetLastError();
    }
    if (s <= kSmallRowsMax) {
        // acc[0 .. s) holds the row maxima.
        *clear_words = static_cast<int>(s);
        const dim3 grid(static_cast<unsigned>((h + kSlabCols - 1) / kSlabCols)), block(256);
        const int si = static_cast<int>(s), hi = static_cast<int>(h);
        const Threshold th = make_threshold(alpha);
#define I8MM_SMALL(RG)                                                                                      \
    hipLaunchKernelGGL(k_small_detect<RG>, grid, block, 0, stream, X, si, hi, th, mask, acc);              \
    hipLaunchKernelGGL(k_small_quant<RG>, grid, block, 0, stream, X, si, hi, mask, acc, idx, n_out, Xq, c_x, \
                       X_O, ldo)
        I8MM_SMALL(1);
#undef I8MM_SMALL
        return hipGetLastError();
    }
    // acc[0 .. h / 32) accumulates the mask.
    *clear_words = static_cast<int>(h / 32);
    hipError_t e = launch_detect_into(X, s, h, alpha, acc, stream);
    if (e != hipSuccess) return e;
    return launch_rows(X, s, h, acc, mask, idx, n_out, Xq, c_x, X_O, ldo, stream);
}

hipError_t launch_forward_prologue_variant(bool zeropoint, const uint16_t* X, int64_t s, int64_t h, float alpha,
                                           uint32_t* acc, uint32_t* mask, int32_t* idx, int32_t* n_out, int8_t* Xq,
                                           float* c_x, int32_t* zp_x, int32_t* rowsum_x, uint16_t* X_O, int64_t ldo,
                                           hipStream_t stream, int* clear_words) {
    // Detection ORs the mask into acc[0 .. h / 32) (zero beforehand, cleared
    // again by the product); the scheme's row quantiser reads it there and
    // its block 0 writes the mask, the index list and |O|.
    *clear_words = static_cast<int>(h / 32);
    hipError_t e = launch_detect_into(X, s, h, alpha, acc, stream);
    if (e != hipSuccess) return e;
    if (zeropoint)
        return launch_quantize_rows_zp(X, s, h, acc, Xq, c_x, zp_x, rowsum_x, X_O, ldo, stream, mask, idx, n_out);
    return launch_quantize_tensorwise(X, s, h, acc, Xq, c_x, X_O, ldo, stream, mask, idx, n_out);
}

hipError_t launch_pack_fp16_panels(const uint16_t* W, int64_t h, int64_t o, uint16_t* Wp, hipStream_t stream) {
    hipLaunchKernelGGL(k_pack_fp16_panels, dim3(static_cast<unsigned>(o / 64), static_cast<unsigned>(h / 32)),
                       dim3(256), 0, stream, W, o, Wp);
    return hipGetLastError();
}

// The column constants of W (SC: Absmax scales, or MaxOnly maxima) via the
// partial maxima kept in the Wq buffer.
template <RowScale SC>
hipError_t launch_col_constants(const uint16_t* W, int64_t h, int64_t o, int8_t* Wq, float* c_w, hipStream_t stream) {
    const int nparts = static_cast<int>((h + kColRows - 1) / kColRows);
    uint16_t* part = reinterpret_cast<uint16_t*>(Wq);
    hipLaunchKernelGGL(k_col_absmax_part, dim3(static_cast<unsigned>((o + 511) / 512), static_cast<unsigned>(nparts)),
                       dim3(256), 0, stream, W, h, o, part);
    hipLaunchKernelGGL(k_col_absmax_reduce<SC>, dim3(static_cast<unsigned>((o + 255) / 256)), dim3(256), 0, stream,
                       part, nparts, o, c_w);
    return hipGetLastError();
}

hipError_t launch_quant_panels(const uint16_t* W, int64_t h, int64_t o, const float* c_w, int8_t* Wq,
                               hipStream_t stream) {
    hipLaunchKernelGGL(k_quant_panels, dim3(static_cast<unsigned>((o + kPanelCols - 1) / kPanelCols),
                                            static_cast<unsigned>(h / 64)),
                       dim3(256), 0, stream, W, o, c_w, Wq);
    return hipGetLastError();
}

hipError_t launch_quantize_cols(const uint16_t* W, int64_t h, int64_t o,
                                int8_t* Wq, float* c_w, hipStream_t stream) {
    hipError_t e = launch_col_constants<RowScale::Absmax>(W, h, o, Wq, c_w, stream);
    if (e != hipSuccess) return e;
    return launch_quant_panels(W, h, o, c_w, Wq, stream);
}

hipError_t launch_quantize_tensorwise(const uint16_t* X, int64_t s, int64_t h, const uint32_t* mask, int8_t* Xq,
                                      float* c_x, uint16_t* X_O, int64_t ldo, hipStream_t stream,
                                      uint32_t* mask_out, int32_t* idx, int32_t* n_out) {
    // row maxima into c_x, one constant over them, then the codes with it
    const size_t dyn = static_cast<size_t>(2 * (h / 32) * 4);
    const int64_t per_lane4 = (h / 8 + 255) / 256;   // chunks per lane with 4 wavefronts per row
    if (s < 2048 && per_lane4 <= 16) {
        // few rows: each row split over 4 wavefronts and held in registers
        const dim3 grid(static_cast<unsigned>(s)), block(256);
#define I8MM_TW(CPL)                                                                                         \
    hipLaunchKernelGGL((k_quant_rows<CPL, RowScale::MaxOnly, 4>), grid, block, dyn, stream, X, s, h, mask,    \
                       mask_out, idx, n_out, Xq, c_x, X_O, ldo);                                              \
    hipLaunchKernelGGL(k_tensor_scale, dim3(1), dim3(1024), 0, stream, c_x, s);                              \
    hipLaunchKernelGGL((k_quant_rows<CPL, RowScale::Given, 4>), grid, block, dyn, stream, X, s, h, mask,      \
                       nullptr, nullptr, nullptr, Xq, c_x, X_O, ldo)
        if (per_lane4 <= 2) { I8MM_TW(2); }
        else if (per_lane4 <= 4) { I8MM_TW(4); }
        else if (per_lane4 <= 8) { I8MM_TW(8); }
        else { I8MM_TW(16); }
#undef I8MM_TW
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>((s + 3) / 4)), block(256);
    hipLaunchKernelGGL((k_quant_rows<0, RowScale::MaxOnly>), grid, block, dyn, stream, X, s, h, mask, mask_out,
                       idx, n_out, Xq, c_x, X_O, ldo);
    hipLaunchKernelGGL(k_tensor_scale, dim3(1), dim3(1024), 0, stream, c_x, s);
    hipLaunchKernelGGL((k_quant_rows<0, RowScale::Given>), grid, block, dyn, stream, X, s, h, mask, nullptr,
                       nullptr, nullptr, Xq, c_x, X_O, ldo);
    return hipGetLastError();
}

hipError_t launch_quantize_weights_tensorwise(const uint16_t* W, int64_t h, int64_t o, int8_t* Wq, float* c_w,
                                              hipStream_t stream) {
    // column maxima, one constant over them in every entry, then the codes
    hipError_t e = launch_col_constants<RowScale::MaxOnly>(W, h, o, Wq, c_w, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_tensor_scale, dim3(1), dim3(1024), 0, stream, c_w, o);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_quant_panels(W, h, o, c_w, Wq, stream);
}

}  // namespace i8mm
