// The decomposed product of LLM.int8() on gfx950 matrix cores:
//   C[s, o] = fp16( C_i32 / (c_x (x) c_w) + X_O W[idx, :] ),  C_i32 = Xq W_i8.
//
// Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for
// Transformers at Scale" (paper-graph-ui digest), "The Full LLM.int8()
// Algorithm", Steps 3-5, and "Mixed-Precision Decomposition" (formal
// definition); [PY] "LLM.int8() 完全拆解" (pinghaoyang.com.cn),
// "第二件武器：混合精度分解".
//
// Operand layouts keep the reduction dimension h contiguous in 16-byte runs:
// Xq is [s, h] row-major, and the weights come in the panel layout
// Wq [h / 64][o][64] (W_i8[k, j] at (k / 64) o 64 + 64 j + k % 64), in which
// the A fragment of a 16x16x64 MFMA (16 columns x 64 reduction bytes) is one
// contiguous KiB and a 256-column tile of one panel is 16 contiguous KiB.
// The matrix core computes D[o][s] (W_i8 as the A operand), so each lane
// ends up holding runs of 4 consecutive output columns of one row of C: the
// decode epilogue stores them as 8-byte fp16 quads, the prefill epilogue
// regroups them through LDS into full 256-byte rows.
//
// Three main loops share the epilogue structure:
//  * k_gemm_prefill (s > 128): 256x256 output tile per 256-thread block, K
//    step 128 (two panels), both operands double buffered in LDS through
//    direct-to-LDS buffer loads, v_mfma_i32_32x32x32_i8, 2x2 waves of
//    128x128.
//  * k_gemm_decode (s <= 16, narrow or evenly filling layers): weight
//    streaming. Four wavefronts per 16*NT
//    output columns (64) split K and read their panels of Wq straight from
//    HBM into the MFMA operand registers with non-temporal loads
//    (v_mfma_i32_16x16x64_i8, rows beyond s read as zero), two register
//    batches in flight.
//  * k_gemm_skinny (s <= 128 otherwise): weight streaming with the columns split
//    between the wavefronts of a block (one block per CU where the columns
//    allow), each over all of K with a ring of weight steps in registers,
//    and X's codes (one to eight row groups of 16) staged once per block
//    in LDS.
// The fused epilogue converts the int32 accumulator to fp32, multiplies by
// 1/c_x_i * 1/c_w_j (S is never materialised), then accumulates the fp16
// outlier product on top with fp16 MFMA (fp32 accumulate), adds the
// optional layer bias and rounds once to fp16.

#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "quant_common.h"

namespace i8mm {
namespace {

// ------------------------------------------------------------------ prefill
constexpr int kTO = 256;   // output columns (o) per block
constexpr int kTS = 256;   // output rows (s) per block
constexpr int kTK = 128;   // reduction bytes per LDS stage
constexpr int kBuf = 256 * kTK / 16;   // v4i slots of one operand's stage buffer (32 KiB)

// LDS layout of a stage buffer: 256 rows of 128 bytes; row r keeps its
// 16-byte chunk c in slot 8 r + (c ^ ((r / 2) & 7)). The LDS serves a
// 16-byte read 16 lanes at a time from 64 banks (16 groups of 16 bytes, two
// consecutive rows per bank row), so the 16 consecutive rows read at one
// chunk hit 16 different groups. (With c ^ (r & 7), rows r and r + 8 met in
// one group and every fragment read took twice as long: measured 1.6x less
// read throughput for this access pattern.)

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero and stores there are dropped, which handles ragged tiles
// without branches. Word 3 selects the
// 32-bit data format that raw loads on gfx9-family parts expect.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ v4i buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Same, marked non-temporal (streamed data that no other block re-reads).
__device__ __forceinline__ v4i buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}

// Bytes from byte `from` to the end of an array of `total` bytes (0 past it).
__device__ __forceinline__ uint32_t bytes_left(int64_t total, int64_t from) {
    return static_cast<uint32_t>(from < total ? total - from : 0);
}

constexpr uint32_t kOutOfRange = 0x80000000u;   // a per-lane offset past every buffer under 2 GiB

// The fp16 W rows span 2 h o bytes, which can pass 2^31 (h o < 2^31 only).
// With h and o multiples of 64, 2 h o <= 2^32 - 8192, so this offset (with
// no scalar or instruction offset added) is past the end of every W.
constexpr uint32_t kOutOfRangeW = 0xfffff000u;

// Block -> output tile. Blocks are dealt to the 8 XCDs round robin (block b
// runs on XCD b % 8), and each XCD is given one contiguous run of a grouped
// tile order: column groups of `group` weight tiles that span every row
// tile, row by row inside a group. The ~32 tiles an XCD runs at once then
// cover about 32 / group row tiles x group weight tiles, i.e. ~12 operand
// panels streamed through its 4 MiB L2 per round (an order with rows
// fastest made each round re-fetch every row panel of Xq). Over the whole
// product the weights are fetched (row tiles / (32 / group)) times and Xq
// (weight tiles / group) times, so the launch takes group 4 when the int8
// weights exceed the 256 MiB Infinity Cache (fewer passes over them) and 8
// otherwise.
// Block and tile indices are 32-bit (as the grid is), which keeps the index
// arithmetic short ahead of the first loads.
__device__ __forceinline__ void grouped_tile(uint32_t b, uint32_t nb, uint32_t n_ts, uint32_t n_to, uint32_t group,
                                             uint32_t& ts, uint32_t& to) {
    const uint32_t q = nb / 8, r = nb % 8, x = b % 8, i = b / 8;
    const uint32_t t = (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;   // place in the grouped order
    const uint32_t per = group * n_ts;
    const uint32_t g = t / per, j = t % per;
    const uint32_t c0 = g * group;
    const uint32_t w = n_to - c0 < group ? n_to - c0 : group;
    ts = j / w;
    to = c0 + j % w;
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// One 16-deep slice (outlier columns 16 kb .. 16 kb + 15) of the fp16
// outlier product's operands for a 256 x 256 tile, staged in LDS by
// direct-to-LDS buffer loads (lane i of a load writes 16 bytes at
// base + 16 i): the first kSlice halves hold W[idx[k], o0 .. o0 + 255] as
// [16][256], the next kSlice hold X_O[s0 .. s0 + 255, k] as [256][16].
// Entries past |O|, past o or past s are written as zeros by the range
// check. Every wavefront issues two 1 KiB loads of each operand.
constexpr int kSlice = 256 * 16;

__device__ __forceinline__ void stage_outlier_slice(int kb, int n, int wid, int lane, int64_t o0, int64_t s0,
                                                    int64_t s, int64_t o, int64_t ldo,
                                                    const int32_t* __restrict__ idx,
                                                    __amdgpu_buffer_rsrc_t rW, __amdgpu_buffer_rsrc_t rX,
                                                    uint16_t* dst, bool with_w = true) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int j = wid + 4 * q;                 // wave-uniform, 0..7
        if (with_w) {
            const int k0 = kb * 16 + 2 * j;        // rows k0 (lanes 0-31) and k0 + 1 (lanes 32-63)
            const int id0 = idx[k0], id1 = idx[k0 + 1];
            const int k = k0 + (lane >> 5);
            const int64_t col = o0 + (lane & 31) * 8;
            const bool okW = k < n && col < o;
            const uint32_t vW = okW ? static_cast<uint32_t>(((lane >> 5) ? id1 : id0) * o * 2 + (lane & 31) * 16)
                                    : kOutOfRangeW;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rW, LDS_PTR(dst + j * 512), 16, vW, 0, 0, 0);
        }
        const int r = 32 * j + (lane >> 1);
        const uint32_t vX = s0 + r < s ? static_cast<uint32_t>(r * ldo * 2 + (kb * 16 + (lane & 1) * 8) * 2)
                                       : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rX, LDS_PTR(dst + kSlice + j * 512), 16, vX, 0, 0, 0);
    }
}

// An outlier row's weight W[k, j] when no fp16 copy of W is resident: the
// int8 code of the panel layout dequantised by multiplying back with the
// column's inverse scale, fl16(fl32(q * inv_cw)), inv_cw = fl32(1 / c_w[j])
// (correctly rounded: see inverse_scale). Exact whenever the quantisation of
// the column was (power-of-two c_w, codes reproducing W).
__device__ __forceinline__ float inverse_scale(float c) { return __fdiv_rn(1.0f, c); }

__device__ __forceinline__ uint16_t dequantized_weight(const int8_t* __restrict__ Wq, float inv_cw, int64_t k,
                                                       int64_t j, int64_t o) {
    const int q = Wq[(k >> 6) * o * 64 + j * 64 + (k & 63)];
    return float_to_half_bits(static_cast<float>(q) * inv_cw);
}

// The W part of slice kb rebuilt from the int8 codes, written directly in
// the transposed layout of transpose_w_slice (column t of the tile holds
// its 16 rows idx[16 kb .. 16 kb + 15] as two 16-byte halves). Thread t
// owns column o0 + t; rows past |O| and columns past o are zero.
__device__ __forceinline__ void stage_w8_slice(int kb, int n, int64_t o0, int64_t o,
                                               const int32_t* __restrict__ idx, const int8_t* __restrict__ Wq,
                                               const float* __restrict__ c_w, uint16_t* dst) {
    const int t = threadIdx.x;
    const int64_t j = o0 + t;
    const bool col_ok = j < o;
    const float inv_cw = inverse_scale(col_ok ? c_w[j] : 1.0f);
    const int sw = (t >> 3) & 1;
    // A rolled loop with 2-byte LDS writes keeps this small: it is inlined
    // into every output block of the epilogue's rounds path.
#pragma unroll 1
    for (int e = 0; e < 16; ++e) {
        const int k = kb * 16 + e;
        const uint16_t w = col_ok && k < n ? dequantized_weight(Wq, inv_cw, idx[k], j, o) : static_cast<uint16_t>(0);
        dst[(t * 2 + ((e >> 3) ^ sw)) * 8 + (e & 7)] = w;
    }
}

// f + wa xb with v_mfma_f32_32x32x16_f16 in its VGPR form. The epilogue's
// dequantised values live in VGPRs while the accumulators of the main loop
// fill the AGPRs; left to the compiler, this MFMA takes its C operand and
// result in AGPRs and every block's values make a round trip (and the
// register shuffles cost ~5 % of the kernel). Written as asm, the wait
// states the hardware needs around a VGPR-form MFMA are explicit: 2 after
// VALU writes of its operands, and more than the 18 a 16-pass result needs
// before anything reads (or overwrites) its registers.
// The accumulator is one tied operand: a result that only partly overlaps
// the C operand is not a valid encoding.
__device__ __forceinline__ v16f mfma_f16_vgpr(const v8h& wa, const v8h& xb, v16f f) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(f)
                 : "v"(wa), "v"(xb));
    return f;
}

// In-place transpose of the W part of a staged slice, [16 k][256 columns]
// -> [256 columns][16 k] as two 16-byte halves per column (k 0-7, 8-15)
// whose order flips with bit 3 of the column, so that 16 consecutive
// columns read at one k half hit 16 different bank groups. Thread t owns
// column t; two block barriers.
__device__ __forceinline__ void transpose_w_slice(uint16_t* sl) {
    const int t = threadIdx.x;
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = static_cast<uint32_t>(sl[(2 * j) * 256 + t]) | (static_cast<uint32_t>(sl[(2 * j + 1) * 256 + t]) << 16);
    __syncthreads();
    const int sw = (t >> 3) & 1;
    uint4* dst = reinterpret_cast<uint4*>(sl);
    dst[t * 2 + sw] = make_uint4(v[0], v[1], v[2], v[3]);
    dst[t * 2 + (sw ^ 1)] = make_uint4(v[4], v[5], v[6], v[7]);
    __syncthreads();
}

// The two operands of a staged, transposed slice: the W part of the
// lane's column in column block ob, and the X_O part of its row in row
// block sb.
__device__ __forceinline__ v8h slice_w_operand(const uint16_t* sl, int wo, int ob, int r32, int khalf) {
    const int col = wo * 128 + ob * 32 + r32;
    return *reinterpret_cast<const v8h*>(sl + (col * 2 + (khalf ^ ((col >> 3) & 1))) * 8);
}

__device__ __forceinline__ v8h slice_x_operand(const uint16_t* sl, int ws, int sb, int r32, int khalf) {
    return *reinterpret_cast<const v8h*>(sl + kSlice + (ws * 128 + sb * 32 + r32) * 16 + 8 * khalf);
}

// f[ob] += wa[ob] xb for the four column blocks of one 32-row block: four
// independent VGPR-form MFMAs back to back under one set of wait states
// (2 before, for the VALU writes of f; more than the 18 a 16-pass result
// needs after, before anything reads f).
__device__ __forceinline__ void mfma4_f16_vgpr(const v8h (&wa)[4], const v8h& xb, v16f (&f)[4]) {
    asm volatile("s_nop 1\n\t"
                 "v_mfma_f32_32x32x16_f16 %0, %4, %8, %0\n\t"
                 "v_mfma_f32_32x32x16_f16 %1, %5, %8, %1\n\t"
                 "v_mfma_f32_32x32x16_f16 %2, %6, %8, %2\n\t"
                 "v_mfma_f32_32x32x16_f16 %3, %7, %8, %3\n\t"
                 "s_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3])
                 : "v"(wa[0]), "v"(wa[1]), "v"(wa[2]), "v"(wa[3]), "v"(xb));
}

// The same for slice q with both operands read from global memory: the
// slices past the ones staged in LDS (more than 96 outlier columns, far
// beyond the handful the method meets), without staging or barriers.
__device__ __forceinline__ v16f apply_outlier_slice_global(int q, int n, int64_t o0, int64_t s0, int64_t s, int64_t o,
                                                           const uint16_t* __restrict__ X_O, int64_t ldo,
                                                           const int32_t* __restrict__ idx,
                                                           const uint16_t* __restrict__ W, const int8_t* __restrict__ Wq,
                                                           const float* __restrict__ c_w, int wo, int ws, int sb, int ob,
                                                           int r32, int khalf, v16f f) {
    const int64_t col = o0 + wo * 128 + ob * 32 + r32;
    const int64_t row = s0 + ws * 128 + sb * 32 + r32;
    const int k0 = q * 16 + 8 * khalf;
    const bool col_ok = col < o;
    const float inv_cw = inverse_scale(W == nullptr && col_ok ? c_w[col] : 1.0f);
    v8h wa;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int k = k0 + e;
        const bool ok = col_ok && k < n;
        const int64_t rk = ok ? idx[k] : 0;
        uint16_t bits = 0;
        if (ok) bits = W != nullptr ? W[rk * o + col] : dequantized_weight(Wq, inv_cw, rk, col, o);
        wa[e] = __builtin_bit_cast(_Float16, bits);
    }
    // columns of X_O up to round_up(|O|, 32) hold the outliers and zeros
    v8h xb = {};
    if (row < s) xb = *reinterpret_cast<const v8h*>(X_O + row * ldo + k0);
    return mfma_f16_vgpr(wa, xb, f);
}

// LDS staging of the fp16 output: each wavefront owns 32 rows x 128
// columns, rows padded to 136 halves (272 bytes) against bank conflicts.
constexpr int kOutRow = 136;
constexpr int kOutWave = 32 * kOutRow;          // halves per wavefront
constexpr int kMaxOnceSlices = 5;               // extra slices staged at once

// Writes a wavefront's staged 32 x 128 fp16 block (rows srow0 .. + 31 and
// columns ocol0 .. + 127 of C) as full 256-byte rows: 16 lanes per row, 4
// rows per store, with no branch: the stores take 32-bit
// offsets from a buffer resource that starts at row srow0 and ends with row
// s - 1, so rows past s fall outside it and columns past o get an
// out-of-range offset (offsets stay below 64 o < 2^31 as h o < 2^31).
__device__ __forceinline__ void store_staged_block(const uint16_t* out_st, uint16_t* C, int64_t srow0, int64_t ocol0,
                                                   int64_t s, int64_t o, int lane) {
    const int64_t rows = s - srow0;
    const uint32_t bytes = rows <= 0 ? 0u : static_cast<uint32_t>((rows < 32 ? rows : 32) * o * 2);
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(C + (rows > 0 ? srow0 * o : 0), bytes);
    const uint32_t o32 = static_cast<uint32_t>(o);
    const uint32_t col = static_cast<uint32_t>(ocol0) + (lane & 15) * 8;
    const bool col_ok = col < o32;
    const uint32_t off0 = ((lane >> 4) * o32 + col) * 2;
    // all eight LDS reads first, so that their latencies overlap
    v4i v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = *reinterpret_cast<const v4i*>(out_st + (4 * i + (lane >> 4)) * kOutRow + (lane & 15) * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t off = col_ok ? off0 + static_cast<uint32_t>(i) * 8 * o32 : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v[i]), rC, off, 0, 0);
    }
}

// Prefill main loop (also the dense fp16 product, MODE Fp16Dense: the same
// byte geometry with 2-byte elements, see launch_fp16_gemm): both operand
// tiles reach LDS through direct-to-LDS
// buffer loads, double buffered in four separate arrays (A0/A1 weights,
// B0/B1 activations) so that the compiler's wait tracking for these loads
// can tell the buffer being filled from the one being read. A stage's
// 16 loads per wavefront go out in three parts spread over three
// sub-steps, interleaved with the MFMAs, so that the loads never queue up
// in front of the matrix-core instructions; the fourth sub-step before the
// barrier covers their latency. The eight weight loads go first, all in
// the sub-step right after the barrier that frees their buffer, and the
// eight activation loads in the two sub-steps after it: the weight panels
// come from HBM or the Infinity Cache (each is read by few tiles at a
// time), while the codes of X, shared by every weight tile, mostly hit L2.
// Interleaved A/B on three GPUs against A and B loads alternating: -3.1 to
// -3.8 % product time on 4096 x 12288 x 36864, -1.4 to -2.0 % on
// 4096 x 8192 x 28672, within 0.3 % on 2048 x 4096 x 16384.
//
// QX (MODE Mixed only): the int8 operand of X is made inside this kernel
// from the fp16 rows Xh instead of being read from Xq, which is then never
// written ([DIGEST] Step 2 folded into the product's operand staging). A
// stage's B slots are filled through registers: the fp16 values of the
// slot's 16 columns, those in O (xmask) cleared, scaled by the row's c_x
// and rounded exactly as the row quantiser does, so the codes, and C, are
// bit-identical to the two-pass forward's.
template <GemmOut MODE, bool QX = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_prefill(const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq,
                    int64_t s, int64_t h /* reduction bytes per row */, int64_t o,
                    const float* __restrict__ c_x, const float* __restrict__ c_w,
                    const uint16_t* __restrict__ X_O, int64_t ldo,
                    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out,
                    const uint16_t* __restrict__ W, const uint16_t* __restrict__ bias, void* __restrict__ Cout,
                    uint32_t* __restrict__ clear, int clear_words, ZpArgs zp, uint32_t group,
                    const uint16_t* __restrict__ Xh, const uint32_t* __restrict__ xmask) {
    static_assert(!QX || MODE == GemmOut::Mixed, "X is quantised in the product only for the LLM.int8() output");
    __shared__ v4i A0[kBuf], A1[kBuf], B0[kBuf], B1[kBuf];
    __shared__ __attribute__((aligned(16))) uint16_t olds[2 * kSlice];
    __shared__ __attribute__((aligned(16))) float scl[512];   // c_x of the tile's rows, then c_w of its columns
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < clear_words; i += 256) clear[i] = 0u;

    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(wid);
    const int wo = wid & 1, ws = wid >> 1;
    const int r32 = lane & 31, khalf = lane >> 5;
    // 32-bit division (a 64-bit one is a long scalar sequence that would
    // delay the first loads): tile < gridDim.x and n_ts < 2^32
    const uint32_t n_ts = static_cast<uint32_t>((s + kTS - 1) / kTS);
    const uint32_t n_to = static_cast<uint32_t>((o + kTO - 1) / kTO);
    uint32_t ts_u, to_u;
    grouped_tile(blockIdx.x, gridDim.x, n_ts, n_to, group, ts_u, to_u);
    const int64_t ts_i = ts_u, to_i = to_u;
    const int64_t o0 = to_i * kTO, s0 = ts_i * kTS;
    const int64_t o_rows = o - o0 < kTO ? o - o0 : kTO;
    const int64_t s_rows = s - s0 < kTS ? s - s0 : kTS;

    // Buffer resources. B: rows past s read as zero. A: one resource per
    // stage, based at the tile's first column in the stage's first panel,
    // ending with the array, so that a missing second panel (h % 128 == 64)
    // and every stage past the last one lie outside it.
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Xq + s0 * h, static_cast<uint32_t>(s_rows * h));
    const int64_t wq_bytes = h * o;

    // Load q (0..7) of wavefront w fills LDS rows 64 w + 8 q .. + 7 (one
    // KiB; lane i writes slot 8 r + i % 8 of row r = 64 w + 8 q + i / 8),
    // so lane i fetches chunk c = (i % 8) ^ ((r / 2) & 7) of its row, i.e.
    // c0 = (i % 8) ^ (i / 16) for even q and c0 ^ 4 for odd q: panel
    // 2 kt + c / 4, bytes 16 (c % 4) of the row's 64 there. Rows past o
    // (whole wavefronts, as o_rows is a multiple of 64) and chunks past h
    // get the out-of-range offset.
    const int dr = lane >> 3;
    const int c0 = (lane & 7) ^ (dr >> 1);
    auto a_offset = [&](int c) {
        return 64 * wu < o_rows ? static_cast<uint32_t>((64 * wu + dr) * 64 + (c & 3) * 16 + (c >> 2) * o * 64)
                                : kOutOfRange;
    };
    const uint32_t vA[2] = {a_offset(c0), a_offset(c0 ^ 4)};
    uint32_t vB[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        vB[q] = static_cast<uint32_t>((64 * wu + 8 * q + dr) * h + (c0 ^ (4 * (q & 1))) * 16);
    const int64_t KT = (h + kTK - 1) / kTK;
    // Loads q in [q0, q1) of stage kt into (A, B).
    auto load_part = [&](int64_t kt, v4i* A, v4i* B, int q0, int q1) {
        const uint32_t k = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kt * kTK));
        const int64_t a0 = o0 * 64 + kt * kTK * o;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(Wq + (a0 < wq_bytes ? a0 : 0), bytes_left(wq_bytes, a0));
        const uint32_t oob[2] = {(k + c0 * 16 < static_cast<uint32_t>(h)) ? 0u : kOutOfRange,
                                 (k + (c0 ^ 4) * 16 < static_cast<uint32_t>(h)) ? 0u : kOutOfRange};
#pragma unroll
        for (int q = q0; q < q1; ++q) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDS_PTR(A + (wu * 8 + q) * 64), 16,
                                                     (vA[q & 1] | oob[q & 1]) + q * 512, 0, 0, 0);
            if constexpr (!QX)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, LDS_PTR(B + (wu * 8 + q) * 64), 16, vB[q] | oob[q & 1],
                                                         k, 0, 0);
        }
    };
    // The weight loads q in [q0, q1) of stage kt into A, and the
    // activation loads into B (the two halves of load_part).
    auto load_a = [&](int64_t kt, v4i* A, int q0, int q1) {
        const uint32_t k = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kt * kTK));
        const int64_t a0 = o0 * 64 + kt * kTK * o;
        const __amdgpu_buffer_rsrc_t rA = make_rsrc(Wq + (a0 < wq_bytes ? a0 : 0), bytes_left(wq_bytes, a0));
        const uint32_t oob[2] = {(k + c0 * 16 < static_cast<uint32_t>(h)) ? 0u : kOutOfRange,
                                 (k + (c0 ^ 4) * 16 < static_cast<uint32_t>(h)) ? 0u : kOutOfRange};
#pragma unroll
        for (int q = q0; q < q1; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, LDS_PTR(A + (wu * 8 + q) * 64), 16,
                                                     (vA[q & 1] | oob[q & 1]) + q * 512, 0, 0, 0);
    };
    auto load_b = [&](int64_t kt, v4i* B, int q0, int q1) {
        const uint32_t k = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kt * kTK));
        const uint32_t oob[2] = {(k + c0 * 16 < static_cast<uint32_t>(h)) ? 0u : kOutOfRange,
                                 (k + (c0 ^ 4) * 16 < static_cast<uint32_t>(h)) ? 0u : kOutOfRange};
#pragma unroll
        for (int q = q0; q < q1; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, LDS_PTR(B + (wu * 8 + q) * 64), 16, vB[q] | oob[q & 1],
                                                     k, 0, 0);
    };

    // QX operand path. Lane (w, q) makes the slot that load q of wavefront
    // w fills above: row 64 w + 8 q + dr, chunk c = c0 (even q) or c0 ^ 4
    // (odd q), i.e. reduction columns k + 16 c .. + 15, read as two 16-byte
    // fp16 chunks. Rows past s and columns past h read zero (code 0); mask
    // words past h read zero.
    const __amdgpu_buffer_rsrc_t rXh = make_rsrc(QX ? Xh + s0 * h : nullptr,
                                                 QX ? static_cast<uint32_t>(s_rows * h * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rMask = make_rsrc(QX ? xmask : nullptr, QX ? static_cast<uint32_t>(h / 8) : 0u);
    // per-lane byte offset of load q's slot: row 64 w + 8 q + dr, chunk c0
    // (even q) or c0 ^ 4 (odd q). Everything that can leave the buffer (the
    // row, the chunk) stays in the per-lane offset, which the range check
    // covers; only the stage's column offset, always inside a row whose
    // chunk is in range, goes in the scalar offset.
    uint32_t vXh[8];
    float xsc[8];
    if constexpr (QX) {
        const __amdgpu_buffer_rsrc_t rcs = make_rsrc(c_x + s0, static_cast<uint32_t>(s_rows * 4));
#pragma unroll
        for (int q = 0; q < 8; ++q)
            vXh[q] = static_cast<uint32_t>(((64 * wu + 8 * q + dr) * h + (c0 ^ (4 * (q & 1))) * 16) * 2);
#pragma unroll
        for (int q = 0; q < 8; ++q)
            xsc[q] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rcs, static_cast<uint32_t>(4 * (64 * wu + 8 * q + dr)), 0, 0));
    }
    uint4 xv[8][2];
    v4u xmw;
    // Loads / stores q in [Q0, Q1) (std::integral_constant bounds, so that
    // the loops unroll and the arrays stay in registers).
    auto x_load = [&](int64_t kt, auto Q0, auto Q1) __attribute__((always_inline)) {
        constexpr int q0 = decltype(Q0)::value, q1 = decltype(Q1)::value;
        const uint32_t k = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kt * kTK));
        const uint32_t oob[2] = {(k + c0 * 16 < static_cast<uint32_t>(h)) ? 0u : kOutOfRange,
                                 (k + (c0 ^ 4) * 16 < static_cast<uint32_t>(h)) ? 0u : kOutOfRange};
        if constexpr (q0 == 0) {
            // word by word: with h % 128 == 64 the last stage's words 2 and
            // 3 lie past the mask and read zero on their own
#pragma unroll
            for (int j = 0; j < 4; ++j) xmw[j] = __builtin_amdgcn_raw_buffer_load_b32(rMask, k / 8 + 4 * j, 0, 0);
        }
#pragma unroll
        for (int q = q0; q < q1; ++q) {
            const uint32_t off = vXh[q] | oob[q & 1];
            xv[q][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rXh, off, 2 * k, 0));
            xv[q][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rXh, off + 16, 2 * k, 0));
        }
    };
    auto x_store = [&](v4i* B, auto Q0, auto Q1) __attribute__((always_inline)) {
        constexpr int q0 = decltype(Q0)::value, q1 = decltype(Q1)::value;
        // O's columns among the stage's 128: bit j of word j / 32 (rarely any)
        const bool any = __builtin_amdgcn_readfirstlane(static_cast<int>(xmw[0] | xmw[1] | xmw[2] | xmw[3])) != 0;
        auto bits_of = [&](int c) {
            const uint32_t w = (c >> 1) == 0 ? xmw[0] : (c >> 1) == 1 ? xmw[1] : (c >> 1) == 2 ? xmw[2] : xmw[3];
            return (w >> (16 * (c & 1))) & 0xffffu;
        };
#pragma unroll
        for (int q = q0; q < q1; ++q) {
            uint4 v0 = xv[q][0], v1 = xv[q][1];
            if (any) {
                const uint32_t b = bits_of(c0 ^ (4 * (q & 1)));
                v0 = chunk_clear(v0, b & 0xffu);
                v1 = chunk_clear(v1, b >> 8);
            }
            const uint2 lo = chunk_quantize(v0, xsc[q]), hi = chunk_quantize(v1, xsc[q]);
            B[(wu * 8 + q) * 64 + lane] = __builtin_bit_cast(v4i, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
    };

    int n_o = 0;
    constexpr bool zpm = MODE == GemmOut::ZeroPoint;
    constexpr bool mixed = MODE == GemmOut::Mixed || zpm;   // fused fp16 epilogue with outliers
    const __amdgpu_buffer_rsrc_t rW = make_rsrc(mixed && W ? W + o0 : nullptr,
                                                mixed && W ? static_cast<uint32_t>((h * o - o0) * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rX = make_rsrc(mixed ? X_O + s0 * ldo : nullptr,
                                                mixed ? static_cast<uint32_t>(s_rows * ldo * 2) : 0u);
    // Without a resident fp16 W (W null) the outlier rows are rebuilt from
    // the int8 codes in the epilogue; only their X part is staged here.
    const bool w8 = W == nullptr;
    if constexpr (mixed) n_o = __builtin_amdgcn_readfirstlane(n_out[0]);

    constexpr bool dense16 = MODE == GemmOut::Fp16Dense;
    using Acc = std::conditional_t<dense16, v16f, v16i>;
    Acc acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    // Fragment slots: the four rows a lane reads share (r / 2) & 7
    // (= (r32 / 2) & 7), so slot(row_i, chunk) = slot(row_0, chunk) + 256 i.
    int offA[4], offB[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int x = (kk * 2 + khalf) ^ ((r32 >> 1) & 7);
        offA[kk] = (wo * 128 + r32) * 8 + x;
        offB[kk] = (ws * 128 + r32) * 8 + x;
    }
    v4i fa[2][4], fb[2][4];
    auto frags = [&](const v4i* A, const v4i* B, int kk, v4i* a, v4i* b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = A[offA[kk] + 256 * i];
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = B[offB[kk] + 256 * i];
    };
    // A sub-step is 32 reduction bytes per row: 32 int8 codes for
    // v_mfma_i32_32x32x32_i8, or 16 fp16 values for v_mfma_f32_32x32x16_f16,
    // whose lane fragments sit in the same 16-byte slots.
    auto mma = [&](const v4i* a, const v4i* b) {
#pragma unroll
        for (int ob = 0; ob < 4; ++ob)
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                if constexpr (dense16)
                    acc[ob][sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a[ob]),
                                                                         __builtin_bit_cast(v8h, b[sb]), acc[ob][sb], 0, 0, 0);
                else
                    acc[ob][sb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ob], b[sb], acc[ob][sb], 0, 0, 0);
            }
    };
    // One sub-step's order: MFMAs interleaved with the next sub-step's LDS
    // reads and with this part's loads.
    // At most one load every second MFMA (measured ~1 % faster than one
    // per MFMA, and faster than one every third, which pushes the last
    // loads of a stage too close to its wait).
    auto sched_sub = [&]() {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // MFMA
            if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
            if (i & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // VMEM read
        }
    };
    // The sub-step after the barrier, which carries the eight weight loads:
    // each one a MFMA earlier (after MFMAs 0, 2, .., 14), the first right
    // behind the first MFMA. Interleaved A/B on two GPUs: -0.6 to -0.8 %
    // product time on all three prefill layers; the same shift in every
    // sub-step was slower on 4096 x 12288 x 36864.
    auto sched_sub_first = [&]() {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // MFMA
            if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
            if (!(i & 1)) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        }
    };
    // Stage kt from (Ac, Bc); stage kt + 1 sits in (An, Bn), of which the
    // activation loads are still to go out (its weight loads left with the
    // previous stage's last sub-step). Software pipeline across the
    // barrier: the fragments of sub-step 3 are read before it and
    // multiplied after it, and right after it (Ac, Bc) are free and Ac
    // receives the weight loads of stage kt + 2. Loads of stages past the
    // last one fall outside their resources and land as zeros in the idle
    // buffers, so the loop carries no branch around them.
    auto stage = [&](int64_t kt, v4i* Ac, v4i* Bc, v4i* An, v4i* Bn) {
        frags(Ac, Bc, 1, fa[1], fb[1]);
        load_b(kt + 1, Bn, 0, 4);
        mma(fa[0], fb[0]);
        sched_sub();
        frags(Ac, Bc, 2, fa[0], fb[0]);
        load_b(kt + 1, Bn, 4, 8);
        mma(fa[1], fb[1]);
        sched_sub();
        frags(Ac, Bc, 3, fa[1], fb[1]);
        mma(fa[0], fb[0]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        // The barrier's fence does not cover direct-to-LDS loads: each
        // wavefront first waits for its own loads of stage kt + 1.
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        __syncthreads();
        frags(An, Bn, 0, fa[0], fb[0]);
        load_a(kt + 2, Ac, 0, 8);
        mma(fa[1], fb[1]);
        sched_sub_first();
    };
    // QX: the same stage, with the fp16 rows of stage kt + 1 loaded in
    // sub-steps 0 and 1 and quantised into Bn in sub-steps 2 and 3 (Bn was
    // last read before the previous barrier).
    auto sched_qx = [&]() {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // MFMA
            if (i < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // DS read
            __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);              // VALU
            if (i & 3) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);     // DS write
        }
    };
    auto stage_qx = [&](int64_t kt, v4i* Ac, v4i* Bc, v4i* An, v4i* Bn) __attribute__((always_inline)) {
        frags(Ac, Bc, 1, fa[1], fb[1]);
        load_part(kt + 1, An, Bn, 3, 6);
        x_load(kt + 1, std::integral_constant<int, 0>{}, std::integral_constant<int, 4>{});
        mma(fa[0], fb[0]);
        sched_sub();
        frags(Ac, Bc, 2, fa[0], fb[0]);
        load_part(kt + 1, An, Bn, 6, 8);
        x_load(kt + 1, std::integral_constant<int, 4>{}, std::integral_constant<int, 8>{});
        mma(fa[1], fb[1]);
        sched_sub();
        frags(Ac, Bc, 3, fa[1], fb[1]);
        x_store(Bn, std::integral_constant<int, 0>{}, std::integral_constant<int, 4>{});
        mma(fa[0], fb[0]);
        sched_qx();
        x_store(Bn, std::integral_constant<int, 4>{}, std::integral_constant<int, 8>{});
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        __syncthreads();
        frags(An, Bn, 0, fa[0], fb[0]);
        load_part(kt + 2, Ac, Bc, 0, 3);
        mma(fa[1], fb[1]);
        sched_sub();
    };

    load_part(0, A0, B0, 0, 8);
    if constexpr (QX)
        load_part(1, A1, B1, 0, 3);
    else
        load_a(1, A1, 0, 8);
    if constexpr (QX) {
        x_load(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 8>{});
        x_store(B0, std::integral_constant<int, 0>{}, std::integral_constant<int, 8>{});
    }
    // Behind the first operand loads: the first slice of the outlier
    // operands to its own LDS region, and the row and column scales of the
    // tile to LDS (direct-to-LDS, one dword per lane; entries past s or o
    // read zero and are never used). Nothing of this is held in registers
    // across the main loop.
    if constexpr (mixed) {
        if (n_o > 0) stage_outlier_slice(0, n_o, wu, lane, o0, s0, s, o, ldo, idx, rW, rX, olds, !w8);
        const __amdgpu_buffer_rsrc_t rcx = make_rsrc(c_x + s0, static_cast<uint32_t>(s_rows * 4));
        const __amdgpu_buffer_rsrc_t rcw = make_rsrc(c_w + o0, static_cast<uint32_t>(o_rows * 4));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rcx, LDS_PTR(scl + 64 * wu), 4, static_cast<uint32_t>(4 * (64 * wu + lane)),
                                                 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rcw, LDS_PTR(scl + 256 + 64 * wu), 4,
                                                 static_cast<uint32_t>(4 * (64 * wu + lane)), 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    __syncthreads();
    frags(A0, B0, 0, fa[0], fb[0]);
    int64_t kt = 0;
    if constexpr (QX) {
        for (; kt + 2 <= KT; kt += 2) {
            stage_qx(kt, A0, B0, A1, B1);
            stage_qx(kt + 1, A1, B1, A0, B0);
        }
        if (kt < KT) stage_qx(kt, A0, B0, A1, B1);
    } else {
        for (; kt + 2 <= KT; kt += 2) {
            stage(kt, A0, B0, A1, B1);
            stage(kt + 1, A1, B1, A0, B0);
        }
        if (kt < KT) stage(kt, A0, B0, A1, B1);   // an odd number of stages
    }

    // Lane layout of a 32x32 accumulator: register r holds
    // D[o = 8 (r / 4) + 4 (lane / 32) + r % 4][s = lane % 32].
    if constexpr (dense16) {
        // fp32 accumulators rounded once to fp16, staged per 32-row block and
        // written as full 256-byte rows.
        uint16_t* C = static_cast<uint16_t*>(Cout);
        // The last stage's loads of the stage after it (all out of range)
        // still write zeros into a stage buffer, and the barrier's fence
        // does not wait for direct-to-LDS loads: wait for them before any
        // wavefront reuses the buffers.
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        __syncthreads();   // every wavefront is done with the stage buffers
        uint16_t* out_st = wid < 3 ? reinterpret_cast<uint16_t*>(A1) + wid * kOutWave : reinterpret_cast<uint16_t*>(B1);
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
#pragma unroll
            for (int ob = 0; ob < 4; ++ob) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const v16f& f = acc[ob][sb];
                    const uint32_t lo = pack_half2(f[4 * g], f[4 * g + 1]);
                    const uint32_t hi = pack_half2(f[4 * g + 2], f[4 * g + 3]);
                    *reinterpret_cast<uint2*>(out_st + r32 * kOutRow + ob * 32 + 8 * g + 4 * khalf) =
                        make_uint2(lo, hi);
                }
            }
            // row and column origin through scalar registers (uniform descriptor)
            store_staged_block(out_st, C, s0 + __builtin_amdgcn_readfirstlane(ws) * 128 + sb * 32,
                               o0 + __builtin_amdgcn_readfirstlane(wo) * 128, s, o, lane);
        }
    } else if constexpr (MODE == GemmOut::Int32) {
        int32_t* C = static_cast<int32_t*>(Cout);
#pragma unroll
        for (int ob = 0; ob < 4; ++ob)
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const int64_t srow = s0 + ws * 128 + sb * 32 + r32;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t ocol = o0 + wo * 128 + ob * 32 + 8 * g + 4 * khalf;
                    if (srow < s && ocol < o) {
                        v4i v = {acc[ob][sb][4 * g], acc[ob][sb][4 * g + 1], acc[ob][sb][4 * g + 2],
                                 acc[ob][sb][4 * g + 3]};
                        *reinterpret_cast<v4i*>(C + srow * o + ocol) = v;
                    }
                }
            }
    } else {
        uint16_t* C = static_cast<uint16_t*>(Cout);
        // As above: the last stage's out-of-range loads must have landed
        // before the stage buffers take slices, staging, bias and scales.
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
        __syncthreads();   // every wavefront is done with the stage buffers
        // Epilogue LDS: extra outlier slices q = 1, 2 in A0, 3, 4 in B0 and
        // 5 in B1; output staging of waves 0-2 in A1, followed there by the
        // bias and the zeropoint vectors, and of wave 3 in B1; the scales in
        // their own array.
        auto slice_at = [&](int q) -> uint16_t* {   // q = 1 .. kMaxOnceSlices
            uint16_t* base = q <= 2 ? reinterpret_cast<uint16_t*>(A0)
                           : q <= 4 ? reinterpret_cast<uint16_t*>(B0)
                                    : reinterpret_cast<uint16_t*>(B1) + kOutWave + 1024;
            return base + (q <= 4 ? ((q - 1) & 1) * 2 * kSlice : 0);
        };
        // after the staging of waves 0-2 in A1: bias, then (zeropoint) zp_w
        // and the column code sums over the non-outlier rows, 128 per wave
        float* a1_tail = reinterpret_cast<float*>(reinterpret_cast<uint16_t*>(A1) + 3 * kOutWave);
        float* bsl = a1_tail + wid * 128;
        int* zpw_l = reinterpret_cast<int*>(a1_tail + 512) + wid * 128;
        int* csw_l = reinterpret_cast<int*>(a1_tail + 1024) + wid * 128;
        // The layer bias of the wave's 128 columns (fp16 -> fp32, exact),
        // fetched under the outlier staging below.
        // Range-checked loads with no branch around them (columns past o, or
        // no bias at all, read zero), so the wait for them falls at their use.
        const bool has_bias = bias != nullptr;
        const __amdgpu_buffer_rsrc_t rBias = make_rsrc(bias, has_bias ? static_cast<uint32_t>(2 * o) : 0u);
        uint16_t bias_bits[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t col = static_cast<uint32_t>(o0 + wo * 128 + lane + 64 * i);
            bias_bits[i] = __builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(rBias, 2 * col, 0, 0));
        }
        // The first nst = min(nsl, 1 + kMaxOnceSlices) slices are staged in
        // LDS (slice 0 in olds, before the K loop); any further ones are
        // read from global memory block by block.
        const int nsl = (n_o + 15) / 16;
        const int nst = nsl < 1 + kMaxOnceSlices ? nsl : 1 + kMaxOnceSlices;
        for (int q = 1; q < nst; ++q)
            stage_outlier_slice(q, n_o, wu, lane, o0, s0, s, o, ldo, idx, rW, rX, slice_at(q), !w8);
        if (w8)
            for (int q = 0; q < nst; ++q) stage_w8_slice(q, n_o, o0, o, idx, Wq, c_w, q ? slice_at(q) : olds);
        // 1 / c_x and 1 / c_w of the tile (reciprocals to 1 ulp), in place
#pragma unroll
        for (int i = 0; i < 2; ++i) scl[t + 256 * i] = __builtin_amdgcn_rcpf(scl[t + 256 * i]);
        if (has_bias) {
#pragma unroll
            for (int i = 0; i < 2; ++i) bsl[lane + 64 * i] = half_bits_to_float(bias_bits[i]);
        }
        if constexpr (zpm) {
            // sum over k not in O of Wq_kj = the column's code sum minus the
            // codes of the outlier rows (read from the panels)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int64_t col = o0 + wo * 128 + lane + 64 * i;
                const bool ok = col < o;
                int cs = ok ? zp.colsum_w[col] : 0;
                for (int q = 0; q < n_o; ++q) {
                    const int64_t k = idx[q];
                    if (ok) cs -= Wq[(k >> 6) * o * 64 + col * 64 + (k & 63)];
                }
                zpw_l[lane + 64 * i] = ok ? zp.zp_w[col] : 0;
                csw_l[lane + 64 * i] = cs;
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (!w8) {
            // W parts transposed once, so that both MFMA operands are 16-byte reads
            if (nst > 0) transpose_w_slice(olds);
            for (int q = 1; q < nst; ++q) transpose_w_slice(slice_at(q));
        }
        // One 32-row block at a time: a lane then holds 4-column runs of one
        // row across all 128 columns of the wave. Written once for the usual
        // case (every outlier slice staged in LDS) and once with the slices
        // past those read from global memory, so that the common path carries
        // none of the other's registers (which pushed values to scratch, and
        // each reload's wait then also waited for the previous block's stores).
        auto blocks = [&](auto with_global) {
        // The lane's indices are derived again here from an opaque copy of
        // the thread index: left to the compiler, it computed them before
        // the K loop and carried them (or spilled them) across it.
        // The wavefront index goes to a scalar register, so that the output
        // descriptor and the LDS bases built from it are known to be uniform
        // (a descriptor in vector registers costs a loop around every store).
        int te = static_cast<int>(threadIdx.x);
        asm volatile("" : "+v"(te));
        const int lane = te & 63, wid = __builtin_amdgcn_readfirstlane(te >> 6), wo = wid & 1, ws = wid >> 1,
                  r32 = lane & 31, khalf = lane >> 5;
        uint16_t* out_st = wid < 3 ? reinterpret_cast<uint16_t*>(A1) + wid * kOutWave : reinterpret_cast<uint16_t*>(B1);
        const float* inv_rows = scl + ws * 128;
        const float* invw = scl + 256 + wo * 128;
        const float* bsl = a1_tail + wid * 128;
        const int* zpw_l = reinterpret_cast<const int*>(a1_tail + 512) + wid * 128;
        const int* csw_l = reinterpret_cast<const int*>(a1_tail + 1024) + wid * 128;
        // 1 / c_w of the lane's 64 columns and slice 0's W operands do not
        // depend on the row block: read once.
        v4f iwr[4][4];
#pragma unroll
        for (int ob = 0; ob < 4; ++ob)
#pragma unroll
            for (int g = 0; g < 4; ++g) iwr[ob][g] = *reinterpret_cast<const v4f*>(invw + ob * 32 + 8 * g + 4 * khalf);
        v8h wa0[4] = {};
        if (nst > 0)
#pragma unroll
            for (int ob = 0; ob < 4; ++ob) wa0[ob] = slice_w_operand(olds, wo, ob, r32, khalf);
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const float inv_x = inv_rows[sb * 32 + r32];
            // zeropoint: zp_x of the lane's row and rowsum + (h - |O|) zp_x
            double zx = 0.0, zr = 0.0;
            if constexpr (zpm) {
                const int64_t srow = s0 + ws * 128 + sb * 32 + r32;
                if (srow < s) {
                    const int z = zp.zp_x[srow];
                    zx = static_cast<double>(z);
                    zr = static_cast<double>(static_cast<int64_t>(zp.rowsum_x[srow]) + (h - n_o) * static_cast<int64_t>(z));
                }
            }
            // Dequantise the four column blocks: f = C_i32 * (1/c_x) *
            // (1/c_w); zeropoint: C' = C_i32 + zp_w (rowsum + (h - |O|) zp_x)
            // + zp_x colsum' by two fp64 FMAs (exact while every term is
            // below 2^53, i.e. for zero points below 2^17 in magnitude), times
            // (1/nd_x) * (1/nd_w). fp64 rather than int64 keeps the
            // accumulators in registers.
            v16f f[4];
#pragma unroll
            for (int ob = 0; ob < 4; ++ob)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const v4f iw = iwr[ob][g];
                    if constexpr (zpm) {
                        const v4i zw = *reinterpret_cast<const v4i*>(zpw_l + ob * 32 + 8 * g + 4 * khalf);
                        const v4i cw = *reinterpret_cast<const v4i*>(csw_l + ob * 32 + 8 * g + 4 * khalf);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const double cp = __fma_rn(zx, static_cast<double>(cw[e]),
                                                       __fma_rn(static_cast<double>(zw[e]), zr,
                                                                static_cast<double>(acc[ob][sb][4 * g + e])));
                            f[ob][4 * g + e] = static_cast<float>(cp) * (inv_x * iw[e]);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            f[ob][4 * g + e] = static_cast<float>(acc[ob][sb][4 * g + e]) * (inv_x * iw[e]);
                    }
                }
            // Outlier product X_O W[idx, :] on top (fp32 accumulate), one
            // staged slice at a time for all four column blocks.
            if (nst > 0) mfma4_f16_vgpr(wa0, slice_x_operand(olds, ws, sb, r32, khalf), f);
            for (int q = 1; q < nst; ++q) {
                const uint16_t* sl = slice_at(q);
                v8h wa[4];
#pragma unroll
                for (int ob = 0; ob < 4; ++ob) wa[ob] = slice_w_operand(sl, wo, ob, r32, khalf);
                mfma4_f16_vgpr(wa, slice_x_operand(sl, ws, sb, r32, khalf), f);
            }
            if constexpr (decltype(with_global)::value)
#pragma unroll
                for (int ob = 0; ob < 4; ++ob)
                    for (int q = nst; q < nsl; ++q)
                        f[ob] = apply_outlier_slice_global(q, n_o, o0, s0, s, o, X_O, ldo, idx, W, Wq, c_w, wo, ws, sb,
                                                           ob, r32, khalf, f[ob]);
#pragma unroll
            for (int ob = 0; ob < 4; ++ob) {
                // The layer bias, in the same fp32 sum before the rounding.
                if (has_bias) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const v4f bv = *reinterpret_cast<const v4f*>(bsl + ob * 32 + 8 * g + 4 * khalf);
#pragma unroll
                        for (int e = 0; e < 4; ++e) f[ob][4 * g + e] += bv[e];
                    }
                }
                // Round once to fp16 and stage in this wavefront's LDS area
                // (LDS operations of one wavefront execute in order, so its
                // own reads below see these writes).
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint32_t lo = pack_half2(f[ob][4 * g], f[ob][4 * g + 1]);
                    const uint32_t hi = pack_half2(f[ob][4 * g + 2], f[ob][4 * g + 3]);
                    *reinterpret_cast<uint2*>(out_st + r32 * kOutRow + ob * 32 + 8 * g + 4 * khalf) =
                        make_uint2(lo, hi);
                }
            }
            store_staged_block(out_st, C, s0 + ws * 128 + sb * 32, o0 + wo * 128, s, o, lane);
        }
        };
        if (nsl > nst)
            blocks(std::true_type{});
        else
            blocks(std::false_type{});
    }
}

// ------------------------------------------------------------------ decode
// Operands of one 32-deep slice (outlier columns 32 kb .. 32 kb + 31) of the
// fp16 outlier product for one 16 x 16 output tile, in the lane layout of
// v_mfma_f32_16x16x32_f16: wa holds W[idx[k], ocol], xb holds X_O[srow, k],
// k = 32 kb + 8 (lane / 16) + e, ocol = ocol0 + lane % 16, srow = srow0 +
// lane % 16. Indices come through scalar loads; columns past |O|, rows past
// s and columns past o read as zero. Shared by the decode epilogue and the
// standalone outlier product (register layout: register r of the result
// holds D[o = 4 (lane / 16) + r][s = lane % 16]).
__device__ __forceinline__ void outlier_operands_16(int kb, int n, int lane, int64_t ocol0, int64_t srow0,
                                                    int64_t s, int64_t o, const uint16_t* __restrict__ X_O,
                                                    int64_t ldo, const int32_t* __restrict__ idx,
                                                    const uint16_t* __restrict__ W, const int8_t* __restrict__ Wq,
                                                    const float* __restrict__ c_w, v8h& wa, v8h& xb) {
    int id[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) id[j] = idx[kb * 32 + j];     // uniform address: scalar loads
    const int g = lane >> 4;
    const int kbase = kb * 32 + 8 * g;
    const int64_t ocol = ocol0 + (lane & 15);
    const bool col_ok = ocol < o;
    // without a resident fp16 W the rows are rebuilt from the int8 codes
    const float inv_cw = inverse_scale(W == nullptr && col_ok ? c_w[ocol] : 1.0f);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bool ok = col_ok && kbase + e < n;
        const int sel = g == 0 ? id[e] : g == 1 ? id[8 + e] : g == 2 ? id[16 + e] : id[24 + e];
        const int row = ok ? sel : 0;
        uint16_t bits = 0;
        if (ok) bits = W != nullptr ? W[static_cast<int64_t>(row) * o + ocol] : dequantized_weight(Wq, inv_cw, row, ocol, o);
        wa[e] = __builtin_bit_cast(_Float16, bits);
    }
    const int64_t srow = srow0 + (lane & 15);
    const bool rok = srow < s;
    const v8h v = *reinterpret_cast<const v8h*>(X_O + (rok ? srow : 0) * ldo + kbase);
#pragma unroll
    for (int e = 0; e < 8; ++e) xb[e] = rok ? v[e] : static_cast<_Float16>(0.0f);
}

// f += X_O W[idx, :] over all outlier columns for one 16 x 16 tile; the
// first slice's operands may be passed in already loaded.
__device__ __forceinline__ v4f outlier_tile_16x16(v4f f, int lane, int64_t ocol0, int64_t srow0, int64_t s,
                                                   int64_t o, const uint16_t* __restrict__ X_O, int64_t ldo,
                                                   const int32_t* __restrict__ idx, int n,
                                                   const uint16_t* __restrict__ W, const int8_t* __restrict__ Wq,
                                                   const float* __restrict__ c_w, const v8h* first) {
    for (int kb = 0; kb * 32 < n; ++kb) {
        v8h wa, xb;
        if (kb == 0 && first != nullptr) {
            wa = first[0];
            xb = first[1];
        } else {
            outlier_operands_16(kb, n, lane, ocol0, srow0, s, o, X_O, ldo, idx, W, Wq, c_w, wa, xb);
        }
        f = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, xb, f, 0, 0, 0);
    }
    return f;
}


// The fused epilogue of one 16 x 16 output tile of the weight-streaming
// products (rows srow0 .. + 15, columns ocol0 .. + 15) from its exact int32
// sum. Lane layout of a 16x16 accumulator: register r holds
// D[o = 4 g + r][s = r16]. bias4 is the layer bias of the lane's 4 columns
// (fetched by the caller ahead of time); first, if not null, holds the
// tile's first outlier slice, also fetched ahead of time.
template <GemmOut MODE>
__device__ __forceinline__ void decode_tile_out(v4i sum, int lane, int64_t srow0, int64_t ocol0, int64_t s, int64_t h,
                                                int64_t o, const float* __restrict__ c_x,
                                                const float* __restrict__ c_w, const uint16_t* __restrict__ X_O,
                                                int64_t ldo, const int32_t* __restrict__ idx, int n_o,
                                                const uint16_t* __restrict__ W, const int8_t* __restrict__ Wq,
                                                bool has_bias, uint2 bias4, void* __restrict__ Cout, const ZpArgs& zp,
                                                const v8h* first) {
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t srow = srow0 + r16;
    const int64_t ocol = ocol0 + 4 * g;
    if constexpr (MODE == GemmOut::Int32) {
        int32_t* C = static_cast<int32_t*>(Cout);
        if (srow < s) *reinterpret_cast<v4i*>(C + srow * o + ocol) = sum;
    } else {
        uint16_t* C = static_cast<uint16_t*>(Cout);
        const float inv_x = __builtin_amdgcn_rcpf(srow < s ? c_x[srow] : 1.0f);
        const v4f cw = *reinterpret_cast<const v4f*>(c_w + ocol);
        v4f f;
        if constexpr (MODE == GemmOut::ZeroPoint) {
            // C' = C_i32 + zp_w (rowsum + (h - |O|) zp_x) + zp_x colsum', exact
            // in int64 (colsum' = the column's code sum over the non-outlier rows)
            const int zx = srow < s ? zp.zp_x[srow] : 0;
            const int64_t zr =
                srow < s ? static_cast<int64_t>(zp.rowsum_x[srow]) + (h - n_o) * static_cast<int64_t>(zx) : 0;
            const v4i zw = *reinterpret_cast<const v4i*>(zp.zp_w + ocol);
            v4i cs = *reinterpret_cast<const v4i*>(zp.colsum_w + ocol);
            for (int q = 0; q < n_o; ++q) {
                const int64_t k = idx[q];
                const int8_t* p = Wq + (k >> 6) * o * 64 + ocol * 64 + (k & 63);
#pragma unroll
                for (int e = 0; e < 4; ++e) cs[e] -= p[e * 64];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t cp = static_cast<int64_t>(sum[e]) + static_cast<int64_t>(zw[e]) * zr +
                                   static_cast<int64_t>(zx) * static_cast<int64_t>(cs[e]);
                f[e] = static_cast<float>(cp) * (inv_x * __builtin_amdgcn_rcpf(cw[e]));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = static_cast<float>(sum[e]) * (inv_x * __builtin_amdgcn_rcpf(cw[e]));
        }
        f = outlier_tile_16x16(f, lane, ocol0, srow0, s, o, X_O, ldo, idx, n_o, W, Wq, c_w, first);
        if (has_bias) {
            f[0] += half_bits_to_float(bias4.x & 0xffffu);
            f[1] += half_bits_to_float(bias4.x >> 16);
            f[2] += half_bits_to_float(bias4.y & 0xffffu);
            f[3] += half_bits_to_float(bias4.y >> 16);
        }
        if (srow < s) {
            const uint32_t lo = pack_half2(f[0], f[1]);
            const uint32_t hi = pack_half2(f[2], f[3]);
            *reinterpret_cast<uint2*>(C + srow * o + ocol) = make_uint2(lo, hi);
        }
    }
}

// Decode: block = kDecodeSplit (4) wavefronts on the same 16*NT output
// columns, each streaming its share of K from HBM with two register batches
// of kDecodeU K steps in flight (range-checked loads: steps past a wave's
// range read as zero), then an exact int32 reduction of the partial tiles
// through LDS. Up to 16 rows of X (one operand of the 16 x 16 x 64 MFMA).
template <GemmOut MODE, int NT, int kDecodeU = 4, int kDecodeSplit = 4>
__global__ __launch_bounds__(256) void k_gemm_decode(const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq,
                                                     int64_t s, int64_t h, int64_t o,
                                                     const float* __restrict__ c_x, const float* __restrict__ c_w,
                                                     const uint16_t* __restrict__ X_O, int64_t ldo,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ n_out,
                                                     const uint16_t* __restrict__ W,
                                                     const uint16_t* __restrict__ bias, void* __restrict__ Cout,
                                                     uint32_t* __restrict__ clear, int clear_words, ZpArgs zp) {
    __shared__ v4i red[kDecodeSplit][NT][64];
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < clear_words; i += 256) clear[i] = 0u;
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int64_t obase = static_cast<int64_t>(blockIdx.x) * 16 * NT;
    const int r16 = lane & 15, g = lane >> 4;

    // Columns obase .. obase + 16 NT - 1 of every panel (always inside o:
    // 16 NT divides 64): panel p of them starts p o 64 bytes past the
    // resource base, a step's uniform offset.
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(Wq + obase * 64, static_cast<uint32_t>(h * o - obase * 64));
    // Xq rows 0 .. s - 1; lanes of rows >= s fall past the range and read zero.
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Xq, static_cast<uint32_t>(s * h));
    uint32_t vA[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vA[nt] = static_cast<uint32_t>((nt * 16 + r16) * 64 + g * 16);
    const uint32_t vB = static_cast<uint32_t>(r16 * h + g * 16);

    // Wavefronts that finish an output tile fetch the first slice of its
    // outlier operands now, so the loads complete under the K loop.
    int n_o = 0;
    v8h pre[2];
    uint2 bias4 = make_uint2(0u, 0u);   // the layer bias of this lane's 4 output columns
    if constexpr (MODE == GemmOut::Mixed || MODE == GemmOut::ZeroPoint) {
        n_o = __builtin_amdgcn_readfirstlane(n_out[0]);
        if (wid < NT && n_o > 0)
            outlier_operands_16(0, n_o, lane, obase + wid * 16, 0, s, o, X_O, ldo, idx, W, Wq, c_w, pre[0], pre[1]);
        if (wid < NT && bias != nullptr)
            bias4 = *reinterpret_cast<const uint2*>(bias + obase + wid * 16 + 4 * g);
    }

    const int64_t nsteps = h / 64;
    const int64_t per = ((nsteps + kDecodeSplit - 1) / kDecodeSplit + kDecodeU - 1) / kDecodeU * kDecodeU;
    const int64_t st0 = wid * per < nsteps ? wid * per : nsteps;
    const int64_t st1 = st0 + per < nsteps ? st0 + per : nsteps;

    v4i acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = v4i{0, 0, 0, 0};
    v4i a0[kDecodeU][NT], b0[kDecodeU], a1[kDecodeU][NT], b1[kDecodeU];

    // Steps past the wave's range get an out-of-range lane offset and a zero
    // scalar offset, so no sum of the two can wrap back into the range; rows
    // of X past s lie past the end of rB through their lane offset.
    auto load = [&](v4i (&a)[kDecodeU][NT], v4i (&b)[kDecodeU], int64_t stb) {
#pragma unroll
        for (int u = 0; u < kDecodeU; ++u) {
            const bool ok = stb + u < st1;
            const uint32_t kA = ok ? static_cast<uint32_t>((stb + u) * o * 64) : 0u;
            const uint32_t kB = ok ? static_cast<uint32_t>((stb + u) * 64) : 0u;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) a[u][nt] = buf_load16_nt(rA, ok ? vA[nt] : kOutOfRange, kA);
            b[u] = buf_load16(rB, ok ? vB : kOutOfRange, kB);
        }
    };
    auto mma = [&](v4i (&a)[kDecodeU][NT], v4i (&b)[kDecodeU]) {
#pragma unroll
        for (int u = 0; u < kDecodeU; ++u)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][nt], b[u], acc[nt], 0, 0, 0);
    };

    load(a0, b0, st0);
    for (int64_t stb = st0; stb < st1; stb += 2 * kDecodeU) {
        load(a1, b1, stb + kDecodeU);
        mma(a0, b0);
        load(a0, b0, stb + 2 * kDecodeU);
        mma(a1, b1);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[wid][nt][lane] = acc[nt];
    __syncthreads();
    if (wid < NT) {
        v4i sum = red[0][wid][lane];
#pragma unroll
        for (int w = 1; w < kDecodeSplit; ++w) sum += red[w][wid][lane];
        // the first outlier slice was fetched before the K loop
        decode_tile_out<MODE>(sum, lane, 0, obase + wid * 16, s, h, o, c_x, c_w, X_O, ldo, idx, n_o, W, Wq,
                              bias != nullptr, bias4, Cout, zp, pre);
    }
}

// Weight streaming for up to 128 rows with the codes of X shared through
// LDS (the forward routes 17..128 rows here, and 1..16 rows on layers that
// the K-split kernel cannot spread evenly over the CUs): each of the kWaves
// wavefronts of a block owns 16 NT adjacent output columns and streams
// their weights over the whole of K, kRing K steps ahead in registers; the
// block stages X's codes (RG row groups of 16) in LDS chunks of
// kSkinnyChunk K steps, double-buffered by direct-to-LDS loads, and every
// wavefront reads them from there. A block thus fetches X once (not once
// per wavefront) and needs no reduction; its wavefronts meet once per
// chunk. The launch sizes blocks to one per CU where the columns allow: a
// CU's texture address unit serves both the weight stream and the staging
// of X (16 bytes per lane each), so every extra block per CU re-staging X
// slows the weight stream. Columns are always whole 16-column tiles (16 NT
// divides 64, which divides o); wavefronts past o stage X and wait with the
// others but read no weights and write nothing.
// Measured on 12288 x 49152 (forward, us): 96.4 / 97.1 / 99.0 / 103.2 /
// 106.9 / 117.5 / 135.9 for 17 / 32 / 48 / 64 / 65 / 96 / 128 rows, where
// the tiled product takes 155-165; with three 4-wavefront blocks per CU
// instead of one, 64 rows took 144.7. NT = 2, longer rings or chunks, three
// LDS stages and X staged through registers measured the same or slower.
constexpr int kSkinnyChunk = 4;

template <GemmOut MODE, int NT, int RG, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void k_gemm_skinny(const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq,
                                                     int64_t s, int64_t h, int64_t o,
                                                     const float* __restrict__ c_x, const float* __restrict__ c_w,
                                                     const uint16_t* __restrict__ X_O, int64_t ldo,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ n_out,
                                                     const uint16_t* __restrict__ W,
                                                     const uint16_t* __restrict__ bias, void* __restrict__ Cout,
                                                     uint32_t* __restrict__ clear, int clear_words, ZpArgs zp) {
    constexpr int kRing = 2 * kSkinnyChunk;   // weight steps in flight
    static_assert(kSkinnyChunk * NT < 16, "the wait below encodes the count in 4 bits");
    // xs[buffer][step of the chunk][row group]: one 16 x 64 operand, lane-ordered
    __shared__ v4i xs[2][kSkinnyChunk][RG][64];
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < clear_words; i += 64 * kWaves) clear[i] = 0u;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t wcol = (static_cast<int64_t>(blockIdx.x) * kWaves + wid) * 16 * NT;
    const bool live = wcol < o;
    const int64_t nsteps = h / 64;

    // this wavefront's weight columns: panel p of them starts p o 64 bytes
    // past the resource base (a step's uniform offset); a wavefront past o
    // gets an empty resource
    const __amdgpu_buffer_rsrc_t rA =
        make_rsrc(live ? Wq + wcol * 64 : Wq, live ? static_cast<uint32_t>(h * o - wcol * 64) : 0u);
    uint32_t vA[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vA[nt] = static_cast<uint32_t>((nt * 16 + r16) * 64 + g * 16);
    auto load_w = [&](v4i (&a)[NT], int64_t st) {
        const bool ok = st < nsteps;
        const uint32_t k = ok ? static_cast<uint32_t>(st * o * 64) : 0u;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) a[nt] = buf_load16_nt(rA, ok ? vA[nt] : kOutOfRange, k);
    };
    // X's codes: rows 0 .. s - 1 (lanes of rows >= s fall past the range and
    // read zero; so do steps past K). Wavefront w stages operands
    // b = w, w + kWaves, ... of each chunk: step b / RG, row group b % RG.
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(Xq, static_cast<uint32_t>(s * h));
    auto stage_x = [&](int64_t chunk, int buf) {
        for (int b = wid; b < kSkinnyChunk * RG; b += kWaves) {
            const int j = b / RG, rg = b % RG;
            const int64_t st = chunk * kSkinnyChunk + j;
            const uint32_t off = st < nsteps ? static_cast<uint32_t>((rg * 16 + r16) * h + st * 64 + g * 16) : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, LDS_PTR(&xs[buf][j][rg][0]), 16, off, 0, 0, 0);
        }
    };

    int n_o = 0;
    uint2 bias4[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bias4[nt] = make_uint2(0u, 0u);
    if constexpr (MODE == GemmOut::Mixed || MODE == GemmOut::ZeroPoint) {
        n_o = __builtin_amdgcn_readfirstlane(n_out[0]);
        if (live && bias != nullptr)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) bias4[nt] = *reinterpret_cast<const uint2*>(bias + wcol + nt * 16 + 4 * g);
    }

    v4i acc[RG][NT];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rg][nt] = v4i{0, 0, 0, 0};
    v4i wr[kRing][NT];
#pragma unroll
    for (int i = 0; i < kRing; ++i) load_w(wr[i], i);
    stage_x(0, 0);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): chunk 0 (and the first weights) in place
    __syncthreads();

    // One chunk from buffer `buf`, whose weights sit in ring slots slot0 ..
    // slot0 + kSkinnyChunk - 1; the next chunk is staged into the other
    // buffer first, and each slot is refilled kRing steps ahead once used.
    auto chunk_step = [&](int64_t c, int buf, int slot0) __attribute__((always_inline)) {
        stage_x(c + 1, buf ^ 1);
        asm volatile("" ::: "memory");   // the weight loads below stay after the staging
#pragma unroll
        for (int j = 0; j < kSkinnyChunk; ++j) {
            v4i b[RG];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) b[rg] = xs[buf][j][rg][lane];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    acc[rg][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wr[slot0 + j][nt], b[rg], acc[rg][nt], 0, 0, 0);
            load_w(wr[slot0 + j], c * kSkinnyChunk + j + kRing);
        }
        // The barrier's fence does not cover direct-to-LDS loads: wait for
        // this wavefront's staging of chunk c + 1, which is older than the
        // kSkinnyChunk NT weight loads issued after it (loads return in order).
        __builtin_amdgcn_s_waitcnt(0x0f70 | (kSkinnyChunk * NT));
        __syncthreads();
    };
    const int64_t nchunks = (nsteps + kSkinnyChunk - 1) / kSkinnyChunk;
    for (int64_t c = 0; c < nchunks; c += 2) {
        chunk_step(c, 0, 0);
        chunk_step(c + 1, 1, kSkinnyChunk);   // past K when nchunks is odd: zeros
    }
    // the last staging (past K) still writes zeros into LDS: let it land
    // before the block can end
    __builtin_amdgcn_s_waitcnt(0x0f70);

    if (!live) return;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
        if (rg * 16 < s)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                decode_tile_out<MODE>(acc[rg][nt], lane, rg * 16, wcol + nt * 16, s, h, o, c_x, c_w, X_O, ldo, idx,
                                      n_o, W, Wq, bias != nullptr, bias4[nt], Cout, zp, nullptr);
}

// ------------------------------------------------------------------ single-launch decode forward
// The whole forward of [DIGEST] "The Full LLM.int8() Algorithm" (Steps 1-5)
// in one launch for few rows (s <= 16), where the two prologue launches of
// the three-launch forward cost a tenth of a weight-streaming step
// ([DIGEST] "Runtime Overhead Makes LLM.int8() Slower Than 16-Bit for
// Models Below ~13B Parameters" names these per-layer steps as the overhead).
// Every block works from X alone and waits for no other block:
//  1. it issues its first weight batch, then scans all of X (s x h fp16, a
//     few hundred KiB at most: L2 hits for all but the first blocks) for
//     the outlier mask and the per-row maxima over the non-outlier columns
//     (each thread sees every row of its 8-column chunks, so a chunk's
//     flags are final before its values enter the row maxima);
//  2. it streams its weight columns as k_gemm_decode does, with the int8
//     operand of X quantised on the fly from X, the mask and the row
//     constants in LDS;
//  3. its epilogue takes the outlier columns by rank from the mask (binary
//     search over the prefix counts) and reads their values from X and W.
// Block 0 also writes the intermediates (mask, index list, |O|, c_x, Xq,
// X_O with its zero padding) for inspection.

// Column of rank k in O (its k-th member in ascending order), k < |O|, from
// the LDS mask words and their exclusive prefix counts.
__device__ __forceinline__ int kth_outlier(const uint32_t* smask, const int* pre, int nw, int k) {
    int lo = 0, hi = nw - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= k)
            lo = mid;
        else
            hi = mid - 1;
    }
    uint32_t bits = smask[lo];
    for (int r = k - pre[lo]; r > 0; --r) bits &= bits - 1u;
    return lo * 32 + __ffs(bits) - 1;
}

template <int NT, int kDecodeU = 2, int kDecodeSplit = 4>
__global__ __launch_bounds__(256) void k_decode_fused(const uint16_t* __restrict__ X, int s, int64_t h, int64_t o,
                                                      Threshold th, const int8_t* __restrict__ Wq,
                                                      const float* __restrict__ c_w, const uint16_t* __restrict__ W,
                                                      const uint16_t* __restrict__ bias, uint16_t* __restrict__ C,
                                                      uint32_t* __restrict__ mask_out, int32_t* __restrict__ idx_out,
                                                      int32_t* __restrict__ n_out_out, int8_t* __restrict__ Xq_out,
                                                      float* __restrict__ c_x_out, uint16_t* __restrict__ X_O_out,
                                                      int64_t ldo) {
    extern __shared__ uint32_t dyn[];   // mask words [nw], then their exclusive prefix counts [nw]
    __shared__ v4i red[kDecodeSplit][NT][64];
    __shared__ uint32_t rmax[4][16];
    __shared__ float cx[16];
    __shared__ int wsum[4];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int nw = static_cast<int>(h / 32);
    uint32_t* smask = dyn;
    int* pre = reinterpret_cast<int*>(dyn + nw);
    const int64_t obase = static_cast<int64_t>(blockIdx.x) * 16 * NT;
    const int r16 = lane & 15, g = lane >> 4;
    const bool first = blockIdx.x == 0;

    // The block's weight columns, as in k_gemm_decode.
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(Wq + obase * 64, static_cast<uint32_t>(h * o - obase * 64));
    uint32_t vA[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) vA[nt] = static_cast<uint32_t>((nt * 16 + r16) * 64 + g * 16);
    const int64_t nsteps = h / 64;
    const int64_t per = ((nsteps + kDecodeSplit - 1) / kDecodeSplit + kDecodeU - 1) / kDecodeU * kDecodeU;
    const int64_t st0 = wid * per < nsteps ? wid * per : nsteps;
    const int64_t st1 = st0 + per < nsteps ? st0 + per : nsteps;
    v4i a0[kDecodeU][NT], a1[kDecodeU][NT];
    auto load_w = [&](v4i (&a)[kDecodeU][NT], int64_t stb) {
#pragma unroll
        for (int u = 0; u < kDecodeU; ++u) {
            const bool ok = stb + u < st1;
            const uint32_t kA = ok ? static_cast<uint32_t>((stb + u) * o * 64) : 0u;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) a[u][nt] = buf_load16_nt(rA, ok ? vA[nt] : kOutOfRange, kA);
        }
    };
    load_w(a0, st0);

    // 1. Scan of X: mask, and the packed |x| maxima of each row over this
    // thread's non-outlier columns (rows past s read zero from the resource,
    // which neither flags a column nor raises a maximum).
    for (int w = t; w < nw; w += 256) smask[w] = 0u;
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rX = range_rsrc(X, static_cast<uint32_t>(2 * static_cast<int64_t>(s) * h));
    uint32_t rm[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) rm[i] = 0u;
    for (int64_t c = t; c < h / 8; c += 256) {
        uint4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            v[i] = i < s ? load_chunk_rsrc(rX, static_cast<uint32_t>(2 * (i * h + c * 8))) : make_uint4(0, 0, 0, 0);
        uint4 d = detect_init();
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (i < s) detect_fold(d, v[i], th.thr2);
        const uint32_t f = detect_flags(d, th.span);
        if (f) atomicOr(&smask[c >> 2], f << ((c & 3) * 8));
#pragma unroll
        for (int i = 0; i < 16; ++i) rm[i] = chunk_absmax_fold(chunk_clear(v[i], f), rm[i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t m2 = rm[i];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            m2 = pk_max_u16(m2, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m2), off, kWave)));
        if (lane == 0) rmax[wid][i] = m2;
    }
    __syncthreads();
    if (t < 16)
        cx[t] = absmax_scale(absmax_value(pk_max_u16(pk_max_u16(rmax[0][t], rmax[1][t]),
                                                     pk_max_u16(rmax[2][t], rmax[3][t]))));
    const int n = block_mask_prefix(smask, pre, nw, wsum, 256);   // its barriers also publish cx

    if (first) {
        emit_outlier_set(smask, pre, nw, n, mask_out, idx_out, n_out_out, 256);
        if (t < s) c_x_out[t] = cx[t];
        // X_O: the outlier columns of every row by rank, zero up to a multiple of 32
        for (int w = t; w < nw; w += 256) {
            int r = pre[w];
            for (uint32_t b = smask[w]; b; b &= b - 1u, ++r) {
                const int64_t col = static_cast<int64_t>(w) * 32 + __ffs(b) - 1;
                for (int i = 0; i < s; ++i) X_O_out[i * ldo + r] = X[i * h + col];
            }
        }
        const int npad = (n + 31) & ~31;
        for (int k = n + t; k < npad; k += 256)
            for (int i = 0; i < s; ++i) X_O_out[i * ldo + k] = 0;
    }

    // 2. Weight stream with the int8 operand of X made on the fly: lane
    // (r16, g) of step st holds the codes of X[r16, 64 st + 16 g .. + 15].
    uint4 x0[kDecodeU][2], x1[kDecodeU][2];
    auto load_x = [&](uint4 (&x)[kDecodeU][2], int64_t stb) {
#pragma unroll
        for (int u = 0; u < kDecodeU; ++u) {
            const bool ok = stb + u < st1;
            const uint32_t off = ok ? static_cast<uint32_t>(2 * (r16 * h + (stb + u) * 64 + 16 * g)) : kOutOfRange;
            x[u][0] = load_chunk_rsrc(rX, off);
            x[u][1] = load_chunk_rsrc(rX, off + 16);
        }
    };
    const float scr = cx[r16];
    auto codes = [&](const uint4 (&x)[kDecodeU][2], int64_t stb, v4i (&b)[kDecodeU]) {
#pragma unroll
        for (int u = 0; u < kDecodeU; ++u) {
            b[u] = v4i{0, 0, 0, 0};
            if (stb + u < st1) {
                const int64_t col = (stb + u) * 64 + 16 * g;
                const uint32_t bits = (smask[col >> 5] >> (col & 31)) & 0xffffu;
                const uint2 q0 = chunk_quantize(chunk_clear(x[u][0], bits & 0xffu), scr);
                const uint2 q1 = chunk_quantize(chunk_clear(x[u][1], bits >> 8), scr);
                b[u] = v4i{static_cast<int>(q0.x), static_cast<int>(q0.y), static_cast<int>(q1.x),
                           static_cast<int>(q1.y)};
                if (first && r16 < s) *reinterpret_cast<v4i*>(Xq_out + r16 * h + col) = b[u];
            }
        }
    };
    v4i acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = v4i{0, 0, 0, 0};
    auto mma = [&](v4i (&a)[kDecodeU][NT], v4i (&b)[kDecodeU]) {
#pragma unroll
        for (int u = 0; u < kDecodeU; ++u)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][nt], b[u], acc[nt], 0, 0, 0);
    };
    v4i b[kDecodeU];
    load_x(x0, st0);
    for (int64_t stb = st0; stb < st1; stb += 2 * kDecodeU) {
        load_w(a1, stb + kDecodeU);
        load_x(x1, stb + kDecodeU);
        codes(x0, stb, b);
        mma(a0, b);
        load_w(a0, stb + 2 * kDecodeU);
        load_x(x0, stb + 2 * kDecodeU);
        codes(x1, stb + kDecodeU, b);
        mma(a1, b);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[wid][nt][lane] = acc[nt];
    __syncthreads();
    if (wid >= NT) return;
    const int nt = wid;
    v4i sum = red[0][nt][lane];
#pragma unroll
    for (int w = 1; w < kDecodeSplit; ++w) sum += red[w][nt][lane];

    // 3. Epilogue (lane layout of a 16x16 accumulator: register r holds
    // D[o = 4 g + r][s = r16]).
    const int64_t ocol0 = obase + nt * 16;
    const int64_t ocol = ocol0 + 4 * g;
    const float inv_x = __builtin_amdgcn_rcpf(scr);
    const v4f cw = *reinterpret_cast<const v4f*>(c_w + ocol);
    v4f f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = static_cast<float>(sum[e]) * (inv_x * __builtin_amdgcn_rcpf(cw[e]));
    // Outlier product X_O W[idx, :], 32 outlier columns per fp16 MFMA.
    {
        const int64_t wcol = ocol0 + r16;   // this lane's column of W in the operand layout
        const float inv_cw = inverse_scale(W == nullptr ? c_w[wcol] : 1.0f);
        for (int kb = 0; kb * 32 < n; ++kb) {
            v8h wa, xb;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = kb * 32 + 8 * g + e;
                uint16_t wbits = 0, xbits = 0;
                if (k < n) {
                    const int id = kth_outlier(smask, pre, nw, k);
                    wbits = W != nullptr ? W[static_cast<int64_t>(id) * o + wcol]
                                         : dequantized_weight(Wq, inv_cw, id, wcol, o);
                    xbits = r16 < s ? X[r16 * h + id] : static_cast<uint16_t>(0);
                }
                wa[e] = __builtin_bit_cast(_Float16, wbits);
                xb[e] = __builtin_bit_cast(_Float16, xbits);
            }
            f = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, xb, f, 0, 0, 0);
        }
    }
    if (bias != nullptr) {
        const uint2 b4 = *reinterpret_cast<const uint2*>(bias + ocol);
        f[0] += half_bits_to_float(b4.x & 0xffffu);
        f[1] += half_bits_to_float(b4.x >> 16);
        f[2] += half_bits_to_float(b4.y & 0xffffu);
        f[3] += half_bits_to_float(b4.y >> 16);
    }
    if (r16 < s) {
        const uint32_t lo = pack_half2(f[0], f[1]);
        const uint32_t hi = pack_half2(f[2], f[3]);
        *reinterpret_cast<uint2*>(C + r16 * o + ocol) = make_uint2(lo, hi);
    }
}

// ------------------------------------------------------------------ outlier product alone
// One wavefront per 16x16 tile of C_O (fp32).
__global__ __launch_bounds__(256) void k_outlier_only(const uint16_t* __restrict__ X_O, int64_t ldo,
                                                      const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ n_out,
                                                      const uint16_t* __restrict__ W, int64_t s, int64_t o,
                                                      float* __restrict__ C_O) {
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int64_t n_to = o / 16;
    const int64_t tile = static_cast<int64_t>(blockIdx.x) * 4 + wid;
    const int64_t n_ts = (s + 15) / 16;
    if (tile >= n_to * n_ts) return;
    const int64_t to_i = tile % n_to, ts_i = tile / n_to;
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t srow = ts_i * 16 + r16;
    v4f f = {0.f, 0.f, 0.f, 0.f};
    f = outlier_tile_16x16(f, lane, to_i * 16, ts_i * 16, s, o, X_O, ldo, idx, n_out[0], W, nullptr, nullptr, nullptr);
    const int64_t ocol = to_i * 16 + 4 * g;
    if (srow < s) *reinterpret_cast<v4f*>(C_O + srow * o + ocol) = f;
}

// Weight tiles per group of the grouped tile order (grouped_tile): 4 when
// the weight operand (hb reduction bytes per column) exceeds the Infinity
// Cache, else 8. Interleaved A/B of the product kernel, groups 4 / 5 / 8
// in us: 4096 x 12288 x 36864 (453 MB of weights) 1464-1468 / 1468-1471 /
// 1500-1506; 4096 x 8192 x 28672 (235 MB) 778-785 / 777-778 / 770-773;
// 2048 x 4096 x 16384 flat within 1 %. (Before the weights-first load
// order, 5 was 0.8-1.3 % faster than 4 on the first layer; now they tie,
// and 4 fetches less: the weights twice and Xq 36 times per launch.)
// Compute units of the current device (read once per device).
int cu_count() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

constexpr int64_t kMallBytes = int64_t(256) << 20;
uint32_t tile_group(int64_t hb, int64_t o) { return hb * o > kMallBytes ? 4u : 8u; }

template <GemmOut MODE>
hipError_t launch_mode(const int8_t* Xq, const float* c_x, const uint16_t* X_O, int64_t ldo,
                       const int32_t* idx, const int32_t* n_out, const int8_t* Wq, const float* c_w,
                       const uint16_t* W, const uint16_t* bias, int64_t s, int64_t h, int64_t o, void* C,
                       hipStream_t stream, uint32_t* clear, int clear_words, ZpArgs zp) {
    // Weight streaming. The K-split kernel: 64 output columns per block (one
    // 16-column tile per wavefront in the epilogue), batches of two K steps:
    // 7.06 TB/s of weights on the 8 x 12288 x 49152 layer against 6.64 TB/s
    // with 32 columns and batches of four. Up to 128 rows otherwise: the
    // column-split kernel with X in LDS (k_gemm_skinny), 1, 2, 3, 4, 6 or 8
    // row groups of 16; on that layer (forward) 96-103 us for 17-64 rows
    // and 107-136 us for 65-128, where the tiled product takes 155-165 us.
    // Up to 16 rows the K-split kernel keeps narrow layers (fewer than four
    // 16-column tiles per CU: its K split keeps more loads in flight) and
    // layers whose 64-column blocks fill the CUs evenly three at a time;
    // other layers take the column-split kernel, which places one block on
    // each CU (forward, 1-16 rows, 12288-deep layers: 76.6-78.5 us against
    // 85.2-94.3 on 36864 columns, 60.8-61.6 against 62.3-68.5 on 28672,
    // 37.5-39.9 against 40.7-41.5 on 16384; equal on 49152).
    const int cus = cu_count();
    if (s <= 16 && (o / 16 < 4 * cus || (o / 64) % (3 * cus) == 0)) {
        hipLaunchKernelGGL((k_gemm_decode<MODE, 4, 2, 4>), dim3(static_cast<unsigned>(o / 64)), dim3(256), 0, stream,
                           Xq, Wq, s, h, o, c_x, c_w, X_O, ldo, idx, n_out, W, bias, C, clear, clear_words, zp);
    } else if (s <= 128) {
        // one block per CU where the 16-column tiles allow: the fewest
        // wavefronts per block (4, 8, 12 or 16) whose blocks fit the CUs
        const int64_t tiles = o / 16;
        const int64_t per_cu = (tiles + cus - 1) / cus;
        const int waves = per_cu <= 4 ? 4 : per_cu <= 8 ? 8 : per_cu <= 12 ? 12 : 16;
        const dim3 grid(static_cast<unsigned>((tiles + waves - 1) / waves)), block(static_cast<unsigned>(64 * waves));
#define I8MM_SKINNY(RG, WV)                                                                                        \
    hipLaunchKernelGGL((k_gemm_skinny<MODE, 1, RG, WV>), grid, block, 0, stream, Xq, Wq, s, h, o, c_x, c_w, X_O, ldo, \
                       idx, n_out, W, bias, C, clear, clear_words, zp)
#define I8MM_SKINNY_RG(WV)          \
    if (s <= 16) {                  \
        I8MM_SKINNY(1, WV);         \
    } else if (s <= 32) {           \
        I8MM_SKINNY(2, WV);         \
    } else if (s <= 48) {           \
        I8MM_SKINNY(3, WV);         \
    } else if (s <= 64) {           \
        I8MM_SKINNY(4, WV);         \
    } else if (s <= 96) {           \
        I8MM_SKINNY(6, WV);         \
    } else {                        \
        I8MM_SKINNY(8, WV);         \
    }
        if (waves == 4) {
            I8MM_SKINNY_RG(4)
        } else if (waves == 8) {
            I8MM_SKINNY_RG(8)
        } else if (waves == 12) {
            I8MM_SKINNY_RG(12)
        } else {
            I8MM_SKINNY_RG(16)
        }
#undef I8MM_SKINNY_RG
#undef I8MM_SKINNY
    } else {
        const int64_t tiles = ((s + kTS - 1) / kTS) * ((o + kTO - 1) / kTO);
        hipLaunchKernelGGL((k_gemm_prefill<MODE>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream,
                           Xq, Wq, s, h, o, c_x, c_w, X_O, ldo, idx, n_out, W, bias, C, clear, clear_words, zp,
                           tile_group(h, o), nullptr, nullptr);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_int8_gemm(GemmOut mode, const int8_t* Xq, const float* c_x,
                            const uint16_t* X_O, int64_t ldo,
                            const int32_t* idx, const int32_t* n_out,
                            const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                            int64_t s, int64_t h, int64_t o, void* C, hipStream_t stream,
                            uint32_t* clear, int clear_words, ZpArgs zp) {
    if (mode == GemmOut::Int32)
        return launch_mode<GemmOut::Int32>(Xq, c_x, X_O, ldo, idx, n_out, Wq, c_w, W, nullptr, s, h, o, C, stream,
                                           clear, clear_words, ZpArgs{});
    if (mode == GemmOut::ZeroPoint)
        return launch_mode<GemmOut::ZeroPoint>(Xq, c_x, X_O, ldo, idx, n_out, Wq, c_w, W, bias, s, h, o, C,
                                               stream, clear, clear_words, zp);
    return launch_mode<GemmOut::Mixed>(Xq, c_x, X_O, ldo, idx, n_out, Wq, c_w, W, bias, s, h, o, C, stream,
                                       clear, clear_words, ZpArgs{});
}

hipError_t launch_fp16_gemm(const uint16_t* X, const uint16_t* Wp, int64_t s, int64_t h, int64_t o, uint16_t* C,
                            hipStream_t stream) {
    // Rows of X and the 64-byte panels of Wp hold 2 h reduction bytes.
    const int64_t tiles = ((s + kTS - 1) / kTS) * ((o + kTO - 1) / kTO);
    hipLaunchKernelGGL((k_gemm_prefill<GemmOut::Fp16Dense>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream,
                       reinterpret_cast<const int8_t*>(X), reinterpret_cast<const int8_t*>(Wp), s, 2 * h, o,
                       nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr, C, nullptr, 0, ZpArgs{},
                       tile_group(2 * h, o), nullptr, nullptr);
    return hipGetLastError();
}

hipError_t launch_int8_gemm_inline_quant(const uint16_t* X, const uint32_t* mask, const float* c_x,
                                         const uint16_t* X_O, int64_t ldo, const int32_t* idx, const int32_t* n_out,
                                         const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                         int64_t s, int64_t h, int64_t o, uint16_t* C, hipStream_t stream,
                                         uint32_t* clear, int clear_words) {
    const int64_t tiles = ((s + kTS - 1) / kTS) * ((o + kTO - 1) / kTO);
    hipLaunchKernelGGL((k_gemm_prefill<GemmOut::Mixed, true>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0,
                       stream, nullptr, Wq, s, h, o, c_x, c_w, X_O, ldo, idx, n_out, W, bias, C, clear, clear_words,
                       ZpArgs{}, tile_group(h, o), X, mask);
    return hipGetLastError();
}

hipError_t launch_decode_fused(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha, const int8_t* Wq,
                               const float* c_w, const uint16_t* W, const uint16_t* bias, uint16_t* C, uint32_t* mask,
                               int32_t* idx, int32_t* n_out, int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo,
                               hipStream_t stream) {
    constexpr int NT = 4;
    const size_t dyn = static_cast<size_t>(8 * (h / 32));
    hipLaunchKernelGGL((k_decode_fused<NT>), dim3(static_cast<unsigned>(o / (16 * NT))), dim3(256), dyn, stream, X,
                       static_cast<int>(s), h, o, make_threshold(alpha), Wq, c_w, W, bias, C, mask, idx, n_out, Xq,
                       c_x, X_O, ldo);
    return hipGetLastError();
}

hipError_t launch_outlier_matmul(const uint16_t* X_O, int64_t ldo, const int32_t* idx, const int32_t* n_out,
                                 const uint16_t* W, int64_t s, int64_t o, float* C_O, hipStream_t stream) {
    const int64_t tiles = (o / 16) * ((s + 15) / 16);
    hipLaunchKernelGGL(k_outlier_only, dim3(static_cast<unsigned>((tiles + 3) / 4)), dim3(256), 0, stream,
                       X_O, ldo, idx, n_out, W, s, o, C_O);
    return hipGetLastError();
}

}  // namespace i8mm
