// Host-side launchers of the gfx950 kernels. Arguments are validated by the
// C-ABI layer (api.cpp) before any of these is called; each launcher only
// picks a grid and enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

hipError_t launch_detect(const uint16_t* X, int64_t s, int64_t h, float alpha,
                         uint32_t* mask, int32_t* idx, int32_t* n_out, hipStream_t stream);

// p[0 .. n) = v (one small kernel; also clears state inside captured graphs,
// where a memset node is avoided).
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t stream);

hipError_t launch_quantize_rows(const uint16_t* X, int64_t s, int64_t h,
                                const uint32_t* mask, const int32_t* idx, const int32_t* n_out,
                                int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo,
                                hipStream_t stream);

// Forward path: detection + index list + row quantisation in two launches,
// or in one for at most 8 rows and at most 24 KiB of X (no cross-block
// state; *clear_words is then 0). Cross-block state (the mask accumulator,
// or the row maxima for other inputs of at most 8 rows) goes to `acc`,
// which must be zero on entry;
// *clear_words is how many of its words the product launch must clear
// again (see launch_int8_gemm). For s > 8, Xq may be null: the codes are
// then not written (launch_int8_gemm_inline_quant makes them).
hipError_t launch_forward_prologue(const uint16_t* X, int64_t s, int64_t h, float alpha, uint32_t* acc,
                                   uint32_t* mask, int32_t* idx, int32_t* n_out, int8_t* Xq, float* c_x,
                                   uint16_t* X_O, int64_t ldo, hipStream_t stream, int* clear_words);

// The same for the tensor-wise (zeropoint = false; c_x receives the one
// constant in every entry) or zeropoint (c_x receives nd_x; zp_x and
// rowsum_x are written) row quantiser: detection into acc[0 .. h / 32),
// then the scheme's row quantiser, whose first block writes the mask, the
// index list and |O|.
hipError_t launch_forward_prologue_variant(bool zeropoint, const uint16_t* X, int64_t s, int64_t h, float alpha,
                                           uint32_t* acc, uint32_t* mask, int32_t* idx, int32_t* n_out, int8_t* Xq,
                                           float* c_x, int32_t* zp_x, int32_t* rowsum_x, uint16_t* X_O, int64_t ldo,
                                           hipStream_t stream, int* clear_words);

hipError_t launch_quantize_cols(const uint16_t* W, int64_t h, int64_t o,
                                int8_t* Wq, float* c_w, hipStream_t stream);

// Tensor-wise absmax: one constant for all of X's non-outlier part (written
// to every c_x[i]) or for all of W (every c_w[j]); same outputs otherwise.
// If idx is non-null, the first pass also writes the index list and |O|
// (and the mask to mask_out if that is non-null) from `mask`.
hipError_t launch_quantize_tensorwise(const uint16_t* X, int64_t s, int64_t h, const uint32_t* mask, int8_t* Xq,
                                      float* c_x, uint16_t* X_O, int64_t ldo, hipStream_t stream,
                                      uint32_t* mask_out = nullptr, int32_t* idx = nullptr,
                                      int32_t* n_out = nullptr);
hipError_t launch_quantize_weights_tensorwise(const uint16_t* W, int64_t h, int64_t o, int8_t* Wq, float* c_w,
                                              hipStream_t stream);

// Zeropoint quantisation: rows of X over the non-outlier columns (codes,
// nd_x, zp_x, code sums over the row, X_O gather) and columns of W at load
// time (panel codes, nd_w, zp_w, code sums over the column).
// (idx, n_out, mask_out: as for launch_quantize_tensorwise.)
hipError_t launch_quantize_rows_zp(const uint16_t* X, int64_t s, int64_t h, const uint32_t* mask, int8_t* Xq,
                                   float* nd_x, int32_t* zp_x, int32_t* rowsum_x, uint16_t* X_O, int64_t ldo,
                                   hipStream_t stream, uint32_t* mask_out = nullptr, int32_t* idx = nullptr,
                                   int32_t* n_out = nullptr);
hipError_t launch_quantize_cols_zp(const uint16_t* W, int64_t h, int64_t o, int8_t* Wq, float* nd_w, int32_t* zp_w,
                                   int32_t* colsum_w, hipStream_t stream);

// mode: product variant of the shared int8 main loop. W (Mixed only) may be
// null: outlier rows rebuilt from Wq / c_w. bias (Mixed only, optional):
// fp16 [o] added before the rounding. `clear` (optional): clear_words
// uint32 words that the first block zeroes (the forward path's
// accumulator, whose readers have finished by then).
// ZeroPoint: the product of zeropoint codes, C' = sum over k not in O of
// (Xq_ik + zp_x_i)(Wq_kj + zp_w_j), dequantised with 1 / (nd_x nd_w) (passed
// as c_x, c_w) plus the fp16 outlier product; ZpArgs carries the zero points
// and code sums (rowsum over the row's codes, colsum over all h codes of the
// column).
enum class GemmOut { Mixed = 0, Int32 = 1, Fp16Dense = 2, ZeroPoint = 3 };

struct ZpArgs {
    const int32_t* zp_x;
    const int32_t* rowsum_x;
    const int32_t* zp_w;
    const int32_t* colsum_w;
};

hipError_t launch_int8_gemm(GemmOut mode, const int8_t* Xq, const float* c_x,
                            const uint16_t* X_O, int64_t ldo,
                            const int32_t* idx, const int32_t* n_out,
                            const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                            int64_t s, int64_t h, int64_t o, void* C, hipStream_t stream,
                            uint32_t* clear = nullptr, int clear_words = 0, ZpArgs zp = ZpArgs{});

// Dense fp16 product C = fp16(X W) with fp32 accumulation; Wp is W in the
// fp16 panel layout [h / 32][o][32] (see launch_pack_fp16_panels).
hipError_t launch_fp16_gemm(const uint16_t* X, const uint16_t* Wp, int64_t s, int64_t h, int64_t o, uint16_t* C,
                            hipStream_t stream);

// The LLM.int8() product with the int8 operand of X made inside the
// product kernel from the fp16 rows X, the final outlier mask and c_x
// (k_gemm_prefill<Mixed, QX>): no Xq. Any s (the tiled product); the other
// arguments as launch_int8_gemm's.
hipError_t launch_int8_gemm_inline_quant(const uint16_t* X, const uint32_t* mask, const float* c_x,
                                         const uint16_t* X_O, int64_t ldo, const int32_t* idx, const int32_t* n_out,
                                         const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                         int64_t s, int64_t h, int64_t o, uint16_t* C, hipStream_t stream,
                                         uint32_t* clear, int clear_words);

hipError_t launch_pack_fp16_panels(const uint16_t* W, int64_t h, int64_t o, uint16_t* Wp, hipStream_t stream);

// The whole forward in one launch for s <= 16 (k_decode_fused); the
// intermediates go to mask .. X_O (block 0 writes them).
hipError_t launch_decode_fused(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha, const int8_t* Wq,
                               const float* c_w, const uint16_t* W, const uint16_t* bias, uint16_t* C, uint32_t* mask,
                               int32_t* idx, int32_t* n_out, int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo,
                               hipStream_t stream);

hipError_t launch_outlier_matmul(const uint16_t* X_O, int64_t ldo,
                                 const int32_t* idx, const int32_t* n_out,
                                 const uint16_t* W, int64_t s, int64_t o,
                                 float* C_O, hipStream_t stream);

// Calibration stream of int8 MFMAs (k_calib_mfma_i8): `blocks` blocks of
// four wavefronts, 32 iters MFMAs per wavefront; codes holds 256 bytes per
// thread, out one int32 per thread.
hipError_t launch_calib_mfma_i8(const int8_t* codes, int64_t blocks, int64_t iters, int32_t* out,
                                hipStream_t stream);

}  // namespace i8mm
