/*
 * i8mm.h - C ABI of the LLM.int8() mixed-precision decomposed int8 matmul
 *          for AMD Instinct MI355X (gfx950).
 *
 * The library computes, for a transformer linear layer C = X W with
 * X fp16 [s, h] and W fp16 [h, o]:
 *   1. the outlier feature columns O = { j : max_i |X_ij| >= alpha };
 *   2. row-wise absmax int8 quantisation of X over the columns not in O;
 *   3. (once, at load time) column-wise absmax int8 quantisation of W;
 *   4. C = fp16( C_i32 / (c_x (x) c_w) + X[:, O] W[O, :] [+ bias] ), where
 *      C_i32 is the exact int8 x int8 -> int32 product over the columns not
 *      in O.
 *
 * Page tags used in the citations below:
 *   [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for Transformers at
 *            Scale" (paper-graph-ui.vercel.app digest of arXiv 2208.07339)
 *   [TM]     transformer-math LLM.int8() tutorial (aicassindra.com)
 *   [PY]     "LLM.int8() 完全拆解：系统离群值的涌现与混合精度分解"
 *            (pinghaoyang.com.cn)
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     owned by the caller; the library never frees or retains them.
 *   - fp16 values are passed as their IEEE binary16 bit patterns (uint16_t).
 *   - All matrices are row-major and dense (leading dimension = row length),
 *     except X_O, whose row stride is the explicit argument ldo.
 *   - Every pointer must be 16-byte aligned.
 *   - Shape limits: s >= 1; h and o multiples of 64; h <= 133120 (so an
 *     int32 accumulator cannot overflow: h * 127^2 < 2^31); for the
 *     products (i8mm_int8_mixed_matmul, i8mm_int8_gemm_i32, i8mm_forward)
 *     also h * o < 2^31 (Wq and W are addressed with 32-bit byte offsets).
 *   - Quantised weights use the PANEL layout Wq [h / 64][o][64]: the code
 *     W_i8[k, j] is the byte at offset (k / 64) * o * 64 + j * 64 + k % 64.
 *     Panel p holds rows 64 p .. 64 p + 63 of W_i8 with each column's 64
 *     codes contiguous, so 16 columns of one panel (the A operand of one
 *     int8 matrix-core instruction) are one contiguous KiB.
 *   - Work is enqueued on `stream` (NULL = the default stream); calls return
 *     without synchronising. Arguments are validated on the host before any
 *     work is enqueued: an invalid call enqueues nothing. Faults of the
 *     device work itself surface at the caller's next synchronisation.
 *   - The library allocates no device memory and holds no per-call state;
 *     concurrent calls on different streams are safe if their output buffers
 *     do not overlap.
 *   - Scales are fp32: c = fl32(127 / m) (IEEE division, round to nearest
 *     even), c = 1 when m == 0. Quantisation is v = fl32(x * c) rounded half
 *     away from zero, in [-127, 127].
 *   - X may hold +-inf (always an outlier: |x| >= alpha for every accepted
 *     alpha). A NaN element never makes its column an outlier, and it does
 *     not hide an element of the same column that reaches alpha (the test is
 *     element by element); a NaN among a row's non-outlier values leaves
 *     that row's scale and codes unspecified.
 *
 * Where this interface departs from the plain signatures one would write
 * from the pages' five steps (W_i8 as a [o, h] matrix, one workspace-size
 * query, no bias), and why:
 *   - Wq is in the panel layout below, not a plain [o, h] matrix: the decode
 *     product streams 16-column panel tiles as contiguous KiB runs (a probe
 *     of the same loop went from 4.6 to 7.0 TB/s of weights). It is written
 *     once by the load-time conversion, so it costs nothing per forward.
 *   - The workspace queries are i8mm_forward_workspace_bytes (plus the
 *     _layout query that returns the offsets of the intermediates, and a
 *     zeropoint variant), named for the call they serve.
 *   - i8mm_int8_mixed_matmul and the one-call forwards take an optional
 *     fp16 layer bias (NULL for none) added before the single rounding, and
 *     accept W = NULL (no resident fp16 weights, outlier rows rebuilt).
 *   - The products require h * o < 2^31: Wq (h o bytes) and W (2 h o bytes)
 *     are read through 32-bit buffer offsets; larger layers are rejected
 *     with I8MM_EINVAL.
 *   - i8mm_quantize_rowwise derives O from the mask alone; idx and n_out are
 *     validated but not read.
 *   - Extra entry points beyond the four steps: the one-call forwards, the
 *     int32 and outlier-only products (inspection), the dense fp16 baseline
 *     and the quantiser variants of Table 1.
 */
#ifndef I8MM_H
#define I8MM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    I8MM_OK = 0,
    I8MM_EINVAL = -1,   /* bad pointer, shape, alignment or argument value */
    I8MM_EDEVICE = -2,  /* no HIP device, or the current device is not gfx950 */
    I8MM_ELAUNCH = -3,  /* a kernel launch was rejected by the runtime */
    I8MM_EWORKSPACE = -4, /* a one-call forward's launch failed after its detection had
                             written the workspace accumulator, and the launch that
                             clears it failed too: zero the accumulator before reuse */
    I8MM_ESCRATCH = -5    /* i8mm_forward_noalloc: the shape needs more workspace than
                             I8MM_NOALLOC_SCRATCH_BYTES */
} i8mm_status;

/* Largest h accepted (int32 accumulator bound, rounded down to 64). */
#define I8MM_MAX_H 133120

/*
 * Load-time weight conversion: W fp16 [h, o] -> Wq int8 (panel layout) and c_w fp32 [o].
 *
 * [DIGEST] "The Full LLM.int8() Algorithm", Step 4, second and third
 * bullets (c_w_j = 127 / max_i |W_ij|, W_i8 = round(W (.) c_w)), and "Why
 * vector-wise rather than row-wise" (the column constants are computed once
 * at load time); [PY] "第一件武器：向量级量化" (one scale per column of W).
 * The max runs over all h rows of W, so the conversion does not depend on
 * the per-forward outlier set.
 *
 * W: [h, o] fp16 (read). Wq: h * o bytes (written), W_i8 in the panel
 * layout described above. c_w: [o] fp32 (written).
 */
i8mm_status i8mm_quantize_colwise_weights(const uint16_t* W, int64_t h, int64_t o,
                                          int8_t* Wq, float* c_w, hipStream_t stream);

/*
 * Outlier-column detection: O = { j in [0, h) : max_i |X_ij| >= alpha }.
 *
 * [DIGEST] "The Full LLM.int8() Algorithm", Step 1; [DIGEST]
 * "Mixed-Precision Decomposition", formal definition of O and "The outlier
 * detection threshold" (alpha = 6.0); [PY] "第二件武器：混合精度分解".
 * The comparison is done in fp32 on the exactly widened fp16 value.
 *
 * X: [s, h] fp16 (read).
 * mask: [ceil(h/32)] uint32 (written): bit (j % 32) of word j / 32 is set iff j in O.
 * idx: [h] int32 (written): the members of O in ascending order in idx[0 .. |O|);
 *      entries from |O| on are unspecified.
 * n_out: [1] int32 (written): |O|. Stays on the device (no host round trip).
 * alpha: finite or +inf, >= 0 (alpha = +inf gives O = {}, pure vector-wise
 *        int8; alpha = 0 puts every column in O).
 */
i8mm_status i8mm_detect_outlier_cols(const uint16_t* X, int64_t s, int64_t h, float alpha,
                                     uint32_t* mask, int32_t* idx, int32_t* n_out,
                                     hipStream_t stream);

/*
 * Row-wise absmax quantisation of the non-outlier columns, plus the gather
 * of the outlier columns.
 *
 * [DIGEST] "The Full LLM.int8() Algorithm", Step 2 (split X into X^O and
 * X^{not O}) and Step 4, first and third bullets (c_x_i = 127 / max over the
 * non-outlier columns of row i; X_i8 = round(c_x (.) X^{not O}));
 * [TM] "Absmax INT8 quantization from first principles" and "Vector-wise:
 * a scale per row and per column".
 *
 * X: [s, h] fp16 (read). mask: as written by i8mm_detect_outlier_cols (read
 * on the device); it alone defines O: the column of rank k in O (its k-th
 * member in ascending order) goes to X_O[:, k]. idx and n_out must be the
 * matching outputs of the same detection call; they are validated like the
 * other pointers but not read.
 * Xq: [s, h] int8 (written): quantised X with the columns in O set to 0.
 * c_x: [s] fp32 (written).
 * X_O: [s, ldo] fp16 (written): X_O[i, k] = X[i, idx[k]] for k < |O|, and 0
 *      for |O| <= k < round_up(|O|, 32); later entries are not touched.
 * ldo: row stride of X_O in elements; must be >= round_up(h, 32) (|O| is
 *      only known on the device, so room for |O| = h is required) and a
 *      multiple of 8.
 */
i8mm_status i8mm_quantize_rowwise(const uint16_t* X, int64_t s, int64_t h,
                                  const uint32_t* mask, const int32_t* idx, const int32_t* n_out,
                                  int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo,
                                  hipStream_t stream);

/*
 * The decomposed product: C = fp16( C_i32 / (c_x (x) c_w) + X_O W[idx, :] ).
 *
 * [DIGEST] "Mixed-Precision Decomposition", formal definition (sum of the
 * fp16 outlier outer products and S times the int8 product); [DIGEST] "The
 * Full LLM.int8() Algorithm", Steps 3-5; [PY] "第二件武器：混合精度分解"
 * (decomposition equation); [TM] "The mixed-precision decomposition".
 *
 * C_i32 = Xq W_i8 is exact (int8 MFMA, int32 accumulate). The dequantised
 * value and the fp16 outlier product (fp16 MFMA, fp32 accumulate) are summed
 * in fp32 and rounded once to fp16 (round to nearest even). S is never
 * materialised. n_out is read on the device; only rows idx[0 .. n_out) of W
 * are read.
 * With a layer bias b the result is C = fp16( C_i32 / (c_x (x) c_w) +
 * X_O W[idx, :] + b ), b added in the same fp32 sum before the one rounding
 * (biases stay in 16 bit: [DIGEST] "Mixed-Precision Decomposition", memory
 * accounting).
 *
 * Xq: [s, h] int8; c_x: [s] fp32; X_O: [s, ldo] fp16 (ldo as above);
 * idx, n_out: as from i8mm_detect_outlier_cols; Wq: panel layout (above);
 * c_w: [o] fp32; C: [s, o] fp16 (written).
 * W: [h, o] fp16, the original weights, or NULL when no fp16 copy of W is
 * kept: the outlier rows are then rebuilt from the int8 codes by multiplying
 * back with the inverse scale, W[k, j] = fl16(fl32(W_i8[k, j] * fl32(1 / c_w[j])))
 * (IEEE round to nearest even at each step; [PY] "量化为什么会崩：一个尺度统治全局":
 * dequantisation multiplies by 1/s), so
 * only Wq and c_w stay resident: about half the weight memory, the saving
 * the pages measure on BLOOM-176B ([DIGEST] "Executive Summary"; [PY]
 * "第二件武器：混合精度分解"); the outlier product then sees the 8-bit weights.
 * bias: [o] fp16 (read), or NULL for none.
 */
i8mm_status i8mm_int8_mixed_matmul(const int8_t* Xq, const float* c_x,
                                   const uint16_t* X_O, int64_t ldo,
                                   const int32_t* idx, const int32_t* n_out,
                                   const int8_t* Wq, const float* c_w, const uint16_t* W,
                                   const uint16_t* bias,
                                   int64_t s, int64_t h, int64_t o, uint16_t* C,
                                   hipStream_t stream);

/*
 * The 16-bit outlier product alone: C_O fp32 [s, o] = X_O W[idx, :].
 *
 * [DIGEST] "The Full LLM.int8() Algorithm", Step 3 (C^O = X^O_f16 W^O_f16);
 * [PY] "第二件武器：混合精度分解" (an s x |O| by |O| x o skinny product).
 * fp16 MFMA with fp32 accumulation; the same device routine that the fused
 * epilogue of i8mm_int8_mixed_matmul uses. Arguments as above.
 */
i8mm_status i8mm_outlier_matmul(const uint16_t* X_O, int64_t ldo,
                                const int32_t* idx, const int32_t* n_out,
                                const uint16_t* W, int64_t s, int64_t h, int64_t o,
                                float* C_O, hipStream_t stream);

/*
 * The int8 product alone: C_i32 int32 [s, o] = Xq W_i8, exact (Wq in the
 * panel layout).
 *
 * [DIGEST] "The Full LLM.int8() Algorithm", Step 4, fourth bullet (Int8
 * matrix multiplication producing an Int32 accumulator). Runs the same
 * main loop as i8mm_int8_mixed_matmul with a plain int32 store.
 */
i8mm_status i8mm_int8_gemm_i32(const int8_t* Xq, const int8_t* Wq,
                               int64_t s, int64_t h, int64_t o, int32_t* C_i32,
                               hipStream_t stream);

/*
 * Dense fp16 baseline, load-time packing: W fp16 [h, o] -> Wp fp16 in the
 * fp16 panel layout [h / 32][o][32] (W[k, j] is element
 * (k / 32) * o * 32 + j * 32 + k % 32 of Wp; 2 * h * o bytes).
 *
 * [DIGEST] "Runtime Performance (Appendix D)": Table 5 reports every variant
 * as a speed-up over the FP16 matrix multiply of the same layer; this and
 * i8mm_fp16_gemm provide that baseline with the library's own kernels.
 * Shape limits as above, plus 2 * h * o < 2^31.
 */
i8mm_status i8mm_pack_fp16_weights(const uint16_t* W, int64_t h, int64_t o, uint16_t* Wp, hipStream_t stream);

/*
 * Dense fp16 product C = fp16(X W), fp16 MFMA with fp32 accumulation, one
 * round-to-nearest-even rounding per output ([DIGEST] "Runtime Performance
 * (Appendix D)", the FP16 baseline of Table 5). The same main loop as the
 * int8 product, run on 2-byte elements.
 * X: [s, h] fp16; Wp: from i8mm_pack_fp16_weights; C: [s, o] fp16 (written).
 */
i8mm_status i8mm_fp16_gemm(const uint16_t* X, const uint16_t* Wp, int64_t s, int64_t h, int64_t o, uint16_t* C,
                           hipStream_t stream);

/*
 * Quantiser variants of Table 1 ([DIGEST] "Quantization Primitives: Absmax
 * and Zeropoint Quantization" and "Vector-wise Quantization": tensor-wise
 * absmax, row-wise absmax with one tensor-wide constant for W, and zeropoint
 * vector-wise; each with the mixed-precision decomposition, or without it
 * when alpha = +inf). The absmax variants reuse i8mm_int8_mixed_matmul: a
 * tensor-wise constant is written to every entry of c_x (or c_w), so the
 * product's 1 / (c_x (x) c_w) applies it unchanged.
 */

/*
 * Tensor-wise absmax for X: c = fl32(127 / m), m the largest |X_ij| over all
 * rows and the columns not in O (c = 1 when m == 0). Arguments and outputs
 * as for i8mm_quantize_rowwise; c_x[i] = c for every row.
 */
i8mm_status i8mm_quantize_tensorwise(const uint16_t* X, int64_t s, int64_t h,
                                     const uint32_t* mask, const int32_t* idx, const int32_t* n_out,
                                     int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo,
                                     hipStream_t stream);

/*
 * Tensor-wise absmax for W (load time; used by tensor-wise and row-wise
 * quantisation): one constant c = fl32(127 / max_ij |W_ij|). Arguments and
 * outputs as for i8mm_quantize_colwise_weights; c_w[j] = c for every column.
 */
i8mm_status i8mm_quantize_weights_tensorwise(const uint16_t* W, int64_t h, int64_t o,
                                             int8_t* Wq, float* c_w, hipStream_t stream);

/*
 * Zeropoint quantisation of each row of X over the columns not in O
 * ([DIGEST] "Quantization Primitives", zeropoint: nd = 2 * 127 / (max - min)
 * and a zero point; [PY] "量化为什么会崩：一个尺度统治全局"). With min and max over the
 * row's non-outlier values:
 *   nd = fl32(254 / fl32(max - min))   (1 when max == min),
 *   zp = round(fl32(nd * min)) + 127   (the pages print the zero point as a
 *        garbled product of X and min; this reading makes the codes fill
 *        [-127, 127] with q + zp ~ nd * x),
 *   q  = clamp(round(fl32(nd * x)) - zp, -127, 127), rounding half away.
 * X, mask, idx, n_out, Xq (0 in the columns in O), X_O and ldo as for
 * i8mm_quantize_rowwise. nd_x: [s] fp32, zp_x: [s] int32 (the zero point
 * can leave int16 for one-signed rows), rowsum_x: [s] int32, the sum of the
 * row's codes (all written).
 */
i8mm_status i8mm_quantize_rowwise_zeropoint(const uint16_t* X, int64_t s, int64_t h,
                                            const uint32_t* mask, const int32_t* idx, const int32_t* n_out,
                                            int8_t* Xq, float* nd_x, int32_t* zp_x, int32_t* rowsum_x,
                                            uint16_t* X_O, int64_t ldo, hipStream_t stream);

/*
 * Zeropoint quantisation of each column of W over all h rows (load time),
 * as above. Wq: panel layout (above); nd_w: [o] fp32; zp_w: [o] int32;
 * colsum_w: [o] int32, the sum of the column's h codes (all written).
 */
i8mm_status i8mm_quantize_colwise_weights_zeropoint(const uint16_t* W, int64_t h, int64_t o,
                                                    int8_t* Wq, float* nd_w, int32_t* zp_w, int32_t* colsum_w,
                                                    hipStream_t stream);

/*
 * The zeropoint vector-wise product with the decomposition ([DIGEST]
 * "Quantization Primitives": the product of two zeropoint-quantised
 * matrices expands into the int8 product and three correction terms;
 * [PY] the same four-term expansion):
 *   C' = sum over k not in O of (Xq_ik + zp_x_i)(Wq_kj + zp_w_j)
 *      = C_i32 + zp_w_j (rowsum_x_i + (h - |O|) zp_x_i) + zp_x_i colsum'_j,
 *   C  = fp16( C' / (nd_x_i nd_w_j) + X_O W[idx, :] [+ bias] ),
 * where C_i32 = Xq W_i8 (the int8 MFMA main loop of the absmax product) and
 * colsum'_j = colsum_w_j minus the codes of column j in the outlier rows
 * (read on the device). The correction is exact for zero points below 2^17
 * in magnitude (sums in fp64 or int64); beyond, it is rounded in fp64.
 * Arguments as for i8mm_int8_mixed_matmul, with nd_x / nd_w in place of
 * c_x / c_w and the zero points and code sums from the two calls above;
 * W (the fp16 weights, for the outlier rows) must not be NULL; bias may be.
 */
i8mm_status i8mm_zeropoint_matmul(const int8_t* Xq, const float* nd_x, const int32_t* zp_x,
                                  const int32_t* rowsum_x, const uint16_t* X_O, int64_t ldo,
                                  const int32_t* idx, const int32_t* n_out,
                                  const int8_t* Wq, const float* nd_w, const int32_t* zp_w,
                                  const int32_t* colsum_w, const uint16_t* W, const uint16_t* bias,
                                  int64_t s, int64_t h, int64_t o, uint16_t* C, hipStream_t stream);

/* Bytes at the start of the forward workspace that hold the cross-block
 * accumulator of the detection (the outlier mask being ORed together, or,
 * for inputs of at most 8 rows and more than 24 KiB, the per-row maxima;
 * smaller inputs of at most 8 rows leave it untouched). */
#define I8MM_FORWARD_ACC_BYTES 16640

/*
 * Bytes of device workspace that i8mm_forward needs for (s, h): the mask
 * accumulator, mask, idx, n_out, Xq, c_x and X_O (ldo = round_up(h, 32)),
 * each 256-byte aligned. Returns 0 for invalid shapes.
 */
size_t i8mm_forward_workspace_bytes(int64_t s, int64_t h);

/*
 * The whole per-forward path for one linear layer ([DIGEST] "The Full
 * LLM.int8() Algorithm", Steps 1-5): detect, quantise rows and gather,
 * decomposed product, in three kernel launches (two when s <= 8 and X
 * holds at most 24 KiB: detection and quantisation then share one).
 * Weights must already be converted by i8mm_quantize_colwise_weights.
 *
 * workspace: caller-owned device buffer of i8mm_forward_workspace_bytes(s, h)
 * bytes, 256-byte aligned. Its first I8MM_FORWARD_ACC_BYTES bytes (the
 * detection's accumulator) must be ZERO before the first call, e.g. by
 * allocating it zero-filled; every i8mm_forward returns them to zero, so a
 * workspace may be reused for any shape whose size fits. Calls that share a
 * workspace must not overlap. After completion the workspace holds the
 * intermediates at the offsets given by i8mm_forward_workspace_layout.
 * Errors: I8MM_EINVAL / I8MM_EDEVICE before anything is enqueued. If a
 * launch fails after the detection was enqueued, one more launch on the
 * same stream clears the accumulator and the call returns I8MM_ELAUNCH (C
 * is not written; the workspace stays valid); if that launch fails as well,
 * the call returns I8MM_EWORKSPACE and the caller must zero the
 * accumulator before the workspace is used again.
 * X: [s, h] fp16; Wq: panel layout (above); c_w: [o] fp32; W: [h, o] fp16
 * or NULL, and bias: [o] fp16 or NULL (both as for i8mm_int8_mixed_matmul);
 * C: [s, o] fp16 (written).
 */
i8mm_status i8mm_forward(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                         const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                         void* workspace, uint16_t* C, hipStream_t stream);

/*
 * The same one-call forward with tensor-wise absmax for X ([DIGEST]
 * "Quantization Primitives": one constant 127 / max |X| over the columns not
 * in O; Table 1's tensor-wise row): detection, then the maxima of the rows,
 * one constant over them and the codes with it, then the decomposed product,
 * in five kernel launches. Arguments, workspace (same size and layout as
 * i8mm_forward's; c_x holds the one constant in every entry) and errors as
 * for i8mm_forward. With c_w from i8mm_quantize_weights_tensorwise this is
 * Table 1's tensor-wise scheme; with column-wise c_w, tensor-wise X against
 * vector-wise W.
 */
i8mm_status i8mm_forward_tensorwise(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                    const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                    void* workspace, uint16_t* C, hipStream_t stream);

/*
 * Bytes of device workspace that i8mm_forward_zeropoint needs for (s, h):
 * i8mm_forward's workspace followed by zp_x [s] int32 and rowsum_x [s]
 * int32, each 256-byte aligned. Returns 0 for invalid shapes.
 */
size_t i8mm_forward_zeropoint_workspace_bytes(int64_t s, int64_t h);

/*
 * The one-call forward of the zeropoint vector-wise scheme with the
 * decomposition (Table 1's zeropoint rows; the product as for
 * i8mm_zeropoint_matmul): detection, zeropoint row quantisation and gather,
 * the zeropoint product, in three kernel launches. Weights from
 * i8mm_quantize_colwise_weights_zeropoint (Wq, nd_w, zp_w, colsum_w); W
 * (fp16, for the outlier rows) must not be NULL; bias may be. workspace:
 * i8mm_forward_zeropoint_workspace_bytes(s, h) bytes, 256-byte aligned, its
 * first I8MM_FORWARD_ACC_BYTES bytes zero before the first call and left
 * zero again (the same workspace may serve i8mm_forward and the other
 * one-call forwards). After completion it holds the intermediates at the
 * offsets of i8mm_forward_workspace_layout (nd_x in place of c_x), then
 * zp_x and rowsum_x. Errors as for i8mm_forward.
 */
i8mm_status i8mm_forward_zeropoint(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                   const int8_t* Wq, const float* nd_w, const int32_t* zp_w, const int32_t* colsum_w,
                                   const uint16_t* W, const uint16_t* bias, void* workspace, uint16_t* C,
                                   hipStream_t stream);

/*
 * Byte offsets inside the forward workspace, in the order accumulator, mask,
 * idx, n_out, Xq, c_x, X_O (7 entries written to offsets[]), and the X_O row
 * stride (elements) in *ldo. Returns I8MM_EINVAL for bad shapes or null
 * pointers. Host-only; touches no device.
 */
i8mm_status i8mm_forward_workspace_layout(int64_t s, int64_t h, size_t offsets[7], int64_t* ldo);

/* Largest row count of i8mm_forward_decode. */
#define I8MM_DECODE_MAX_ROWS 16

/*
 * The whole per-forward path of i8mm_forward in ONE kernel launch, for few
 * rows (1 <= s <= I8MM_DECODE_MAX_ROWS: token-by-token decoding). [DIGEST]
 * "The Full LLM.int8() Algorithm", Steps 1-5; the single launch removes
 * the per-layer detection and quantisation launches that [DIGEST]
 * "Runtime Overhead Makes LLM.int8() Slower Than 16-Bit for Models Below
 * ~13B Parameters" and [PY] "实验：无损扩展到 175B" name as the overhead
 * of the method. Every block derives the outlier set and the row constants
 * from all of X itself while its first weights are in flight, then streams
 * its weight columns with the int8 operand of X quantised on the fly; no
 * block waits for another. Results equal i8mm_forward's: the same codes,
 * constants and int32 products, and C from the same epilogue arithmetic.
 * Arguments as for i8mm_forward (W and bias may be NULL). The workspace
 * (i8mm_forward_workspace_bytes(s, h) bytes, 256-byte aligned) receives the
 * intermediates at the offsets of i8mm_forward_workspace_layout; its
 * accumulator is neither read nor written. s > I8MM_DECODE_MAX_ROWS gives
 * I8MM_EINVAL.
 */
i8mm_status i8mm_forward_decode(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                void* workspace, uint16_t* C, hipStream_t stream);

/* Smallest row count of i8mm_forward_inline_quant. */
#define I8MM_INLINE_QUANT_MIN_ROWS 129

/*
 * i8mm_forward with the row quantisation folded into the product: the
 * int8 codes of X are made inside the product kernel, from X, the outlier
 * mask and c_x, while it stages its operand tiles, and are never stored
 * (the fusion of [DIGEST] "The Full LLM.int8() Algorithm" Step 2 into
 * Step 4 that drops the Xq round trip; [DIGEST] "Runtime Overhead Makes
 * LLM.int8() Slower Than 16-Bit for Models Below ~13B Parameters" names
 * input quantisation as overhead). Two launches: detection, then the row
 * pass that writes c_x, X_O and the outlier set only; then the product.
 * Every row block of X is quantised once per column tile of the product
 * (o / 256 times) instead of once. Results equal i8mm_forward's bit for
 * bit (the same codes, made by the same rounding). Arguments, workspace
 * and errors as for i8mm_forward; the workspace's Xq region is not
 * written. s < I8MM_INLINE_QUANT_MIN_ROWS gives I8MM_EINVAL: with fewer
 * rows the forward's product is one of the weight-streaming kernels, not
 * the tiled one this variant changes.
 */
i8mm_status i8mm_forward_inline_quant(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                      const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                      void* workspace, uint16_t* C, hipStream_t stream);

/* Bytes of the static device scratch that i8mm_forward_noalloc uses as its
 * workspace (64 MiB per GPU the library runs on). */
#define I8MM_NOALLOC_SCRATCH_BYTES 67108864

/*
 * i8mm_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation. The call allocates nothing (no
 * hipMalloc, no allocating library routine); its workspace is a static
 * device array of I8MM_NOALLOC_SCRATCH_BYTES bytes that every GPU the
 * library runs on holds from module load until the process ends. Shapes
 * whose i8mm_forward_workspace_bytes(s, h) exceeds that return
 * I8MM_ESCRATCH before anything is enqueued (e.g. s * h up to about 21 M
 * elements fits: 2048 x 8192, or any few-row decode step). The array's
 * device address is looked up once per device on the first call, which
 * also enqueues one small launch that zeroes its accumulator.
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * intermediates; calls that overlap on one GPU (concurrent streams or
 * threads) race on it and must not be issued. Other arguments, the
 * computation, the launches and the errors are those of i8mm_forward.
 */
i8mm_status i8mm_forward_noalloc(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                 const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                 uint16_t* C, hipStream_t stream);

/*
 * Test hook: the next `count` one-call forwards (i8mm_forward and its
 * tensor-wise and zeropoint variants) report their product launch as
 * failed without launching it, so that tests can drive the error path
 * above from the host; count <= 0 turns it off. Not for production use.
 */
void i8mm_test_fail_product_launches(int count);

/*
 * Measurement calibration, not part of the method: the int8 matrix-core
 * rate the chip sustains under load, for the roofline of the products
 * (whose published int8 peak assumes the full 2.4 GHz clock). Enqueues one
 * launch of `blocks` blocks of four wavefronts; each wavefront issues
 * 32 * iters v_mfma_i32_32x32x32_i8 (65536 integer operations each) on
 * operands held in registers, with no memory traffic inside its loop, so the
 * launch performs blocks * 4 * 32 * iters * 65536 operations.
 *   codes  device, blocks * 65536 bytes: the int8 operands (random codes make
 *          the matrix cores switch as they do on real data); read once.
 *   out    device, blocks * 256 int32: an XOR of each thread's accumulators
 *          (keeps the work from being optimised away; no meaning otherwise).
 * Errors: I8MM_EINVAL for null or unaligned pointers, blocks outside
 * [1, 2^20] or iters outside [1, 2^24]; I8MM_EDEVICE, I8MM_ELAUNCH as above.
 */
i8mm_status i8mm_calib_mfma_i8(const int8_t* codes, int64_t blocks, int64_t iters, int32_t* out,
                               hipStream_t stream);

/* Library version string (static storage). */
const char* i8mm_version(void);

/* Human-readable name of a status code (static storage). */
const char* i8mm_status_string(i8mm_status status);

#ifdef __cplusplus
}
#endif

#endif /* I8MM_H */
