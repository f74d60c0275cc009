// Host-side checks of the libi8mm C ABI, built with the host sanitizers
// (AddressSanitizer, UndefinedBehaviorSanitizer) from a host-only compile of
// the library sources: argument validation of every entry point, the
// workspace size and layout queries at the extreme accepted shapes, and the
// status strings. Every call made here must be rejected before anything is
// enqueued; the calls with valid arguments (answered I8MM_EDEVICE) are made
// only when the runtime reports no device, so no pointer below is ever
// handed to a kernel.
#include "i8mm.h"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

namespace {

int g_fail = 0;
int g_checks = 0;

void expect(bool ok, const char* what, int line) {
    ++g_checks;
    if (!ok) {
        std::printf("FAILED line %d: %s\n", line, what);
        ++g_fail;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)
#define EXPECT_STATUS(call, want) expect((call) == (want), #call " == " #want, __LINE__)

// Distinct, 256-byte-aligned addresses that are never dereferenced.
template <typename T>
T* fake(uintptr_t k) { return reinterpret_cast<T*>(uintptr_t(1) << 40 | k << 12); }
template <typename T>
T* misaligned(uintptr_t k) { return reinterpret_cast<T*>((uintptr_t(1) << 40 | k << 12) + 2); }

const int64_t kBigS = (int64_t(1) << 31) - 1;

struct Shape { int64_t s, h; };

void check_workspace_queries() {
    const int64_t ss[] = {1, 2, 16, 17, 63, 64, 65, 255, 256, 257, 4096, 1 << 20, kBigS};
    const int64_t hs[] = {64, 128, 192, 4096, 12288, 32768, I8MM_MAX_H - 64, I8MM_MAX_H};
    for (int64_t s : ss)
        for (int64_t h : hs) {
            const size_t total = i8mm_forward_workspace_bytes(s, h);
            size_t off[7];
            int64_t ldo = -1;
            EXPECT_STATUS(i8mm_forward_workspace_layout(s, h, off, &ldo), I8MM_OK);
            EXPECT(total > 0);
            EXPECT(ldo >= (h + 31) / 32 * 32 && ldo % 8 == 0);
            // regions: acc, mask, idx, n_out, Xq, c_x, X_O, in this order,
            // each 256-byte aligned, large enough, inside the total
            const size_t need[7] = {I8MM_FORWARD_ACC_BYTES, size_t(h / 32) * 4, size_t(h) * 4, 4,
                                    size_t(s) * size_t(h), size_t(s) * 4, size_t(s) * size_t(ldo) * 2};
            for (int r = 0; r < 7; ++r) {
                EXPECT(off[r] % 256 == 0);
                const size_t end = off[r] + need[r];
                EXPECT(end <= (r < 6 ? off[r + 1] : total));
            }
            const size_t zp = i8mm_forward_zeropoint_workspace_bytes(s, h);
            EXPECT(zp >= total);
        }
    const Shape bad[] = {{0, 64}, {-1, 64}, {1, 0}, {1, 63}, {1, 96}, {1, -64}, {1, I8MM_MAX_H + 64},
                         {kBigS + 1, 64}, {INT64_MIN, 64}, {1, INT64_MIN}, {INT64_MAX, INT64_MAX}};
    for (const Shape& b : bad) {
        size_t off[7];
        int64_t ldo = 0;
        EXPECT(i8mm_forward_workspace_bytes(b.s, b.h) == 0);
        EXPECT(i8mm_forward_zeropoint_workspace_bytes(b.s, b.h) == 0);
        EXPECT_STATUS(i8mm_forward_workspace_layout(b.s, b.h, off, &ldo), I8MM_EINVAL);
    }
    size_t off[7];
    int64_t ldo = 0;
    EXPECT_STATUS(i8mm_forward_workspace_layout(4, 64, nullptr, &ldo), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_forward_workspace_layout(4, 64, off, nullptr), I8MM_EINVAL);
}

void check_strings() {
    EXPECT(i8mm_version() != nullptr && std::strlen(i8mm_version()) > 0);
    for (int st = -8; st <= 3; ++st) {
        const char* m = i8mm_status_string(static_cast<i8mm_status>(st));
        EXPECT(m != nullptr && std::strlen(m) > 0);
    }
}

// Shapes the products reject: every (s, h, o) below has one bad extent.
struct Dims { int64_t s, h, o; };
const Dims kBadDims[] = {{0, 64, 64},       {1, 63, 64},         {1, 64, 0},          {1, 64, 96},
                         {-5, 64, 64},      {1, I8MM_MAX_H + 64, 64}, {1, 64, -64},   {kBigS + 1, 64, 64},
                         {1, 32768, 65536}, {1, INT64_MAX, 64},  {1, 64, INT64_MAX},  {INT64_MIN, 64, 64}};

void check_weight_conversions() {
    const uint16_t* W = fake<uint16_t>(1);
    int8_t* Wq = fake<int8_t>(2);
    float* cw = fake<float>(3);
    int32_t* zp = fake<int32_t>(4);
    int32_t* cs = fake<int32_t>(5);
    uint16_t* Wp = fake<uint16_t>(6);
    const int64_t h = 256, o = 512;
    EXPECT_STATUS(i8mm_quantize_colwise_weights(nullptr, h, o, Wq, cw, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_quantize_colwise_weights(W, h, o, nullptr, cw, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_quantize_colwise_weights(W, h, o, Wq, nullptr, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_quantize_colwise_weights(misaligned<uint16_t>(1), h, o, Wq, cw, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_quantize_weights_tensorwise(W, h, o, nullptr, cw, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_quantize_colwise_weights_zeropoint(W, h, o, Wq, cw, zp, nullptr, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_pack_fp16_weights(W, h, o, nullptr, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_pack_fp16_weights(W, 32768, 32768, Wp, nullptr), I8MM_EINVAL);   // 2 h o >= 2^31
    for (const Dims& d : kBadDims) {
        if (d.s != 1 || d.h == 32768) continue;   // conversions take no s; 32768 x 65536 is a legal weight shape
        EXPECT_STATUS(i8mm_quantize_colwise_weights(W, d.h, d.o, Wq, cw, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_quantize_weights_tensorwise(W, d.h, d.o, Wq, cw, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_quantize_colwise_weights_zeropoint(W, d.h, d.o, Wq, cw, zp, cs, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_pack_fp16_weights(W, d.h, d.o, Wp, nullptr), I8MM_EINVAL);
    }
}

void check_row_steps() {
    const uint16_t* X = fake<uint16_t>(10);
    uint32_t* mask = fake<uint32_t>(11);
    int32_t* idx = fake<int32_t>(12);
    int32_t* n = fake<int32_t>(13);
    int8_t* Xq = fake<int8_t>(14);
    float* cx = fake<float>(15);
    uint16_t* XO = fake<uint16_t>(16);
    int32_t* zp = fake<int32_t>(17);
    int32_t* rs = fake<int32_t>(18);
    const int64_t s = 8, h = 256, ldo = 256;
    const float bad_alpha[] = {-1.0f, -1e-30f, std::nanf(""), -INFINITY};
    for (float a : bad_alpha)
        EXPECT_STATUS(i8mm_detect_outlier_cols(X, s, h, a, mask, idx, n, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_detect_outlier_cols(nullptr, s, h, 6.0f, mask, idx, n, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_detect_outlier_cols(X, s, h, 6.0f, nullptr, idx, n, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_detect_outlier_cols(X, s, h, 6.0f, mask, misaligned<int32_t>(12), n, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_quantize_rowwise(X, s, h, mask, idx, n, Xq, cx, XO, 224, nullptr), I8MM_EINVAL);  // ldo < h
    EXPECT_STATUS(i8mm_quantize_rowwise(X, s, h, mask, idx, n, Xq, cx, XO, 260, nullptr), I8MM_EINVAL);  // ldo % 8
    EXPECT_STATUS(i8mm_quantize_rowwise(X, s, h, mask, idx, n, nullptr, cx, XO, ldo, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_quantize_tensorwise(X, s, h, mask, idx, n, Xq, nullptr, XO, ldo, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_quantize_rowwise_zeropoint(X, s, h, mask, idx, n, Xq, cx, zp, rs, nullptr, ldo, nullptr),
                  I8MM_EINVAL);
    for (const Dims& d : kBadDims) {
        if (d.o != 64) continue;      // bad s or h
        EXPECT_STATUS(i8mm_detect_outlier_cols(X, d.s, d.h, 6.0f, mask, idx, n, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_quantize_rowwise(X, d.s, d.h, mask, idx, n, Xq, cx, XO, ldo, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_quantize_tensorwise(X, d.s, d.h, mask, idx, n, Xq, cx, XO, ldo, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_quantize_rowwise_zeropoint(X, d.s, d.h, mask, idx, n, Xq, cx, zp, rs, XO, ldo, nullptr),
                      I8MM_EINVAL);
    }
}

void check_products() {
    const int8_t* Xq = fake<int8_t>(20);
    const float* cx = fake<float>(21);
    const uint16_t* XO = fake<uint16_t>(22);
    const int32_t* idx = fake<int32_t>(23);
    const int32_t* n = fake<int32_t>(24);
    const int8_t* Wq = fake<int8_t>(25);
    const float* cw = fake<float>(26);
    const uint16_t* W = fake<uint16_t>(27);
    uint16_t* C = fake<uint16_t>(28);
    float* CO = fake<float>(29);
    int32_t* Ci = fake<int32_t>(30);
    const int32_t* zp = fake<int32_t>(31);
    const int64_t s = 8, h = 256, o = 512, ldo = 256;
    EXPECT_STATUS(i8mm_int8_mixed_matmul(nullptr, cx, XO, ldo, idx, n, Wq, cw, W, nullptr, s, h, o, C, nullptr),
                  I8MM_EINVAL);
    EXPECT_STATUS(i8mm_int8_mixed_matmul(Xq, cx, XO, 128, idx, n, Wq, cw, W, nullptr, s, h, o, C, nullptr),
                  I8MM_EINVAL);
    EXPECT_STATUS(i8mm_int8_mixed_matmul(Xq, cx, XO, ldo, idx, n, Wq, cw, misaligned<uint16_t>(27), nullptr, s, h,
                                         o, C, nullptr),
                  I8MM_EINVAL);
    EXPECT_STATUS(i8mm_int8_mixed_matmul(Xq, cx, XO, ldo, idx, n, Wq, cw, W, misaligned<uint16_t>(32), s, h, o, C,
                                         nullptr),
                  I8MM_EINVAL);
    EXPECT_STATUS(i8mm_outlier_matmul(XO, ldo, idx, n, nullptr, s, h, o, CO, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_int8_gemm_i32(Xq, Wq, s, h, o, nullptr, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_fp16_gemm(XO, nullptr, s, h, o, C, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_zeropoint_matmul(Xq, cx, zp, zp, XO, ldo, idx, n, Wq, cw, zp, nullptr, W, nullptr, s, h, o, C,
                                        nullptr),
                  I8MM_EINVAL);
    for (const Dims& d : kBadDims) {
        const int64_t l = d.h > 0 && d.h < (int64_t(1) << 40) ? (d.h + 31) / 32 * 32 : 64;
        EXPECT_STATUS(i8mm_int8_mixed_matmul(Xq, cx, XO, l, idx, n, Wq, cw, W, nullptr, d.s, d.h, d.o, C, nullptr),
                      I8MM_EINVAL);
        EXPECT_STATUS(i8mm_int8_gemm_i32(Xq, Wq, d.s, d.h, d.o, Ci, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_zeropoint_matmul(Xq, cx, zp, zp, XO, l, idx, n, Wq, cw, zp, zp, W, nullptr, d.s, d.h, d.o,
                                            C, nullptr),
                      I8MM_EINVAL);
        if (d.h != 32768) {
            EXPECT_STATUS(i8mm_outlier_matmul(XO, l, idx, n, W, d.s, d.h, d.o, CO, nullptr), I8MM_EINVAL);
            EXPECT_STATUS(i8mm_fp16_gemm(XO, W, d.s, d.h, d.o, C, nullptr), I8MM_EINVAL);
        }
    }
}

void check_forwards(bool no_device) {
    const uint16_t* X = fake<uint16_t>(40);
    const int8_t* Wq = fake<int8_t>(41);
    const float* cw = fake<float>(42);
    const uint16_t* W = fake<uint16_t>(43);
    uint16_t* C = fake<uint16_t>(44);
    void* ws = fake<void>(45);
    const int32_t* zp = fake<int32_t>(46);
    const int64_t s = 8, h = 256, o = 512;
    const float bad_alpha[] = {-1.0f, std::nanf(""), -INFINITY};
    for (float a : bad_alpha) {
        EXPECT_STATUS(i8mm_forward(X, s, h, o, a, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_decode(X, s, h, o, a, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_noalloc(X, s, h, o, a, Wq, cw, W, nullptr, C, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_tensorwise(X, s, h, o, a, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_zeropoint(X, s, h, o, a, Wq, cw, zp, zp, W, nullptr, ws, C, nullptr),
                      I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_inline_quant(X, 128, h, o, a, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EINVAL);
    }
    // workspace missing or not 256-byte aligned
    EXPECT_STATUS(i8mm_forward(X, s, h, o, 6.0f, Wq, cw, W, nullptr, nullptr, C, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_forward(X, s, h, o, 6.0f, Wq, cw, W, nullptr, misaligned<void>(45), C, nullptr), I8MM_EINVAL);
    void* ws16 = reinterpret_cast<void*>(reinterpret_cast<uintptr_t>(ws) + 16);
    // inline-quantisation forward: at least I8MM_INLINE_QUANT_MIN_ROWS rows, a workspace
    for (int64_t few : {int64_t(1), int64_t(16), int64_t(I8MM_INLINE_QUANT_MIN_ROWS - 1)})
        EXPECT_STATUS(i8mm_forward_inline_quant(X, few, h, o, 6.0f, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_forward_inline_quant(X, 128, h, o, 6.0f, Wq, cw, W, nullptr, nullptr, C, nullptr),
                  I8MM_EINVAL);
    EXPECT_STATUS(i8mm_forward_inline_quant(X, 128, h, o, 6.0f, Wq, cw, W, nullptr, ws16, C, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_forward_inline_quant(X, 128, h, o, 6.0f, Wq, cw, misaligned<uint16_t>(43), nullptr, ws, C,
                                            nullptr),
                  I8MM_EINVAL);
    EXPECT_STATUS(i8mm_forward(X, s, h, o, 6.0f, Wq, cw, W, nullptr, ws16, C, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_forward_decode(X, s, h, o, 6.0f, Wq, cw, W, nullptr, ws16, C, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_forward_tensorwise(X, s, h, o, 6.0f, Wq, cw, W, nullptr, nullptr, C, nullptr), I8MM_EINVAL);
    EXPECT_STATUS(i8mm_forward_zeropoint(X, s, h, o, 6.0f, Wq, cw, zp, zp, W, nullptr, ws16, C, nullptr),
                  I8MM_EINVAL);
    // single-launch decode: at most I8MM_DECODE_MAX_ROWS rows
    EXPECT_STATUS(i8mm_forward_decode(X, I8MM_DECODE_MAX_ROWS + 1, h, o, 6.0f, Wq, cw, W, nullptr, ws, C, nullptr),
                  I8MM_EINVAL);
    // allocation-free forward: shapes whose workspace passes the static scratch
    int64_t big_s = 1;
    while (i8mm_forward_workspace_bytes(big_s, 4096) <= I8MM_NOALLOC_SCRATCH_BYTES) big_s *= 2;
    EXPECT_STATUS(i8mm_forward_noalloc(X, big_s, 4096, o, 6.0f, Wq, cw, W, nullptr, C, nullptr), I8MM_ESCRATCH);
    EXPECT_STATUS(i8mm_forward_noalloc(X, kBigS, I8MM_MAX_H, o, 6.0f, Wq, cw, nullptr, nullptr, C, nullptr),
                  I8MM_ESCRATCH);
    EXPECT_STATUS(i8mm_forward_noalloc(nullptr, s, h, o, 6.0f, Wq, cw, W, nullptr, C, nullptr), I8MM_EINVAL);
    for (const Dims& d : kBadDims) {
        EXPECT_STATUS(i8mm_forward(X, d.s, d.h, d.o, 6.0f, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_decode(X, d.s, d.h, d.o, 6.0f, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_noalloc(X, d.s, d.h, d.o, 6.0f, Wq, cw, W, nullptr, C, nullptr), I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_tensorwise(X, d.s, d.h, d.o, 6.0f, Wq, cw, W, nullptr, ws, C, nullptr),
                      I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_zeropoint(X, d.s, d.h, d.o, 6.0f, Wq, cw, zp, zp, W, nullptr, ws, C, nullptr),
                      I8MM_EINVAL);
        EXPECT_STATUS(i8mm_forward_inline_quant(X, d.s, d.h, d.o, 6.0f, Wq, cw, W, nullptr, ws, C, nullptr),
                      I8MM_EINVAL);
    }
    if (!no_device) return;
    // valid arguments and no device: rejected before anything is enqueued
    i8mm_test_fail_product_launches(0);
    EXPECT_STATUS(i8mm_forward(X, s, h, o, 6.0f, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EDEVICE);
    EXPECT_STATUS(i8mm_forward(X, s, h, o, INFINITY, Wq, cw, nullptr, nullptr, ws, C, nullptr), I8MM_EDEVICE);
    EXPECT_STATUS(i8mm_forward_decode(X, s, h, o, 0.0f, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EDEVICE);
    EXPECT_STATUS(i8mm_forward_noalloc(X, s, h, o, 6.0f, Wq, cw, W, nullptr, C, nullptr), I8MM_EDEVICE);
    EXPECT_STATUS(i8mm_forward_inline_quant(X, I8MM_INLINE_QUANT_MIN_ROWS, h, o, 6.0f, Wq, cw, W, nullptr, ws, C,
                                            nullptr),
                  I8MM_EDEVICE);
    EXPECT_STATUS(i8mm_forward_tensorwise(X, s, h, o, 6.0f, Wq, cw, W, nullptr, ws, C, nullptr), I8MM_EDEVICE);
    EXPECT_STATUS(i8mm_forward_zeropoint(X, s, h, o, 6.0f, Wq, cw, zp, zp, W, nullptr, ws, C, nullptr),
                  I8MM_EDEVICE);
    EXPECT_STATUS(i8mm_int8_gemm_i32(fake<int8_t>(50), Wq, s, h, o, fake<int32_t>(51), nullptr), I8MM_EDEVICE);
    EXPECT_STATUS(i8mm_quantize_colwise_weights(W, h, o, fake<int8_t>(52), fake<float>(53), nullptr), I8MM_EDEVICE);
}

}  // namespace

int main() {
    int ndev = 0;
    const bool no_device = hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0;
    (void)hipGetLastError();
    check_strings();
    check_workspace_queries();
    check_weight_conversions();
    check_row_steps();
    check_products();
    check_forwards(no_device);
    std::printf("%d checks, %d failed (device present: %s)\n", g_checks, g_fail, no_device ? "no" : "yes");
    return g_fail == 0 ? 0 : 1;
}
