// C-ABI layer of libi8mm: host-side validation, the device check and the
// launch sequence of each entry point declared in include/i8mm.h.
//
// Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for
// Transformers at Scale" (paper-graph-ui digest), "The Full LLM.int8()
// Algorithm" (Steps 1-5, composed by i8mm_forward).

#include "../../include/i8mm.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

bool valid_shape_sh(int64_t s, int64_t h) {
    return s >= 1 && h >= 64 && h % 64 == 0 && h <= I8MM_MAX_H && s <= (int64_t(1) << 31) - 1;
}

bool valid_o(int64_t o) { return o >= 64 && o % 64 == 0 && o <= (int64_t(1) << 31) - 64; }

// The products address Wq (h o bytes) and W (2 h o bytes, fused product
// only) through 32-bit buffer offsets.
bool valid_w_extent(int64_t h, int64_t o) { return h * o < (int64_t(1) << 31); }

// The dense fp16 product addresses Wp (2 h o bytes) with 32-bit offsets.
bool valid_fp16_extent(int64_t h, int64_t o) { return 2 * h * o < (int64_t(1) << 31); }

i8mm_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return I8MM_EDEVICE;
    }
    if (dev < kMaxDevices) {
        const int cached = g_device_ok[dev].load(std::memory_order_relaxed);
        if (cached == 1) return I8MM_OK;
        if (cached == 2) return I8MM_EDEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return I8MM_EDEVICE;
    }
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices) g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? I8MM_OK : I8MM_EDEVICE;
}

i8mm_status launched(hipError_t e) { return e == hipSuccess ? I8MM_OK : I8MM_ELAUNCH; }

// Test hook: the number of one-call forwards whose product launch is to
// report a failure without launching (i8mm_test_fail_product_launches).
std::atomic<int> g_fail_products{0};

bool product_launch_suppressed() {
    int n = g_fail_products.load(std::memory_order_relaxed);
    while (n > 0)
        if (g_fail_products.compare_exchange_weak(n, n - 1, std::memory_order_relaxed)) return true;
    return false;
}

// Status of a one-call forward whose launches after the first (the
// detection, which writes the workspace accumulator) may have failed: on a
// failure the accumulator is cleared again by one more launch on the same
// stream, so that the workspace stays valid for the next call.
i8mm_status forward_status(hipError_t e, uint32_t* acc, hipStream_t stream) {
    if (e == hipSuccess) return I8MM_OK;
    (void)hipGetLastError();
    if (i8mm::launch_fill_u32(acc, I8MM_FORWARD_ACC_BYTES / 4, 0u, stream) != hipSuccess) {
        (void)hipGetLastError();
        return I8MM_EWORKSPACE;
    }
    return I8MM_ELAUNCH;
}

// The product launch of a one-call forward (or the simulated failure).
template <typename F>
hipError_t product_launch(F&& launch) {
    return product_launch_suppressed() ? hipErrorLaunchFailure : launch();
}

// Workspace of i8mm_forward: the detection accumulator (fixed size, so that its
// place does not depend on the shape), then mask, idx, n_out, Xq, c_x, X_O;
// each 256-byte aligned.
constexpr size_t kAccBytes = I8MM_FORWARD_ACC_BYTES;
void forward_layout(int64_t s, int64_t h, size_t off[7], int64_t* ldo, size_t* total) {
    const int64_t nw = (h + 31) / 32;
    const int64_t l = round_up(h, 32);
    size_t cur = 0;
    auto take = [&](size_t bytes) {
        size_t at = cur;
        cur += static_cast<size_t>(round_up(static_cast<int64_t>(bytes), 256));
        return at;
    };
    off[0] = take(kAccBytes);
    off[1] = take(4 * nw);
    off[2] = take(4 * h);
    off[3] = take(4);
    off[4] = take(static_cast<size_t>(s) * h);
    off[5] = take(4 * s);
    off[6] = take(2 * static_cast<size_t>(s) * l);
    *ldo = l;
    *total = cur;
}

// Scratch of i8mm_forward_noalloc: the forward workspace (accumulator,
// mask, idx, n_out, Xq, c_x, X_O) in a static device array, so that the
// call allocates nothing. Each GPU the library runs on holds its own copy
// from module load until the process ends; zero-initialised at load, and
// the forward leaves its accumulator zero again after every call.
__device__ __align__(256) unsigned char scratch[I8MM_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on each GPU, looked up once per device with
// that device current (the array's name is only a host-side stand-in).
struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
};
ScratchSlot g_scratch[kMaxDevices];

void* scratch_on_current_device(hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&slot, stream] {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        // The array is zero from load; clearing the accumulator once more on
        // the first call's stream costs one small launch per device.
        if (i8mm::launch_fill_u32(static_cast<uint32_t*>(p), I8MM_FORWARD_ACC_BYTES / 4, 0u, stream) != hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        slot.ptr = p;
    });
    return slot.ptr;
}

}  // namespace

extern "C" {

const char* i8mm_version(void) { return "i8mm 0.1.0 (gfx950)"; }

const char* i8mm_status_string(i8mm_status st) {
    switch (st) {
        case I8MM_OK: return "ok";
        case I8MM_EINVAL: return "invalid argument";
        case I8MM_EDEVICE: return "no gfx950 device";
        case I8MM_ELAUNCH: return "kernel launch failed";
        case I8MM_EWORKSPACE: return "kernel launch failed and the workspace accumulator could not be cleared";
        case I8MM_ESCRATCH: return "shape needs more workspace than the static scratch holds";
    }
    return "unknown status";
}

i8mm_status i8mm_quantize_colwise_weights(const uint16_t* W, int64_t h, int64_t o,
                                          int8_t* Wq, float* c_w, hipStream_t stream) {
    if (!W || !Wq || !c_w) return I8MM_EINVAL;
    if (!valid_shape_sh(1, h) || !valid_o(o)) return I8MM_EINVAL;
    if (!aligned16(W) || !aligned16(Wq) || !aligned16(c_w)) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_quantize_cols(W, h, o, Wq, c_w, stream));
}

i8mm_status i8mm_detect_outlier_cols(const uint16_t* X, int64_t s, int64_t h, float alpha,
                                     uint32_t* mask, int32_t* idx, int32_t* n_out,
                                     hipStream_t stream) {
    if (!X || !mask || !idx || !n_out) return I8MM_EINVAL;
    if (!valid_shape_sh(s, h)) return I8MM_EINVAL;
    if (std::isnan(alpha) || alpha < 0.0f) return I8MM_EINVAL;
    if (!aligned16(X) || !aligned16(mask) || !aligned16(idx) || !aligned16(n_out)) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_detect(X, s, h, alpha, mask, idx, n_out, stream));
}

i8mm_status i8mm_quantize_rowwise(const uint16_t* X, int64_t s, int64_t h,
                                  const uint32_t* mask, const int32_t* idx, const int32_t* n_out,
                                  int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo,
                                  hipStream_t stream) {
    if (!X || !mask || !idx || !n_out || !Xq || !c_x || !X_O) return I8MM_EINVAL;
    if (!valid_shape_sh(s, h)) return I8MM_EINVAL;
    if (ldo < round_up(h, 32) || ldo % 8 != 0) return I8MM_EINVAL;
    if (!aligned16(X) || !aligned16(mask) || !aligned16(idx) || !aligned16(n_out) || !aligned16(Xq) ||
        !aligned16(c_x) || !aligned16(X_O))
        return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_quantize_rows(X, s, h, mask, idx, n_out, Xq, c_x, X_O, ldo, stream));
}

i8mm_status i8mm_int8_mixed_matmul(const int8_t* Xq, const float* c_x, const uint16_t* X_O, int64_t ldo,
                                   const int32_t* idx, const int32_t* n_out,
                                   const int8_t* Wq, const float* c_w, const uint16_t* W,
                                   const uint16_t* bias,
                                   int64_t s, int64_t h, int64_t o, uint16_t* C, hipStream_t stream) {
    // W and bias may be null
    if (!Xq || !c_x || !X_O || !idx || !n_out || !Wq || !c_w || !C) return I8MM_EINVAL;
    if (!valid_shape_sh(s, h) || !valid_o(o) || !valid_w_extent(h, o)) return I8MM_EINVAL;
    if (ldo < round_up(h, 32) || ldo % 8 != 0) return I8MM_EINVAL;
    if (!aligned16(Xq) || !aligned16(c_x) || !aligned16(X_O) || !aligned16(idx) || !aligned16(n_out) ||
        !aligned16(Wq) || !aligned16(c_w) || !aligned16(W) || !aligned16(bias) || !aligned16(C))
        return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_int8_gemm(i8mm::GemmOut::Mixed, Xq, c_x, X_O, ldo, idx, n_out, Wq, c_w, W,
                                           bias, s, h, o, C, stream));
}

i8mm_status i8mm_outlier_matmul(const uint16_t* X_O, int64_t ldo, const int32_t* idx, const int32_t* n_out,
                                const uint16_t* W, int64_t s, int64_t h, int64_t o, float* C_O,
                                hipStream_t stream) {
    if (!X_O || !idx || !n_out || !W || !C_O) return I8MM_EINVAL;
    if (!valid_shape_sh(s, h) || !valid_o(o)) return I8MM_EINVAL;
    if (ldo < round_up(h, 32) || ldo % 8 != 0) return I8MM_EINVAL;
    if (!aligned16(X_O) || !aligned16(idx) || !aligned16(n_out) || !aligned16(W) || !aligned16(C_O))
        return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_outlier_matmul(X_O, ldo, idx, n_out, W, s, o, C_O, stream));
}

i8mm_status i8mm_int8_gemm_i32(const int8_t* Xq, const int8_t* Wq, int64_t s, int64_t h, int64_t o,
                               int32_t* C_i32, hipStream_t stream) {
    if (!Xq || !Wq || !C_i32) return I8MM_EINVAL;
    if (!valid_shape_sh(s, h) || !valid_o(o) || !valid_w_extent(h, o)) return I8MM_EINVAL;
    if (!aligned16(Xq) || !aligned16(Wq) || !aligned16(C_i32)) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_int8_gemm(i8mm::GemmOut::Int32, Xq, nullptr, nullptr, 0, nullptr, nullptr, Wq,
                                           nullptr, nullptr, nullptr, s, h, o, C_i32, stream));
}

i8mm_status i8mm_pack_fp16_weights(const uint16_t* W, int64_t h, int64_t o, uint16_t* Wp, hipStream_t stream) {
    if (!W || !Wp) return I8MM_EINVAL;
    if (!valid_shape_sh(1, h) || !valid_o(o) || !valid_fp16_extent(h, o)) return I8MM_EINVAL;
    if (!aligned16(W) || !aligned16(Wp)) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_pack_fp16_panels(W, h, o, Wp, stream));
}

i8mm_status i8mm_fp16_gemm(const uint16_t* X, const uint16_t* Wp, int64_t s, int64_t h, int64_t o, uint16_t* C,
                           hipStream_t stream) {
    if (!X || !Wp || !C) return I8MM_EINVAL;
    if (!valid_shape_sh(s, h) || !valid_o(o) || !valid_fp16_extent(h, o)) return I8MM_EINVAL;
    if (!aligned16(X) || !aligned16(Wp) || !aligned16(C)) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_fp16_gemm(X, Wp, s, h, o, C, stream));
}

i8mm_status i8mm_quantize_tensorwise(const uint16_t* X, int64_t s, int64_t h,
                                     const uint32_t* mask, const int32_t* idx, const int32_t* n_out,
                                     int8_t* Xq, float* c_x, uint16_t* X_O, int64_t ldo, hipStream_t stream) {
    if (!X || !mask || !idx || !n_out || !Xq || !c_x || !X_O) return I8MM_EINVAL;
    if (!valid_shape_sh(s, h)) return I8MM_EINVAL;
    if (ldo < round_up(h, 32) || ldo % 8 != 0) return I8MM_EINVAL;
    if (!aligned16(X) || !aligned16(mask) || !aligned16(idx) || !aligned16(n_out) || !aligned16(Xq) ||
        !aligned16(c_x) || !aligned16(X_O))
        return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_quantize_tensorwise(X, s, h, mask, Xq, c_x, X_O, ldo, stream));
}

i8mm_status i8mm_quantize_weights_tensorwise(const uint16_t* W, int64_t h, int64_t o, int8_t* Wq, float* c_w,
                                             hipStream_t stream) {
    if (!W || !Wq || !c_w) return I8MM_EINVAL;
    if (!valid_shape_sh(1, h) || !valid_o(o)) return I8MM_EINVAL;
    if (!aligned16(W) || !aligned16(Wq) || !aligned16(c_w)) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_quantize_weights_tensorwise(W, h, o, Wq, c_w, stream));
}

i8mm_status i8mm_quantize_rowwise_zeropoint(const uint16_t* X, int64_t s, int64_t h,
                                            const uint32_t* mask, const int32_t* idx, const int32_t* n_out,
                                            int8_t* Xq, float* nd_x, int32_t* zp_x, int32_t* rowsum_x,
                                            uint16_t* X_O, int64_t ldo, hipStream_t stream) {
    if (!X || !mask || !idx || !n_out || !Xq || !nd_x || !zp_x || !rowsum_x || !X_O) return I8MM_EINVAL;
    if (!valid_shape_sh(s, h)) return I8MM_EINVAL;
    if (ldo < round_up(h, 32) || ldo % 8 != 0) return I8MM_EINVAL;
    if (!aligned16(X) || !aligned16(mask) || !aligned16(idx) || !aligned16(n_out) || !aligned16(Xq) ||
        !aligned16(nd_x) || !aligned16(zp_x) || !aligned16(rowsum_x) || !aligned16(X_O))
        return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_quantize_rows_zp(X, s, h, mask, Xq, nd_x, zp_x, rowsum_x, X_O, ldo, stream));
}

i8mm_status i8mm_quantize_colwise_weights_zeropoint(const uint16_t* W, int64_t h, int64_t o, int8_t* Wq,
                                                    float* nd_w, int32_t* zp_w, int32_t* colsum_w,
                                                    hipStream_t stream) {
    if (!W || !Wq || !nd_w || !zp_w || !colsum_w) return I8MM_EINVAL;
    if (!valid_shape_sh(1, h) || !valid_o(o)) return I8MM_EINVAL;
    if (!aligned16(W) || !aligned16(Wq) || !aligned16(nd_w) || !aligned16(zp_w) || !aligned16(colsum_w))
        return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_quantize_cols_zp(W, h, o, Wq, nd_w, zp_w, colsum_w, stream));
}

i8mm_status i8mm_zeropoint_matmul(const int8_t* Xq, const float* nd_x, const int32_t* zp_x,
                                  const int32_t* rowsum_x, const uint16_t* X_O, int64_t ldo,
                                  const int32_t* idx, const int32_t* n_out,
                                  const int8_t* Wq, const float* nd_w, const int32_t* zp_w,
                                  const int32_t* colsum_w, const uint16_t* W, const uint16_t* bias,
                                  int64_t s, int64_t h, int64_t o, uint16_t* C, hipStream_t stream) {
    // bias may be null
    if (!Xq || !nd_x || !zp_x || !rowsum_x || !X_O || !idx || !n_out || !Wq || !nd_w || !zp_w || !colsum_w ||
        !W || !C)
        return I8MM_EINVAL;
    if (!valid_shape_sh(s, h) || !valid_o(o) || !valid_w_extent(h, o)) return I8MM_EINVAL;
    if (ldo < round_up(h, 32) || ldo % 8 != 0) return I8MM_EINVAL;
    if (!aligned16(Xq) || !aligned16(nd_x) || !aligned16(zp_x) || !aligned16(rowsum_x) || !aligned16(X_O) ||
        !aligned16(idx) || !aligned16(n_out) || !aligned16(Wq) || !aligned16(nd_w) || !aligned16(zp_w) ||
        !aligned16(colsum_w) || !aligned16(W) || !aligned16(bias) || !aligned16(C))
        return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_int8_gemm(i8mm::GemmOut::ZeroPoint, Xq, nd_x, X_O, ldo, idx, n_out, Wq, nd_w, W,
                                           bias, s, h, o, C, stream, nullptr, 0,
                                           i8mm::ZpArgs{zp_x, rowsum_x, zp_w, colsum_w}));
}

size_t i8mm_forward_workspace_bytes(int64_t s, int64_t h) {
    if (!valid_shape_sh(s, h)) return 0;
    size_t off[7], total;
    int64_t ldo;
    forward_layout(s, h, off, &ldo, &total);
    return total;
}

i8mm_status i8mm_forward_workspace_layout(int64_t s, int64_t h, size_t offsets[7], int64_t* ldo) {
    if (!offsets || !ldo || !valid_shape_sh(s, h)) return I8MM_EINVAL;
    size_t total;
    forward_layout(s, h, offsets, ldo, &total);
    return I8MM_OK;
}

}  // extern "C"

namespace {

// Arguments of the absmax one-call forward other than its workspace.
i8mm_status check_forward_args(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha, const int8_t* Wq,
                               const float* c_w, const uint16_t* W, const uint16_t* bias, const uint16_t* C) {
    if (!X || !Wq || !c_w || !C) return I8MM_EINVAL;   // W and bias may be null
    if (!valid_shape_sh(s, h) || !valid_o(o) || !valid_w_extent(h, o)) return I8MM_EINVAL;
    if (std::isnan(alpha) || alpha < 0.0f) return I8MM_EINVAL;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(c_w) || !aligned16(W) || !aligned16(bias) ||
        !aligned16(C))
        return I8MM_EINVAL;
    return I8MM_OK;
}

// The launches of the absmax one-call forward over a checked workspace.
i8mm_status run_forward(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha, const int8_t* Wq,
                        const float* c_w, const uint16_t* W, const uint16_t* bias, void* workspace, uint16_t* C,
                        hipStream_t stream) {
    size_t off[7], total;
    int64_t ldo;
    forward_layout(s, h, off, &ldo, &total);
    char* ws = static_cast<char*>(workspace);
    uint32_t* acc = reinterpret_cast<uint32_t*>(ws + off[0]);
    uint32_t* mask = reinterpret_cast<uint32_t*>(ws + off[1]);
    int32_t* idx = reinterpret_cast<int32_t*>(ws + off[2]);
    int32_t* n_out = reinterpret_cast<int32_t*>(ws + off[3]);
    int8_t* Xq = reinterpret_cast<int8_t*>(ws + off[4]);
    float* c_x = reinterpret_cast<float*>(ws + off[5]);
    uint16_t* X_O = reinterpret_cast<uint16_t*>(ws + off[6]);
    int clear_words = 0;
    hipError_t e = i8mm::launch_forward_prologue(X, s, h, alpha, acc, mask, idx, n_out, Xq, c_x, X_O, ldo, stream,
                                                 &clear_words);
    if (e == hipSuccess)
        e = product_launch([&] {
            return i8mm::launch_int8_gemm(i8mm::GemmOut::Mixed, Xq, c_x, X_O, ldo, idx, n_out, Wq, c_w, W, bias, s,
                                          h, o, C, stream, clear_words > 0 ? acc : nullptr, clear_words);
        });
    return forward_status(e, acc, stream);
}

}  // namespace

extern "C" {

i8mm_status i8mm_forward(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                         const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                         void* workspace, uint16_t* C, hipStream_t stream) {
    if (!workspace) return I8MM_EINVAL;
    if (i8mm_status a = check_forward_args(X, s, h, o, alpha, Wq, c_w, W, bias, C)) return a;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return run_forward(X, s, h, o, alpha, Wq, c_w, W, bias, workspace, C, stream);
}

i8mm_status i8mm_forward_decode(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                void* workspace, uint16_t* C, hipStream_t stream) {
    if (!workspace) return I8MM_EINVAL;
    if (i8mm_status a = check_forward_args(X, s, h, o, alpha, Wq, c_w, W, bias, C)) return a;
    if (s > I8MM_DECODE_MAX_ROWS) return I8MM_EINVAL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    size_t off[7], total;
    int64_t ldo;
    forward_layout(s, h, off, &ldo, &total);
    char* ws = static_cast<char*>(workspace);
    return launched(i8mm::launch_decode_fused(
        X, s, h, o, alpha, Wq, c_w, W, bias, C, reinterpret_cast<uint32_t*>(ws + off[1]),
        reinterpret_cast<int32_t*>(ws + off[2]), reinterpret_cast<int32_t*>(ws + off[3]),
        reinterpret_cast<int8_t*>(ws + off[4]), reinterpret_cast<float*>(ws + off[5]),
        reinterpret_cast<uint16_t*>(ws + off[6]), ldo, stream));
}

i8mm_status i8mm_forward_noalloc(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                 const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                 uint16_t* C, hipStream_t stream) {
    if (i8mm_status a = check_forward_args(X, s, h, o, alpha, Wq, c_w, W, bias, C)) return a;
    if (i8mm_forward_workspace_bytes(s, h) > I8MM_NOALLOC_SCRATCH_BYTES) return I8MM_ESCRATCH;
    if (i8mm_status d = check_device()) return d;
    void* ws = scratch_on_current_device(stream);
    if (ws == nullptr) return I8MM_EDEVICE;
    return run_forward(X, s, h, o, alpha, Wq, c_w, W, bias, ws, C, stream);
}

i8mm_status i8mm_forward_inline_quant(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                      const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                      void* workspace, uint16_t* C, hipStream_t stream) {
    if (!workspace) return I8MM_EINVAL;
    if (i8mm_status a = check_forward_args(X, s, h, o, alpha, Wq, c_w, W, bias, C)) return a;
    if (s < I8MM_INLINE_QUANT_MIN_ROWS) return I8MM_EINVAL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    size_t off[7], total;
    int64_t ldo;
    forward_layout(s, h, off, &ldo, &total);
    char* ws = static_cast<char*>(workspace);
    uint32_t* acc = reinterpret_cast<uint32_t*>(ws + off[0]);
    uint32_t* mask = reinterpret_cast<uint32_t*>(ws + off[1]);
    int32_t* idx = reinterpret_cast<int32_t*>(ws + off[2]);
    int32_t* n_out = reinterpret_cast<int32_t*>(ws + off[3]);
    float* c_x = reinterpret_cast<float*>(ws + off[5]);
    uint16_t* X_O = reinterpret_cast<uint16_t*>(ws + off[6]);
    int clear_words = 0;
    hipError_t e = i8mm::launch_forward_prologue(X, s, h, alpha, acc, mask, idx, n_out, nullptr, c_x, X_O, ldo,
                                                 stream, &clear_words);
    if (e == hipSuccess)
        e = product_launch([&] {
            return i8mm::launch_int8_gemm_inline_quant(X, mask, c_x, X_O, ldo, idx, n_out, Wq, c_w, W, bias, s, h, o,
                                                       C, stream, acc, clear_words);
        });
    return forward_status(e, acc, stream);
}

i8mm_status i8mm_forward_tensorwise(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                    const int8_t* Wq, const float* c_w, const uint16_t* W, const uint16_t* bias,
                                    void* workspace, uint16_t* C, hipStream_t stream) {
    if (!X || !Wq || !c_w || !workspace || !C) return I8MM_EINVAL;   // W and bias may be null
    if (!valid_shape_sh(s, h) || !valid_o(o) || !valid_w_extent(h, o)) return I8MM_EINVAL;
    if (std::isnan(alpha) || alpha < 0.0f) return I8MM_EINVAL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return I8MM_EINVAL;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(c_w) || !aligned16(W) || !aligned16(bias) ||
        !aligned16(C))
        return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    size_t off[7], total;
    int64_t ldo;
    forward_layout(s, h, off, &ldo, &total);
    char* ws = static_cast<char*>(workspace);
    uint32_t* acc = reinterpret_cast<uint32_t*>(ws + off[0]);
    int8_t* Xq = reinterpret_cast<int8_t*>(ws + off[4]);
    float* c_x = reinterpret_cast<float*>(ws + off[5]);
    uint16_t* X_O = reinterpret_cast<uint16_t*>(ws + off[6]);
    int32_t* idx = reinterpret_cast<int32_t*>(ws + off[2]);
    int32_t* n_out = reinterpret_cast<int32_t*>(ws + off[3]);
    int clear_words = 0;
    hipError_t e = i8mm::launch_forward_prologue_variant(false, X, s, h, alpha, acc,
                                                         reinterpret_cast<uint32_t*>(ws + off[1]), idx, n_out, Xq,
                                                         c_x, nullptr, nullptr, X_O, ldo, stream, &clear_words);
    if (e == hipSuccess)
        e = product_launch([&] {
            return i8mm::launch_int8_gemm(i8mm::GemmOut::Mixed, Xq, c_x, X_O, ldo, idx, n_out, Wq, c_w, W, bias, s,
                                          h, o, C, stream, acc, clear_words);
        });
    return forward_status(e, acc, stream);
}

size_t i8mm_forward_zeropoint_workspace_bytes(int64_t s, int64_t h) {
    if (!valid_shape_sh(s, h)) return 0;
    size_t off[7], total;
    int64_t ldo;
    forward_layout(s, h, off, &ldo, &total);
    return total + 2 * static_cast<size_t>(round_up(4 * s, 256));
}

i8mm_status i8mm_forward_zeropoint(const uint16_t* X, int64_t s, int64_t h, int64_t o, float alpha,
                                   const int8_t* Wq, const float* nd_w, const int32_t* zp_w, const int32_t* colsum_w,
                                   const uint16_t* W, const uint16_t* bias, void* workspace, uint16_t* C,
                                   hipStream_t stream) {
    if (!X || !Wq || !nd_w || !zp_w || !colsum_w || !W || !workspace || !C) return I8MM_EINVAL;   // bias may be null
    if (!valid_shape_sh(s, h) || !valid_o(o) || !valid_w_extent(h, o)) return I8MM_EINVAL;
    if (std::isnan(alpha) || alpha < 0.0f) return I8MM_EINVAL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return I8MM_EINVAL;
    if (!aligned16(X) || !aligned16(Wq) || !aligned16(nd_w) || !aligned16(zp_w) || !aligned16(colsum_w) ||
        !aligned16(W) || !aligned16(bias) || !aligned16(C))
        return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    size_t off[7], total;
    int64_t ldo;
    forward_layout(s, h, off, &ldo, &total);
    char* ws = static_cast<char*>(workspace);
    uint32_t* acc = reinterpret_cast<uint32_t*>(ws + off[0]);
    int8_t* Xq = reinterpret_cast<int8_t*>(ws + off[4]);
    float* nd_x = reinterpret_cast<float*>(ws + off[5]);
    uint16_t* X_O = reinterpret_cast<uint16_t*>(ws + off[6]);
    int32_t* idx = reinterpret_cast<int32_t*>(ws + off[2]);
    int32_t* n_out = reinterpret_cast<int32_t*>(ws + off[3]);
    int32_t* zp_x = reinterpret_cast<int32_t*>(ws + total);
    int32_t* rowsum_x = reinterpret_cast<int32_t*>(ws + total + round_up(4 * s, 256));
    int clear_words = 0;
    hipError_t e = i8mm::launch_forward_prologue_variant(true, X, s, h, alpha, acc,
                                                         reinterpret_cast<uint32_t*>(ws + off[1]), idx, n_out, Xq,
                                                         nd_x, zp_x, rowsum_x, X_O, ldo, stream, &clear_words);
    if (e == hipSuccess)
        e = product_launch([&] {
            return i8mm::launch_int8_gemm(i8mm::GemmOut::ZeroPoint, Xq, nd_x, X_O, ldo, idx, n_out, Wq, nd_w, W, bias,
                                          s, h, o, C, stream, acc, clear_words,
                                          i8mm::ZpArgs{zp_x, rowsum_x, zp_w, colsum_w});
        });
    return forward_status(e, acc, stream);
}

i8mm_status i8mm_calib_mfma_i8(const int8_t* codes, int64_t blocks, int64_t iters, int32_t* out,
                               hipStream_t stream) {
    if (!codes || !out || !aligned16(codes) || !aligned16(out)) return I8MM_EINVAL;
    if (blocks < 1 || blocks > (int64_t(1) << 20) || iters < 1 || iters > (int64_t(1) << 24)) return I8MM_EINVAL;
    if (i8mm_status d = check_device()) return d;
    return launched(i8mm::launch_calib_mfma_i8(codes, blocks, iters, out, stream));
}

void i8mm_test_fail_product_launches(int count) {
    g_fail_products.store(count > 0 ? count : 0, std::memory_order_relaxed);
}

}  // extern "C"
