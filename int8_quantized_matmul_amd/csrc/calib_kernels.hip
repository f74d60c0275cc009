// Measurement calibration for the product kernels' roofline: a stream of
// v_mfma_i32_32x32x32_i8 on register-resident operands, with no memory
// traffic inside its loop. It gives the int8 matrix-core rate this chip
// sustains under load (clock and power limits included), the practical
// ceiling beside the published peak. Not part of the method.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace i8mm {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Each wavefront holds two sets of four A and four B fragments (the caller's
// random codes, so the matrix cores switch as on real data) and sixteen
// independent 32 x 32 int32 accumulators (256 accumulator registers, as in
// the prefill product); one iteration is 32 MFMAs, each set once against
// every accumulator. The XOR of the accumulators keeps the work alive.
__global__ __launch_bounds__(256) void k_calib_mfma_i8(const v4i* __restrict__ codes, int64_t iters,
                                                       int32_t* __restrict__ out) {
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    v4i a[2][4], b[2][4];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a[p][i] = codes[t * 16 + p * 8 + i];
            b[p][i] = codes[t * 16 + p * 8 + 4 + i];
        }
    v16i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16i{};
    for (int64_t it = 0; it < iters; ++it)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[p][i], b[p][j], acc[i][j], 0, 0, 0);
    v16i x = acc[0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (i + j > 0) x ^= acc[i][j];
    int32_t y = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) y ^= x[r];
    out[t] = y;
}

}  // namespace

hipError_t launch_calib_mfma_i8(const int8_t* codes, int64_t blocks, int64_t iters, int32_t* out,
                                hipStream_t stream) {
    hipLaunchKernelGGL(k_calib_mfma_i8, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       reinterpret_cast<const v4i*>(codes), iters, out);
    return hipGetLastError();
}

}  // namespace i8mm
