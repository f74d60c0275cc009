// Device-side types and helpers shared by the gfx950 kernels of libi8mm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i8mm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
    // The empty asm pins f as an fp32 register value: otherwise the
    // compiler may fold the multiply that produced f into a mixed-precision
    // FMA that rounds the exact product once, straight to fp16, which
    // differs from rounding to fp32 first at fp16 ties. It emits nothing.
    asm("" : "+v"(f));
    // v_cvt_f16_f32 rounds to nearest even in the default mode.
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Two fp32 values rounded to fp16 (to nearest even) and packed, lo in the
// low half, by one v_cvt_pk_f16_f32 (checked bit-equal to converting each
// value on its own, for every fp32 input). Being asm it also pins both
// values as fp32, like float_to_half_bits.
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
    uint32_t r;
    asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}

// fl32(127 / m) with an IEEE correctly rounded division; 1 when m == 0.
__device__ __forceinline__ float absmax_scale(float m) {
    return m > 0.0f ? __fdiv_rn(127.0f, m) : 1.0f;
}

// One fp32 multiply, then round half away from zero. v = fl32(x c) is
// taken as an FMA with a -0 addend, which is the rounded product exactly
// (also for a zero product, whose sign it keeps) and lets an fp16 x enter
// the multiply without a separate conversion. Rounding: the float-to-int
// conversion truncates, and adding the largest float below 1/2 with v's
// sign first pushes exactly the ties and everything above them past the
// next integer (checked for every fp32 value of magnitude at most 256).
// Every caller scales by c = fl32(127 / m) with |x| <= m (m the absmax of
// the values of its row, column or tensor), so |v| <= 127 and the code is
// in [-127, 127] without a clamp.
__device__ __forceinline__ int quantize_one(float x, float c) {
    const float v = __builtin_fmaf(x, c, -0.0f);
    const float t = __fadd_rn(v, copysignf(0.49999997f, v));
    return static_cast<int>(t);
}

// The low bytes of four ints packed into one word, b0 lowest.
__device__ __forceinline__ uint32_t pack_bytes(int b0, int b1, int b2, int b3) {
    // v_perm_b32 selector bytes 0-3 pick bytes of the second operand, 4-7
    // bytes of the first, 0x0c a zero byte
    const uint32_t lo = __builtin_amdgcn_perm(static_cast<uint32_t>(b1), static_cast<uint32_t>(b0), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(static_cast<uint32_t>(b3), static_cast<uint32_t>(b2), 0x04000c0cu);
    return lo | hi;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int t = __shfl_up(v, off, kWave);
        if (lane >= off) v += t;
    }
    return v;
}

}  // namespace i8mm
