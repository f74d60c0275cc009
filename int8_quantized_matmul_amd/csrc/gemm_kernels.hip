// The decomposed product of LLM.int8() on gfx950 matrix cores:
//   C[s, o] = fp16( C_i32 / (c_x (x) c_w) + X_O W[idx, :] ),  C_i32 = Xq Wq_t^T.
//
// Page tags: [DIGEST] "LLM.int8(): 8-bit Matrix Multiplication for
// Transformers at Scale" (paper-graph-ui digest), "The Full LLM.int8()
// Algorithm", Steps 3-5, and "Mixed-Precision Decomposition" (formal
// definition); [PY] "LLM.int8() 完全拆解" (pinghaoyang.com.cn),
// "第二件武器：混合精度分解".
//
// Both operands of the int8 product keep the reduction dimension h
// contiguous (Xq [s, h], Wq_t [o, h]), so every lane feeds the MFMA from one
// 16-byte run. The matrix core computes D[o][s] (Wq_t as the A operand), so
// each lane ends up holding runs of 4 consecutive output columns of one row
// of C and stores them as one 8-byte fp16 quad.
//
// Two main loops share the epilogue structure:
//  * k_gemm_prefill: 256x256 output tile per 256-thread block, K step 128,
//    LDS double buffering with a register-staged global prefetch,
//    v_mfma_i32_32x32x32_i8, 2x2 waves of 128x128.
//  * k_gemm_decode (s <= 16): weight streaming. One wavefront per 16*NT
//    output columns reads its rows of Wq_t straight from HBM into the MFMA
//    operand registers (v_mfma_i32_16x16x64_i8, rows of X beyond s are
//    zero), several K steps in flight.
// The fused epilogue converts the int32 accumulator to fp32, multiplies by
// 1/c_x_i * 1/c_w_j (S is never materialised), then accumulates the fp16
// outlier product on top with fp16 MFMA (fp32 accumulate) and rounds once
// to fp16.

#include "device_common.h"
#include "launch.h"

namespace i8mm {
namespace {

// ------------------------------------------------------------------ prefill
constexpr int kTO = 256;   // output columns (o) per block
constexpr int kTS = 256;   // output rows (s) per block
constexpr int kTK = 128;   // reduction bytes per LDS stage
constexpr int kStageA = kTO * kTK / 16;  // v4i slots
constexpr int kStageB = kTS * kTK / 16;
constexpr int kStage = kStageA + kStageB;

// 16-byte slot of chunk `c` (0..7) of LDS row `row` (rows are 128 bytes):
// XOR swizzle so that 8 consecutive rows reading the same chunk hit 8
// different 16-byte bank groups.
__device__ __forceinline__ int swz(int row, int c) { return row * 8 + (c ^ (row & 7)); }

template <GemmOut MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_gemm_prefill(const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq_t,
                    int64_t s, int64_t h, int64_t o,
                    const float* __restrict__ c_x, const float* __restrict__ c_w,
                    const uint16_t* __restrict__ X_O, int64_t ldo,
                    const int32_t* __restrict__ idx, const int32_t* __restrict__ n_out,
                    const uint16_t* __restrict__ W, void* __restrict__ Cout) {
    __shared__ v4i lds[2 * kStage];

    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int wo = wid & 1, ws = wid >> 1;
    const int64_t n_ts = (s + kTS - 1) / kTS;
    const int64_t ts_i = static_cast<int64_t>(blockIdx.x) % n_ts;
    const int64_t to_i = static_cast<int64_t>(blockIdx.x) / n_ts;
    const int64_t o0 = to_i * kTO, s0 = ts_i * kTS;

    // Global -> register staging: thread t moves chunk (t & 7) of rows
    // (t >> 3) + 32 p, p = 0..7, of both tiles.
    const int st_c = t & 7, st_r = t >> 3;
    v4i ra[8], rb[8];
    const int64_t KT = (h + kTK - 1) / kTK;
    const v4i zero4 = {0, 0, 0, 0};

    auto gload = [&](int64_t kt) {
        const int64_t k = kt * kTK + st_c * 16;
        const bool kin = k < h;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int64_t row = st_r + 32 * p;
            const int64_t orow = o0 + row, srow = s0 + row;
            ra[p] = (kin && orow < o) ? *reinterpret_cast<const v4i*>(Wq_t + orow * h + k) : zero4;
            rb[p] = (kin && srow < s) ? *reinterpret_cast<const v4i*>(Xq + srow * h + k) : zero4;
        }
    };
    auto lstore = [&](int buf) {
        v4i* A = lds + buf * kStage;
        v4i* B = A + kStageA;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int row = st_r + 32 * p;
            A[swz(row, st_c)] = ra[p];
            B[swz(row, st_c)] = rb[p];
        }
    };

    v16i acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0;

    gload(0);
    lstore(0);
    __syncthreads();
    const int r32 = lane & 31, khalf = lane >> 5;
    for (int64_t kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) gload(kt + 1);
        const v4i* A = lds + (kt & 1) * kStage;
        const v4i* B = A + kStageA;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int c = kk * 2 + khalf;
            v4i a[4], b[4];
#pragma unroll
            for (int ob = 0; ob < 4; ++ob) a[ob] = A[swz(wo * 128 + ob * 32 + r32, c)];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) b[sb] = B[swz(ws * 128 + sb * 32 + r32, c)];
#pragma unroll
            for (int ob = 0; ob < 4; ++ob)
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
                    acc[ob][sb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[ob], b[sb], acc[ob][sb], 0, 0, 0);
        }
        if (kt + 1 < KT) lstore((kt + 1) & 1);
        __syncthreads();
    }

    // Lane layout of a 32x32 accumulator: register r holds
    // D[o = 8 (r / 4) + 4 (lane / 32) + r % 4][s = lane % 32].
    if constexpr (MODE == GemmOut::Int32) {
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
        float inv_x[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const int64_t srow = s0 + ws * 128 + sb * 32 + r32;
            inv_x[sb] = 1.0f / (srow < s ? c_x[srow] : 1.0f);
        }
        const int n = n_out[0];
        // One 32-column block at a time, so that only 64 fp32 values are
        // live next to the remaining int32 accumulators.
#pragma unroll
        for (int ob = 0; ob < 4; ++ob) {
            // Dequantise: f = C_i32 * (1/c_x) * (1/c_w).
            v16f f[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int64_t ocol = o0 + wo * 128 + ob * 32 + 8 * g + 4 * khalf;
                v4f cw = ocol < o ? *reinterpret_cast<const v4f*>(c_w + ocol) : v4f{1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float inv_w = 1.0f / cw[e];
#pragma unroll
                    for (int sb = 0; sb < 4; ++sb)
                        f[sb][4 * g + e] = static_cast<float>(acc[ob][sb][4 * g + e]) * (inv_x[sb] * inv_w);
                }
            }
            // Outlier product X_O W[idx, :] with v_mfma_f32_32x32x16_f16. The A
            // operand holds W[idx[k], ocol] for ocol = lane % 32 of the block
            // and k = 16 kb + 8 (lane / 32) + e; the B operand holds the same
            // k range of X_O row srow (zero-padded past |O|).
            const int64_t ocol_a = o0 + wo * 128 + ob * 32 + r32;
            for (int kb = 0; kb * 16 < n; ++kb) {
                const int kbase = kb * 16 + 8 * khalf;
                v8h wa;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int k = kbase + e;
                    uint16_t bits = (k < n && ocol_a < o) ? W[static_cast<int64_t>(idx[k]) * o + ocol_a]
                                                          : static_cast<uint16_t>(0);
                    wa[e] = __builtin_bit_cast(_Float16, bits);
                }
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) {
                    const int64_t srow = s0 + ws * 128 + sb * 32 + r32;
                    v8h xb;
                    if (srow < s) {
                        xb = *reinterpret_cast<const v8h*>(X_O + srow * ldo + kbase);
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) xb[e] = static_cast<_Float16>(0.0f);
                    }
                    f[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wa, xb, f[sb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const int64_t srow = s0 + ws * 128 + sb * 32 + r32;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int64_t ocol = o0 + wo * 128 + ob * 32 + 8 * g + 4 * khalf;
                    if (srow < s && ocol < o) {
                        const uint32_t lo = float_to_half_bits(f[sb][4 * g]) |
                                            (static_cast<uint32_t>(float_to_half_bits(f[sb][4 * g + 1])) << 16);
                        const uint32_t hi = float_to_half_bits(f[sb][4 * g + 2]) |
                                            (static_cast<uint32_t>(float_to_half_bits(f[sb][4 * g + 3])) << 16);
                        *reinterpret_cast<uint2*>(C + srow * o + ocol) = make_uint2(lo, hi);
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ decode
// 16x16 fp16 outlier accumulation shared by the decode epilogue and the
// standalone outlier product: f (16x16 fp32 tile, lane layout of
// v_mfma_f32_16x16x32_f16: register r <-> D[o = 4 (lane / 16) + r][s = lane % 16])
// += X_O[s, k] W[idx[k], o] over k < n.
__device__ __forceinline__ v4f outlier_tile_16x16(v4f f, int lane, int64_t ocol, int64_t srow, int64_t s,
                                                   int64_t o, const uint16_t* __restrict__ X_O, int64_t ldo,
                                                   const int32_t* __restrict__ idx, int n,
                                                   const uint16_t* __restrict__ W) {
    const int g = lane >> 4;
    for (int kb = 0; kb * 32 < n; ++kb) {
        const int kbase = kb * 32 + 8 * g;
        v8h wa, xb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = kbase + e;
            uint16_t bits = (k < n && ocol < o) ? W[static_cast<int64_t>(idx[k]) * o + ocol] : static_cast<uint16_t>(0);
            wa[e] = __builtin_bit_cast(_Float16, bits);
        }
        if (srow < s) {
            xb = *reinterpret_cast<const v8h*>(X_O + srow * ldo + kbase);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) xb[e] = static_cast<_Float16>(0.0f);
        }
        f = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, xb, f, 0, 0, 0);
    }
    return f;
}

constexpr int kDecodeUnroll = 8;

template <GemmOut MODE, int NT>
__global__ __launch_bounds__(256) void k_gemm_decode(const int8_t* __restrict__ Xq, const int8_t* __restrict__ Wq_t,
                                                     int64_t s, int64_t h, int64_t o,
                                                     const float* __restrict__ c_x, const float* __restrict__ c_w,
                                                     const uint16_t* __restrict__ X_O, int64_t ldo,
                                                     const int32_t* __restrict__ idx,
                                                     const int32_t* __restrict__ n_out,
                                                     const uint16_t* __restrict__ W, void* __restrict__ Cout) {
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + wid;
    const int64_t obase = gw * 16 * NT;
    if (obase >= o) return;   // whole wavefront; no block-level synchronisation below

    const int r16 = lane & 15, g = lane >> 4;
    const int8_t* wp[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        int64_t orow = obase + nt * 16 + r16;
        if (orow >= o) orow = o - 1;   // never used for output; keeps loads in bounds
        wp[nt] = Wq_t + orow * h + g * 16;
    }
    const bool xvalid = r16 < s;
    const int8_t* xp = Xq + (xvalid ? r16 : 0) * h + g * 16;
    const v4i zero4 = {0, 0, 0, 0};

    v4i acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = zero4;

    const int64_t nsteps = h / 64;
    int64_t st = 0;
    for (; st + kDecodeUnroll <= nsteps; st += kDecodeUnroll) {
        v4i a[kDecodeUnroll][NT], b[kDecodeUnroll];
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u) {
            const int64_t k = (st + u) * 64;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                a[u][nt] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp[nt] + k));
            b[u] = xvalid ? *reinterpret_cast<const v4i*>(xp + k) : zero4;
        }
#pragma unroll
        for (int u = 0; u < kDecodeUnroll; ++u)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[u][nt], b[u], acc[nt], 0, 0, 0);
    }
    for (; st < nsteps; ++st) {
        const int64_t k = st * 64;
        v4i b = xvalid ? *reinterpret_cast<const v4i*>(xp + k) : zero4;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            v4i a = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wp[nt] + k));
            acc[nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[nt], 0, 0, 0);
        }
    }

    // Lane layout of a 16x16 accumulator: register r holds D[o = 4 g + r][s = r16].
    const int64_t srow = r16;
    if constexpr (MODE == GemmOut::Int32) {
        int32_t* C = static_cast<int32_t*>(Cout);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int64_t ocol = obase + nt * 16 + 4 * g;
            if (srow < s && ocol < o) *reinterpret_cast<v4i*>(C + srow * o + ocol) = acc[nt];
        }
    } else {
        uint16_t* C = static_cast<uint16_t*>(Cout);
        const float inv_x = 1.0f / (srow < s ? c_x[srow] : 1.0f);
        const int n = n_out[0];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int64_t ocol = obase + nt * 16 + 4 * g;
            v4f cw = ocol < o ? *reinterpret_cast<const v4f*>(c_w + ocol) : v4f{1.f, 1.f, 1.f, 1.f};
            v4f f;
#pragma unroll
            for (int e = 0; e < 4; ++e) f[e] = static_cast<float>(acc[nt][e]) * (inv_x * (1.0f / cw[e]));
            f = outlier_tile_16x16(f, lane, obase + nt * 16 + r16, srow, s, o, X_O, ldo, idx, n, W);
            if (srow < s && ocol < o) {
                const uint32_t lo = float_to_half_bits(f[0]) | (static_cast<uint32_t>(float_to_half_bits(f[1])) << 16);
                const uint32_t hi = float_to_half_bits(f[2]) | (static_cast<uint32_t>(float_to_half_bits(f[3])) << 16);
                *reinterpret_cast<uint2*>(C + srow * o + ocol) = make_uint2(lo, hi);
            }
        }
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
    f = outlier_tile_16x16(f, lane, to_i * 16 + r16, srow, s, o, X_O, ldo, idx, n_out[0], W);
    const int64_t ocol = to_i * 16 + 4 * g;
    if (srow < s) *reinterpret_cast<v4f*>(C_O + srow * o + ocol) = f;
}

template <GemmOut MODE>
hipError_t launch_mode(const int8_t* Xq, const float* c_x, const uint16_t* X_O, int64_t ldo,
                       const int32_t* idx, const int32_t* n_out, const int8_t* Wq_t, const float* c_w,
                       const uint16_t* W, int64_t s, int64_t h, int64_t o, void* C, hipStream_t stream) {
    if (s <= 16) {
        constexpr int NT = 2;
        const int64_t waves = (o + 16 * NT - 1) / (16 * NT);
        hipLaunchKernelGGL((k_gemm_decode<MODE, NT>), dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0,
                           stream, Xq, Wq_t, s, h, o, c_x, c_w, X_O, ldo, idx, n_out, W, C);
    } else {
        const int64_t tiles = ((s + kTS - 1) / kTS) * ((o + kTO - 1) / kTO);
        hipLaunchKernelGGL((k_gemm_prefill<MODE>), dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream,
                           Xq, Wq_t, s, h, o, c_x, c_w, X_O, ldo, idx, n_out, W, C);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_int8_gemm(GemmOut mode, const int8_t* Xq, const float* c_x,
                            const uint16_t* X_O, int64_t ldo,
                            const int32_t* idx, const int32_t* n_out,
                            const int8_t* Wq_t, const float* c_w, const uint16_t* W,
                            int64_t s, int64_t h, int64_t o, void* C, hipStream_t stream) {
    if (mode == GemmOut::Int32)
        return launch_mode<GemmOut::Int32>(Xq, c_x, X_O, ldo, idx, n_out, Wq_t, c_w, W, s, h, o, C, stream);
    return launch_mode<GemmOut::Mixed>(Xq, c_x, X_O, ldo, idx, n_out, Wq_t, c_w, W, s, h, o, C, stream);
}

hipError_t launch_outlier_matmul(const uint16_t* X_O, int64_t ldo, const int32_t* idx, const int32_t* n_out,
                                 const uint16_t* W, int64_t s, int64_t o, float* C_O, hipStream_t stream) {
    const int64_t tiles = (o / 16) * ((s + 15) / 16);
    hipLaunchKernelGGL(k_outlier_only, dim3(static_cast<unsigned>((tiles + 3) / 4)), dim3(256), 0, stream,
                       X_O, ldo, idx, n_out, W, s, o, C_O);
    return hipGetLastError();
}

}  // namespace i8mm
