// gdn_device.h -- small device helpers shared by the gfx950 kernels:
// 16-lane DPP reductions and 8-element vector loads/stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// Rotate a value by N lanes inside each 16-lane DPP row (row_ror:N).
template <int N>
__device__ __forceinline__ float row_ror(float x)
{
    static_assert(N >= 1 && N <= 15, "row_ror takes 1..15");
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the same
// bits (each step adds a pair of equal partial sums in swapped order, and fp32
// addition is commutative).
__device__ __forceinline__ float row_sum16(float x)
{
    x += row_ror<8>(x);
    x += row_ror<4>(x);
    x += row_ror<2>(x);
    x += row_ror<1>(x);
    return x;
}

// ---- fast elementwise functions on the hardware transcendental unit -------
// e^x = 2^(x log2 e) on v_exp_f32 (about 1 ulp of the power of two, plus the
// rounding of x log2 e: relative error below 1e-6 for |x| < 40).
__device__ __forceinline__ float exp_fast(float x)
{
    return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
// x * sigmoid(x) = x / (1 + e^-x), with the v_rcp_f32 reciprocal (1 ulp).
// For x -> -inf, e^-x overflows to inf and the result is x * 0 = -0.
__device__ __forceinline__ float silu_fast(float x)
{
    return x * __builtin_amdgcn_rcpf(1.0f + exp_fast(-x));
}
// 1 / sqrt(x) on v_rsq_f32 (1 ulp).
__device__ __forceinline__ float rsqrt_fast(float x) { return __builtin_amdgcn_rsqf(x); }

// ---- per-element arithmetic of the pre stage, shared by every kernel that
// runs it (one expression, so the compiler rounds it the same way everywhere)
// 4-tap conv of one channel: taps in order, tap 3 on the current token
__device__ __forceinline__ float conv4(float w0, float w1, float w2, float w3, float x0, float x1,
                                       float x2, float x3)
{
    float acc = w0 * x0;
    acc = fmaf(w1, x1, acc);
    acc = fmaf(w2, x2, acc);
    acc = fmaf(w3, x3, acc);
    return acc;
}
// g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b), on the libm
// exp/log1p (these feed every decay of the scan)
__device__ __forceinline__ void gates(float a, float dt_bias, float A_log, float b, float &g,
                                      float &beta)
{
    const float x = a + dt_bias;
    const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
    g = -expf(A_log) * sp;
    beta = 1.0f / (1.0f + expf(-b));
}

// ---- 8 consecutive elements, widened to / narrowed from fp32 -------------

__device__ __forceinline__ void load8(const float *__restrict__ p, float (&x)[8])
{
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void load8(const _Float16 *__restrict__ p, float (&x)[8])
{
    const half8 v = *reinterpret_cast<const half8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}

__device__ __forceinline__ void store8(float *__restrict__ p, const float (&x)[8])
{
    reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

// fp32 -> fp16 conversion rounds to nearest even (the default mode).
__device__ __forceinline__ void store8(_Float16 *__restrict__ p, const float (&x)[8])
{
    half8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (_Float16)x[i];
    *reinterpret_cast<half8 *>(p) = v;
}

__device__ __forceinline__ float ld1(const float *p) { return *p; }
__device__ __forceinline__ float ld1(const _Float16 *p) { return (float)*p; }

// Raw (not widened) storage of 8 elements, kept packed in registers.
template <typename T> struct Raw8;
template <> struct Raw8<_Float16> {
    half8 v;
    __device__ __forceinline__ void load(const _Float16 *__restrict__ p) { v = *reinterpret_cast<const half8 *>(p); }
    __device__ __forceinline__ void store(_Float16 *__restrict__ p) const { *reinterpret_cast<half8 *>(p) = v; }
    __device__ __forceinline__ void zero() { v = half8(0); }
    __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
};
template <> struct Raw8<float> {
    typedef float f8 __attribute__((ext_vector_type(8), aligned(16)));
    f8 v;
    __device__ __forceinline__ void load(const float *__restrict__ p) { v = *reinterpret_cast<const f8 *>(p); }
    __device__ __forceinline__ void store(float *__restrict__ p) const { *reinterpret_cast<f8 *>(p) = v; }
    __device__ __forceinline__ void zero() { v = f8(0.f); }
    __device__ __forceinline__ float get(int i) const { return v[i]; }
};

} // namespace gdn
