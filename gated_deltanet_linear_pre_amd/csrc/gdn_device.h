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

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt
// left at their maximum, i.e. not waited for).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait for every vector-memory operation this wave has issued.  A kernel that
// issues all its loads first and then calls this before its first store keeps
// the compiler from waiting on earlier stores later on: with loads and stores
// outstanding together, the compiler cannot count either in order and waits
// for everything (vmcnt(0)) wherever a loaded value is next used.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); }

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

// ---- the post stage's arithmetic on one row, shared by every kernel that
// runs it (so that their results agree bit for bit): a 16-lane DPP row holds
// 128 values, 8 per lane; y = ((x inv) gamma) silu(z), inv = 1 / sqrt(mean(x^2)
// + eps), the sum of squares in lane order then across the row.
__device__ __forceinline__ void post_row(const float (&x)[8], const float (&zz)[8],
                                         const float (&gm)[8], float eps, float (&out)[8])
{
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
    ss = row_sum16(ss);
    const float inv = rsqrt_fast(ss * (1.0f / 128.0f) + eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = ((x[i] * inv) * gm[i]) * silu_fast(zz[i]);
}

// ---- per-element arithmetic of the pre stage, shared by every kernel that
// runs it (one expression, so the compiler rounds it the same way everywhere)
// 4-tap conv of one channel: taps in order, tap 3 on the current token.  The
// first tap is w0 x0 + 0 (equal to w0 x0, but a product of -0 becomes +0): as
// a fused multiply-add it, like the other three, takes an fp16 x straight
// from its packed register (v_fma_mix_f32), with no separate conversion.
__device__ __forceinline__ float conv4(float w0, float w1, float w2, float w3, float x0, float x1,
                                       float x2, float x3)
{
    float acc = fmaf(w0, x0, 0.0f);
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

// x[0..3] to p[0..3] and x[4..7] to p[64..67]: the split channel mapping,
// where the 16 lanes of a row cover channels 0..63 with one instruction and
// 64..127 with the next
__device__ __forceinline__ void store8_split(float *__restrict__ p, const float (&x)[8])
{
    reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4 *>(p + 64)[0] = make_float4(x[4], x[5], x[6], x[7]);
}

// store8_split with non-temporal stores, for outputs no later access of the
// same kernel reads (they are not kept in the caches on their way out)
__device__ __forceinline__ void store8_split_nt(float *__restrict__ p, const float (&x)[8])
{
    typedef float v4 __attribute__((ext_vector_type(4)));
    const v4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<v4 *>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<v4 *>(p + 64));
}

// the split channel mapping for whole rows: x[0..3] from p[0..3], x[4..7]
// from p[64..67] (and back)
__device__ __forceinline__ void load8_split(const float *__restrict__ p, float (&x)[8])
{
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p + 64)[0];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void load8_split(const _Float16 *__restrict__ p, float (&x)[8])
{
    typedef _Float16 h4v __attribute__((ext_vector_type(4)));
    const h4v a = *reinterpret_cast<const h4v *>(p);
    const h4v b = *reinterpret_cast<const h4v *>(p + 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = (float)a[i];
        x[4 + i] = (float)b[i];
    }
}

__device__ __forceinline__ void store8_split(_Float16 *__restrict__ p, const float (&x)[8])
{
    typedef _Float16 h4v __attribute__((ext_vector_type(4)));
    h4v a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = (_Float16)x[i];
        b[i] = (_Float16)x[4 + i];
    }
    *reinterpret_cast<h4v *>(p) = a;
    *reinterpret_cast<h4v *>(p + 64) = b;
}

// 16-byte non-temporal load and store, for data one pass touches once
__device__ __forceinline__ float4 load4_nt(const float *__restrict__ p)
{
    typedef float v4 __attribute__((ext_vector_type(4)));
    const v4 t = __builtin_nontemporal_load(reinterpret_cast<const v4 *>(p));
    return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void store4_nt(float *__restrict__ p, float4 x)
{
    typedef float v4 __attribute__((ext_vector_type(4)));
    const v4 t = {x.x, x.y, x.z, x.w};
    __builtin_nontemporal_store(t, reinterpret_cast<v4 *>(p));
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
// load_split / store_split: elements 0..3 at p[0..3], 4..7 at p[64..67].
template <> struct Raw8<_Float16> {
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    half8 v;
    __device__ __forceinline__ void load(const _Float16 *__restrict__ p) { v = *reinterpret_cast<const half8 *>(p); }
    __device__ __forceinline__ void store(_Float16 *__restrict__ p) const { *reinterpret_cast<half8 *>(p) = v; }
    __device__ __forceinline__ void load_split(const _Float16 *__restrict__ p)
    {
        const half4 a = *reinterpret_cast<const half4 *>(p);
        const half4 b = *reinterpret_cast<const half4 *>(p + 64);
        v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ __forceinline__ void store_split(_Float16 *__restrict__ p) const
    {
        *reinterpret_cast<half4 *>(p) = __builtin_shufflevector(v, v, 0, 1, 2, 3);
        *reinterpret_cast<half4 *>(p + 64) = __builtin_shufflevector(v, v, 4, 5, 6, 7);
    }
    __device__ __forceinline__ void zero() { v = half8(0); }
    __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
};
template <> struct Raw8<float> {
    typedef float f8 __attribute__((ext_vector_type(8), aligned(16)));
    typedef float f4v __attribute__((ext_vector_type(4)));
    f8 v;
    __device__ __forceinline__ void load(const float *__restrict__ p) { v = *reinterpret_cast<const f8 *>(p); }
    __device__ __forceinline__ void store(float *__restrict__ p) const { *reinterpret_cast<f8 *>(p) = v; }
    __device__ __forceinline__ void load_split(const float *__restrict__ p)
    {
        const f4v a = *reinterpret_cast<const f4v *>(p);
        const f4v b = *reinterpret_cast<const f4v *>(p + 64);
        v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ __forceinline__ void store_split(float *__restrict__ p) const
    {
        *reinterpret_cast<f4v *>(p) = __builtin_shufflevector(v, v, 0, 1, 2, 3);
        *reinterpret_cast<f4v *>(p + 64) = __builtin_shufflevector(v, v, 4, 5, 6, 7);
    }
    __device__ __forceinline__ void zero() { v = f8(0.f); }
    __device__ __forceinline__ float get(int i) const { return v[i]; }
};

} // namespace gdn
