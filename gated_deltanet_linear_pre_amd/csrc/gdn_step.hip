// gdn_step.hip -- one decode token per sequence through the whole layer:
// conv with the carried history, SiLU, L2 norms, gates, one step of the gated
// delta rule on the fp32 state, RMSNorm with gamma and the SiLU(z) gate.
//
// "Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1
// (gdn_scan_r findings): the state of a value head is updated token by token
// in the pass that forms the dot products against the old state; the pages
// check every scan variant against the single-token step.  Per sequence n,
// value head h (key head j = h / G), with X = [hist[n]; qkv[n]] (4 rows):
//   x~[c] = sum_m conv_w[c][m] X[m][c],  s = SiLU(x~)
//   q^ = s_q / sqrt(|s_q|^2 + eps), k^ likewise, v = s_v
//   alpha = exp(g), g = -exp(A_log[h]) softplus(a + dt_bias[h]), beta = sigmoid(b)
//   S <- alpha S + beta (v - alpha S k^) k^T,  o = S q^ / sqrt(dk)
//   y = o / sqrt(mean(o^2) + eps_rms) * gamma * z * sigmoid(z)
//   hist[n] <- X[1 .. 3]
//
// gfx950 mapping.  Decode moves the whole state (64 KB per head) in and out
// for 7 flop per element, so it is bound by HBM bandwidth and launch latency.
// One 256-thread block per (sequence, value head):
//   - each thread issues the loads of its 64 state elements first, so they
//     are in flight while the block computes the token's q, k, v and gates.
//     A group of 8 lanes owns 4 rows; in each of its 16 loads (and stores)
//     the group covers one whole 128-byte line (32 keys) of one row, lane e
//     taking keys 4e..4e+3 of it, so every memory instruction moves whole
//     lines (with half a row per thread each instruction touched 64 lines,
//     16 bytes of each).  The state goes in and out non-temporally: a layer's
//     state is next needed one decode step later, after every other layer's
//     (at batch 64 this took the step from 85 to 73 us per layer);
//   - threads 0..127 each take channel c of the key head's q and k and of the
//     value head's v: 4-tap conv, SiLU, and the three sums q.q, k.k, q.k,
//     reduced over the block (DPP inside a 16-lane row, then LDS);
//   - the state step: each thread forms its 16-key parts of S k^ and S q^
//     for its 4 rows, the group adds them in a 3-step butterfly (every lane
//     ends with the same bits), and writes alpha S + u k^T back;
//     o = alpha (S q^) + u (k^.q^) is the same quantity as (alpha S + u k^T) q^
//     in one pass;
//   - the RMSNorm over the head's 128 outputs and the gated output.
// With the new history going to its own buffer (hist_out), the step kernel
// writes it too: each block the rows of its value head's v channels, the
// first block of each key-head group those of the group's q and k channels,
// all read from the old history, which no block writes: one launch.  In
// place, a second launch shifts the history (every block of a key-head group
// reads the group's q/k history, so no block of the first launch may
// overwrite it).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

struct StepDims {
    int hk, hv, G, C;
    float eps_l2, eps_rms;
};

constexpr float STEP_SCALE = 0.08838834764831845f;  // 1 / sqrt(128)

// Sum over a 64-lane wave (DPP inside rows of 16, then the four row sums).
__device__ __forceinline__ float wave_sum(float x)
{
    x = row_sum16(x);
    float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    s += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return s;
}

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void step_kernel(StepArgs p, StepDims d)
{
    __shared__ float sq[128], sk[128], sv[128];
    __shared__ float red[4][4];
    __shared__ float orow[128];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = blockIdx.x / d.hv;
    const int h = blockIdx.x - n * d.hv;
    const int j = h / d.G;
    const int C = d.C;

    // ---- the token's inputs, then the state -------------------------------
    // Every thread loads the inputs of channel tid % 128 of the key head's q
    // and k and of the value head's v, and the head's gate inputs (the same
    // for all), unconditionally and before the state: loads complete in
    // order, so the conv and the norms below wait only for these, while the
    // state's 64 KB is still on its way.
    const TI *qkv = static_cast<const TI *>(p.qkv) + (int64_t)n * C;
    const TI *hist = static_cast<const TI *>(p.hist) + (int64_t)n * 3 * C;
    const TI *cw = static_cast<const TI *>(p.conv_w);
    const int c = tid & 127;
    const int chq = j * 128 + c, chk = d.hk * 128 + j * 128 + c, chv = 2 * d.hk * 128 + h * 128 + c;
    // raw values first (converted only once the state loads are out)
    TI wq[4], wk[4], wv[4], xq[4], xk[4], xv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        wq[m] = cw[(int64_t)chq * 4 + m];
        wk[m] = cw[(int64_t)chk * 4 + m];
        wv[m] = cw[(int64_t)chv * 4 + m];
    }
#pragma unroll
    for (int m = 0; m < 3; ++m) {
        xq[m] = hist[m * C + chq];
        xk[m] = hist[m * C + chk];
        xv[m] = hist[m * C + chv];
    }
    xq[3] = qkv[chq];
    xk[3] = qkv[chk];
    xv[3] = qkv[chv];
    const TI ga = static_cast<const TI *>(p.a)[(int64_t)n * d.hv + h];
    const TI gb = static_cast<const TI *>(p.b)[(int64_t)n * d.hv + h];
    const TI gdt = static_cast<const TI *>(p.dt_bias)[h];
    const TI gal = static_cast<const TI *>(p.A_log)[h];

    // S[4 m + l] = keys 32 l + 4 e .. + 3 of row 4 grp + m
    const int grp = tid >> 3, e = tid & 7;
    float *Sblk = p.state + (((int64_t)n * d.hv + h) * 128 + 4 * grp) * 128 + 4 * e;
    float4 S[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        S[i] = load4_nt(Sblk + (i >> 2) * 128 + (i & 3) * 32);
    __builtin_amdgcn_sched_barrier(0);  // every load is out before the first use

    // ---- the token's q, k (key head j) and v (value head h) ---------------
    auto cv4 = [](const TI (&w)[4], const TI (&x)[4]) {
        return silu_fast(conv4((float)w[0], (float)w[1], (float)w[2], (float)w[3], (float)x[0],
                               (float)x[1], (float)x[2], (float)x[3]));
    };
    const float q = cv4(wq, xq);
    const float k = cv4(wk, xk);
    const float v = cv4(wv, xv);
    // the new history X[1..3] of this block's channels, when it has a
    // buffer of its own
    if (p.hist_out && tid < 128) {
        TI *ho = static_cast<TI *>(p.hist_out) + (int64_t)n * 3 * C;
#pragma unroll
        for (int m = 0; m < 3; ++m) ho[m * C + chv] = xv[m + 1];
        if (h % d.G == 0) {
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                ho[m * C + chq] = xq[m + 1];
                ho[m * C + chk] = xk[m + 1];
            }
        }
    }
    float sumq = 0.f, sumk = 0.f, sumqk = 0.f;
    if (tid < 128) {
        sq[c] = q;
        sk[c] = k;
        sv[c] = v;
        sumq = q * q;
        sumk = k * k;
        sumqk = q * k;
    }
    if (wave < 2) {
        sumq = wave_sum(sumq);
        sumk = wave_sum(sumk);
        sumqk = wave_sum(sumqk);
        if (lane == 0) {
            red[wave][0] = sumq;
            red[wave][1] = sumk;
            red[wave][2] = sumqk;
        }
    }
    // the gates, formed by every thread from the same inputs in the same way
    float g, beta;
    gates((float)ga, (float)gdt, (float)gal, (float)gb, g, beta);
    const float alpha = expf(g);
    __syncthreads();
    const float inv_q = rsqrt_fast((red[0][0] + red[1][0]) + d.eps_l2);
    const float inv_k = rsqrt_fast((red[0][1] + red[1][1]) + d.eps_l2);
    const float kq = (red[0][2] + red[1][2]) * inv_q * inv_k;

    // ---- one step of the delta rule on this thread's 4 row pieces -----------
    float4 kv[4], qv[4];  // keys 32 l + 4 e .. + 3
#pragma unroll
    for (int l = 0; l < 4; ++l) {
        kv[l] = *reinterpret_cast<const float4 *>(&sk[32 * l + 4 * e]);
        qv[l] = *reinterpret_cast<const float4 *>(&sq[32 * l + 4 * e]);
    }
    // the sum over the 8 lanes of the group: lanes exchange with lane ^ 1,
    // lane ^ 2 (quad permutes) and 7 - lane (half-row mirror); each addition
    // pairs equal partial sums, so every lane gets the same bits
    auto group_sum = [](float x) {
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
        return x;
    };
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float Sk = 0.f, Sq = 0.f;
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const float4 s4 = S[4 * m + l];
            Sk = fmaf(s4.x, kv[l].x, Sk); Sk = fmaf(s4.y, kv[l].y, Sk);
            Sk = fmaf(s4.z, kv[l].z, Sk); Sk = fmaf(s4.w, kv[l].w, Sk);
            Sq = fmaf(s4.x, qv[l].x, Sq); Sq = fmaf(s4.y, qv[l].y, Sq);
            Sq = fmaf(s4.z, qv[l].z, Sq); Sq = fmaf(s4.w, qv[l].w, Sq);
        }
        const float Skf = group_sum(Sk) * inv_k;
        const float Sqf = group_sum(Sq) * inv_q;
        const int r = 4 * grp + m;
        const float u = beta * (sv[r] - alpha * Skf);
        const float uk = u * inv_k;
#pragma unroll
        for (int l = 0; l < 4; ++l) {
            const float4 s4 = S[4 * m + l];
            float4 x;
            x.x = fmaf(uk, kv[l].x, alpha * s4.x);
            x.y = fmaf(uk, kv[l].y, alpha * s4.y);
            x.z = fmaf(uk, kv[l].z, alpha * s4.z);
            x.w = fmaf(uk, kv[l].w, alpha * s4.w);
            store4_nt(Sblk + m * 128 + l * 32, x);
        }
        if (e == 0) orow[r] = (alpha * Sqf + u * kq) * STEP_SCALE;
    }
    __syncthreads();

    // ---- RMSNorm over the head's 128 outputs, gamma, SiLU(z) --------------
    float oo = 0.f;
    if (tid < 128) oo = orow[tid] * orow[tid];
    if (wave < 2) {
        oo = wave_sum(oo);
        if (lane == 0) red[wave][3] = oo;
    }
    __syncthreads();
    if (tid < 128) {
        const float inv = rsqrt_fast((red[0][3] + red[1][3]) * (1.0f / 128.0f) + d.eps_rms);
        const int64_t e = ((int64_t)n * d.hv + h) * 128 + tid;
        const float zz = ld1(static_cast<const TI *>(p.z) + e);
        const float gm = ld1(static_cast<const TI *>(p.gamma) + tid);
        static_cast<TO *>(p.y)[e] = (TO)(((orow[tid] * inv) * gm) * silu_fast(zz));
    }
}

// hist[n] <- [hist[n][1], hist[n][2], qkv[n]], 8 channels per thread.
template <typename TI>
__global__ __launch_bounds__(256) void step_hist_kernel(const TI *__restrict__ qkv,
                                                        TI *__restrict__ hist, int C, int n_seq)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int per_seq = C / 8;
    if (i >= (int64_t)n_seq * per_seq) return;
    const int64_t n = i / per_seq;
    const int c = (int)(i - n * per_seq) * 8;
    TI *hs = hist + n * 3 * C + c;
    Raw8<TI> r1, r2, x;
    r1.load(hs + C);
    r2.load(hs + 2 * C);
    x.load(qkv + n * C + c);
    r1.store(hs);
    r2.store(hs + C);
    x.store(hs + 2 * C);
}

template <typename TI, typename TO>
static hipError_t launch_step_t(const gdn_shape &s, const StepArgs &a, hipStream_t st)
{
    StepDims d;
    d.hk = s.hk;
    d.hv = s.hv;
    d.G = s.hv / s.hk;
    d.C = 2 * s.hk * 128 + s.hv * 128;
    d.eps_l2 = s.eps_l2;
    d.eps_rms = s.eps_rms;
    hipLaunchKernelGGL((step_kernel<TI, TO>), dim3((unsigned)(s.n_seq * (int64_t)s.hv)), dim3(256),
                       0, st, a, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.hist_out) return e;
    const int64_t threads = (int64_t)s.n_seq * (d.C / 8);
    hipLaunchKernelGGL((step_hist_kernel<TI>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       st, static_cast<const TI *>(a.qkv), static_cast<TI *>(a.hist), d.C, s.n_seq);
    return hipGetLastError();
}

hipError_t launch_step(const gdn_shape &s, const StepArgs &a, hipStream_t st)
{
    if (s.io_dtype == GDN_F16)
        return s.out_dtype == GDN_F16 ? launch_step_t<_Float16, _Float16>(s, a, st)
                                      : launch_step_t<_Float16, float>(s, a, st);
    return s.out_dtype == GDN_F16 ? launch_step_t<float, _Float16>(s, a, st)
                                  : launch_step_t<float, float>(s, a, st);
}

} // namespace gdn
