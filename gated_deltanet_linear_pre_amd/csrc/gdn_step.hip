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
//   - each thread issues the loads of its 64 state elements (row r = t / 2,
//     key half t % 2, sixteen 16-byte loads) first, so they are in flight
//     while the block computes the token's q, k, v and gates;
//   - threads 0..127 each take channel c of the key head's q and k and of the
//     value head's v: 4-tap conv, SiLU, and the three sums q.q, k.k, q.k,
//     reduced over the block (DPP inside a 16-lane row, then LDS);
//   - the state step: each thread forms its half-row dot products S k^ and
//     S q^ over 64 keys, adds its neighbour lane's half (the pair sums in one
//     order), and writes alpha S + u k^T back; o = alpha (S q^) + u (k^.q^)
//     is the same quantity as (alpha S + u k^T) q^ in one pass;
//   - the RMSNorm over the head's 128 outputs and the gated output.
// A second launch shifts the history (every block of a key-head group reads
// the group's q/k history, so no block of the first launch may overwrite it).
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
    __shared__ float gates[2];
    __shared__ float orow[128];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int n = blockIdx.x / d.hv;
    const int h = blockIdx.x - n * d.hv;
    const int j = h / d.G;
    const int C = d.C;

    // ---- issue the state loads first ---------------------------------------
    const int r = tid >> 1, kh = tid & 1;
    float *Srow = p.state + (((int64_t)n * d.hv + h) * 128 + r) * 128 + 64 * kh;
    float4 S[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = reinterpret_cast<const float4 *>(Srow)[i];

    // ---- the token's q, k (key head j) and v (value head h) ---------------
    const TI *qkv = static_cast<const TI *>(p.qkv) + (int64_t)n * C;
    const TI *hist = static_cast<const TI *>(p.hist) + (int64_t)n * 3 * C;
    const TI *cw = static_cast<const TI *>(p.conv_w);
    float sumq = 0.f, sumk = 0.f, sumqk = 0.f;
    if (tid < 128) {
        const int c = tid;
        auto conv_silu = [&](int ch) {
            float acc = ld1(cw + (int64_t)ch * 4 + 0) * ld1(hist + ch);
            acc = fmaf(ld1(cw + (int64_t)ch * 4 + 1), ld1(hist + C + ch), acc);
            acc = fmaf(ld1(cw + (int64_t)ch * 4 + 2), ld1(hist + 2 * C + ch), acc);
            acc = fmaf(ld1(cw + (int64_t)ch * 4 + 3), ld1(qkv + ch), acc);
            return silu_fast(acc);
        };
        const float q = conv_silu(j * 128 + c);
        const float k = conv_silu(d.hk * 128 + j * 128 + c);
        const float v = conv_silu(2 * d.hk * 128 + h * 128 + c);
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
    if (tid == 0) {
        const TI *a = static_cast<const TI *>(p.a);
        const TI *b = static_cast<const TI *>(p.b);
        const float x = ld1(a + (int64_t)n * d.hv + h) + ld1(static_cast<const TI *>(p.dt_bias) + h);
        const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
        const float g = -expf(ld1(static_cast<const TI *>(p.A_log) + h)) * sp;
        gates[0] = expf(g);
        gates[1] = 1.0f / (1.0f + expf(-ld1(b + (int64_t)n * d.hv + h)));
    }
    __syncthreads();
    const float inv_q = rsqrt_fast((red[0][0] + red[1][0]) + d.eps_l2);
    const float inv_k = rsqrt_fast((red[0][1] + red[1][1]) + d.eps_l2);
    const float kq = (red[0][2] + red[1][2]) * inv_q * inv_k;
    const float alpha = gates[0], beta = gates[1];

    // ---- one step of the delta rule on this thread's half row --------------
    float Sk = 0.f, Sq = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float4 kv = *reinterpret_cast<const float4 *>(&sk[64 * kh + 4 * i]);
        const float4 qv = *reinterpret_cast<const float4 *>(&sq[64 * kh + 4 * i]);
        Sk = fmaf(S[i].x, kv.x, Sk); Sk = fmaf(S[i].y, kv.y, Sk);
        Sk = fmaf(S[i].z, kv.z, Sk); Sk = fmaf(S[i].w, kv.w, Sk);
        Sq = fmaf(S[i].x, qv.x, Sq); Sq = fmaf(S[i].y, qv.y, Sq);
        Sq = fmaf(S[i].z, qv.z, Sq); Sq = fmaf(S[i].w, qv.w, Sq);
    }
    // the key halves of a row sit in neighbouring lanes; both add them in
    // the order (lower keys) + (upper keys)
    const float Sk_o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(Sk), 0xB1, 0xF, 0xF, false));
    const float Sq_o = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(Sq), 0xB1, 0xF, 0xF, false));
    const float Skf = (kh == 0 ? Sk + Sk_o : Sk_o + Sk) * inv_k;
    const float Sqf = (kh == 0 ? Sq + Sq_o : Sq_o + Sq) * inv_q;
    const float u = beta * (sv[r] - alpha * Skf);
    const float uk = u * inv_k;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float4 kv = *reinterpret_cast<const float4 *>(&sk[64 * kh + 4 * i]);
        float4 x;
        x.x = fmaf(uk, kv.x, alpha * S[i].x);
        x.y = fmaf(uk, kv.y, alpha * S[i].y);
        x.z = fmaf(uk, kv.z, alpha * S[i].z);
        x.w = fmaf(uk, kv.w, alpha * S[i].w);
        reinterpret_cast<float4 *>(Srow)[i] = x;
    }
    const float o = (alpha * Sqf + u * kq) * STEP_SCALE;
    if (kh == 0) orow[r] = o;
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
    if (e != hipSuccess) return e;
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
