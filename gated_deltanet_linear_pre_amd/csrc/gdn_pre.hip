// gdn_pre.hip -- conv + SiLU + per-key-head L2 norm + gates, with history carry.
//
// "Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1
// (gdn_pre): a 4-tap conv loop with separate handling of the first three
// tokens (taps reach into the carried history) and a history write at the last
// token, then per-key-head sums of squares of q and k.  "round 10 track b: gdn
// vectorization and scan", "variants": four ordered multiply-adds per element,
// SiLU also on the value channels, history rows written back whole.
//
// Per sequence with X = [hist (3 rows); qkv rows]:
//   x~[t][c] = sum_{m=0..3} w[c][m] X[t+m][c],  s = x~ * sigmoid(x~)
//   q^ = s_q / sqrt(|s_q|^2 + eps), k^ likewise, v = s_v
//   g = -exp(A_log) softplus(a + dt_bias),  beta = sigmoid(b)
//   hist <- X[T .. T+2]
//
// gfx950 mapping.  The stage reads about 21 KB and writes about 41 KB per
// token at production width, so it is bound by HBM bandwidth.  Channels come in
// units of one head (128 channels).  A 16-lane DPP row owns one unit, 8
// consecutive channels per lane, so a wave covers 4 units = 512 channels and
// each token row arrives as one contiguous 1 KB (fp16) load instruction.  A
// wave walks a tile of TT tokens.  It loads the TT + 3 rows it needs up front
// (history rows for the first three tokens of a sequence), slides the 4-tap
// window in registers, and reduces the q/k sums of squares with a 4-step DPP
// rotate-add, with no LDS and no barrier.  One extra wave per tile computes the
// gates of its tokens.
//
// History carry without a race: only the tile holding tokens 0..TT-1 of a
// sequence reads the old history (TT >= 3), and that same tile writes the new
// history, for the same channels and lanes, after its reads.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

struct PreDims {
    int hk, hv, C, U;          // U = C / 128 head units
    int n_ug;                  // unit groups of 4 (waves doing conv)
    int tiles_per_seq;
    float eps;
};

template <typename TI, int TT>
__global__ __launch_bounds__(256) void pre_kernel(PreArgs p, PreDims d)
{
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int wg = blockIdx.y * 4 + wave;  // unit group, or the gates wave
    if (wg > d.n_ug) return;
    const int n = blockIdx.x / d.tiles_per_seq;
    const int tile = blockIdx.x - n * d.tiles_per_seq;
    const int64_t s0 = p.cu[n];
    const int64_t T_n = (int64_t)p.cu[n + 1] - s0;
    const int64_t tau0 = (int64_t)tile * TT;
    if (tau0 >= T_n) return;
    const int nt = (int)((T_n - tau0) < TT ? (T_n - tau0) : TT);

    if (wg == d.n_ug) {
        // ---- gates for tokens tau0 .. tau0 + nt - 1 --------------------
        const TI *a = static_cast<const TI *>(p.a);
        const TI *b = static_cast<const TI *>(p.b);
        const TI *A_log = static_cast<const TI *>(p.A_log);
        const TI *dt_bias = static_cast<const TI *>(p.dt_bias);
        const int hv = d.hv;
        for (int idx = lane; idx < nt * hv; idx += 64) {
            const int i = idx / hv;
            const int h = idx - i * hv;
            const int64_t e = (s0 + tau0 + i) * hv + h;
            gates(ld1(a + e), ld1(dt_bias + h), ld1(A_log + h), ld1(b + e), p.g[e], p.beta[e]);
        }
        return;
    }

    // ---- conv + SiLU + norm for one unit per 16-lane row ---------------
    const TI *qkv = static_cast<const TI *>(p.qkv);
    const TI *cw = static_cast<const TI *>(p.conv_w);
    TI *hist = static_cast<TI *>(p.hist);
    const int C = d.C;
    const int u = wg * 4 + (lane >> 4);
    const int l16 = lane & 15;
    const bool active = u < d.U;
    const int c0 = (active ? u : 0) * 128 + l16 * 8;

    // 4 taps of 8 channels = 32 consecutive weights
    float w[8][4];
    {
        float t[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (active) load8(cw + (int64_t)c0 * 4 + k * 8, t);
            else {
#pragma unroll
                for (int e = 0; e < 8; ++e) t[e] = 0.f;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) w[(k * 8 + e) >> 2][(k * 8 + e) & 3] = t[e];
        }
    }

    // window rows X[tau0 + r], r = 0 .. TT+2
    Raw8<TI> win[TT + 3];
#pragma unroll
    for (int r = 0; r < TT + 3; ++r) {
        const int64_t xi = tau0 + r;
        if (!active || r >= nt + 3) win[r].zero();
        else if (xi < 3) win[r].load(hist + ((int64_t)n * 3 + xi) * C + c0);
        else win[r].load(qkv + (s0 + xi - 3) * C + c0);
    }

    // destination of this row's unit
    float *dst;
    int64_t stride;
    const bool is_v = u >= 2 * d.hk;
    if (u < d.hk) { dst = p.qn + u * 128 + l16 * 8; stride = (int64_t)d.hk * 128; }
    else if (!is_v) { dst = p.kn + (u - d.hk) * 128 + l16 * 8; stride = (int64_t)d.hk * 128; }
    else { dst = p.vc + (u - 2 * d.hk) * 128 + l16 * 8; stride = (int64_t)d.hv * 128; }

#pragma unroll
    for (int i = 0; i < TT; ++i) {
        if (i < nt) {  // uniform across the wave
            float s[8];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float acc = conv4(w[e][0], w[e][1], w[e][2], w[e][3], win[i].get(e),
                                        win[i + 1].get(e), win[i + 2].get(e), win[i + 3].get(e));
                s[e] = silu_fast(acc);
                ss = fmaf(s[e], s[e], ss);
            }
            ss = row_sum16(ss);
            const float sc = is_v ? 1.0f : rsqrt_fast(ss + d.eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] *= sc;
            if (active) store8(dst + (s0 + tau0 + i) * stride, s);
        }
    }

    // ---- history carry (tile 0 only; see header) ------------------------
    if (tile == 0 && active) {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int64_t xi = T_n + r;  // row of X that becomes history row r
            Raw8<TI> v;
            if (xi == 0) v = win[0];
            else if (xi == 1) v = win[1];
            else if (xi == 2) v = win[2];
            else v.load(qkv + (s0 + xi - 3) * C + c0);
            v.store(hist + ((int64_t)n * 3 + r) * C + c0);
        }
    }
}

template <typename TI, int TT>
static hipError_t launch_pre_t(const gdn_shape &s, const PreArgs &a, hipStream_t st)
{
    PreDims d;
    d.hk = s.hk;
    d.hv = s.hv;
    d.C = 2 * s.hk * 128 + s.hv * 128;
    d.U = d.C / 128;
    d.n_ug = (d.U + 3) / 4;
    d.tiles_per_seq = (int)((s.max_T + TT - 1) / TT);
    d.eps = s.eps_l2;
    const dim3 grid((unsigned)(s.n_seq * (int64_t)d.tiles_per_seq), (unsigned)((d.n_ug + 1 + 3) / 4));
    hipLaunchKernelGGL((pre_kernel<TI, TT>), grid, dim3(256), 0, st, a, d);
    return hipGetLastError();
}

hipError_t launch_pre(const gdn_shape &s, const PreArgs &a, hipStream_t st)
{
    if (s.io_dtype == GDN_F16) return launch_pre_t<_Float16, PRE_TILE_F16>(s, a, st);
    return launch_pre_t<float, PRE_TILE_F32>(s, a, st);
}

} // namespace gdn
