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
// token at production width, so it is bound by HBM bandwidth; what sets its
// speed is how whole its memory instructions are.  Channels come in units of
// one head (128 channels).  A 16-lane DPP row owns one unit: lane l takes
// channels 4l..4l+3 and 64+4l..64+4l+3, so each load or store instruction of
// a wave covers whole 64-channel runs of its 4 units (whole cache lines; with
// 8 consecutive channels per lane the fp32 stores each wrote half of every
// line they touched, and ran 15% slower).  A block of 4 waves takes a tile of
// 4 x 4 tokens of one group of 4 units; each wave loads the 4 + 3 rows its 4
// tokens need (history rows for the first three tokens of a sequence; the
// 3-row overlap between waves is an L1/L2 hit), slides the 4-tap window in
// registers, and reduces the q/k sums of squares with a 4-step DPP rotate-add,
// with no LDS and no barrier.  One extra row of blocks computes the gates.
// Every wave issues all its loads before its first store and waits for them
// once: with loads and stores outstanding together each later use of a loaded
// value would wait for the stores too.  The outputs go out as non-temporal
// stores.
//
// History carry without a race: only the first wave of a sequence reads the
// old history (its rows 0..2 are X rows 0..2, and every later wave starts at
// X row 4 or beyond), and that same wave writes the new history, for the same
// channels and lanes, after its reads.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

struct PreDims {
    int hk, hv, C, U;          // U = C / 128 head units
    int n_ug;                  // unit groups of 4 (blockIdx.x of the conv blocks)
    int tiles_per_seq;
    int64_t n_tiles;           // n_seq x tiles_per_seq (grid y and z)
    float eps;
};

// One block per (unit group of 4 units, tile of 4 TW tokens); wave w takes the
// tile's tokens w TW .. w TW + TW - 1.  blockIdx.x == n_ug: the tile's gates.
// The unit group is the fast grid index, so the blocks resident at one time
// read whole token rows (measured: 25.5 us per production layer, against 28.1
// with the tile as the fast index, and 27.4 with runs of tiles kept on one XCD).
template <typename TI, int TW>
__global__ __launch_bounds__(256) void pre_kernel(PreArgs p, PreDims d)
{
    static_assert(TW >= 3, "only the first wave of a sequence may read the history");
    constexpr int TT = 4 * TW;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    // tile index over grid y and z (grid y holds at most 65535 blocks)
    const int64_t bxl = (int64_t)blockIdx.z * gridDim.y + blockIdx.y;
    if (bxl >= d.n_tiles) return;
    const int bx = (int)bxl;
    const int n = bx / d.tiles_per_seq;
    const int tile = bx - n * d.tiles_per_seq;
    const int64_t s0 = p.cu[n];
    const int64_t T_n = (int64_t)p.cu[n + 1] - s0;
    const int64_t tau0 = (int64_t)tile * TT;
    if (tau0 >= T_n) return;

    if ((int)blockIdx.x == d.n_ug) {
        // ---- gates of the tile's tokens, GB per thread per round; every
        // load of a round is issued before the round's first store
        constexpr int GB = 4;
        const TI *a = static_cast<const TI *>(p.a);
        const TI *b = static_cast<const TI *>(p.b);
        const TI *A_log = static_cast<const TI *>(p.A_log);
        const TI *dt_bias = static_cast<const TI *>(p.dt_bias);
        const int hv = d.hv;
        const int total = (int)((T_n - tau0) < TT ? (T_n - tau0) : TT) * hv;
        for (int r0 = 0; r0 < total; r0 += 256 * GB) {  // uniform
            float av[GB], bv[GB], dv[GB], lv[GB];
            int64_t e[GB];
#pragma unroll
            for (int k = 0; k < GB; ++k) {
                const int idx = min(r0 + 256 * k + tid, total - 1);
                const int i = idx / hv, h = idx - i * hv;
                e[k] = (s0 + tau0 + i) * hv + h;
                av[k] = ld1(a + e[k]);
                bv[k] = ld1(b + e[k]);
                dv[k] = ld1(dt_bias + h);
                lv[k] = ld1(A_log + h);
            }
            wait_vmem_all();
#pragma unroll
            for (int k = 0; k < GB; ++k) {
                float g, bt;
                gates(av[k], dv[k], lv[k], bv[k], g, bt);
                if (r0 + 256 * k + tid < total) {
                    p.g[e[k]] = g;
                    p.beta[e[k]] = bt;
                }
            }
        }
        return;
    }

    // ---- conv + SiLU + norm for one unit per 16-lane row ---------------
    const int64_t t0 = tau0 + wave * TW;  // this wave's first token
    if (t0 >= T_n) return;                // uniform across the wave
    const int nt = (int)((T_n - t0) < TW ? (T_n - t0) : TW);
    const TI *qkv = static_cast<const TI *>(p.qkv);
    const TI *cw = static_cast<const TI *>(p.conv_w);
    TI *hist = static_cast<TI *>(p.hist);
    const int C = d.C;
    const int u = (int)blockIdx.x * 4 + (lane >> 4);
    const int l16 = lane & 15;
    const bool active = u < d.U;
    // lane l16 of the row owns channels 4 l16 .. + 3 (values 0..3) and
    // 64 + 4 l16 .. + 3 (values 4..7) of its unit, so that every load and
    // store instruction covers whole 64-channel runs of each of its 4 units
    const int c0 = (active ? u : 0) * 128 + l16 * 4;  // valid for every lane

    // Every load is unconditional (rows past the last token repeat its row;
    // inactive rows read unit 0) and all are issued before the first store.
    // 4 taps of 4 channels = 16 consecutive weights, twice
    float w[8][4];
    {
        float t[4][8];
#pragma unroll
        for (int k = 0; k < 4; ++k) load8(cw + (int64_t)(c0 + 64 * (k >> 1)) * 4 + (k & 1) * 8, t[k]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) w[(k * 8 + e) >> 2][(k * 8 + e) & 3] = t[k][e];
    }
    // window rows X[t0 + r], r = 0 .. TW + 2 (history rows for X index < 3)
    Raw8<TI> win[TW + 3];
#pragma unroll
    for (int r = 0; r < TW + 3; ++r) {
        const int64_t xi = t0 + (r < nt + 3 ? r : nt + 2);
        const TI *src = xi < 3 ? hist + ((int64_t)n * 3 + xi) * C + c0 : qkv + (s0 + xi - 3) * C + c0;
        win[r].load_split(src);
    }
    wait_vmem_all();

    // destination of this row's unit
    float *dst;
    int64_t stride;
    const bool is_v = u >= 2 * d.hk;
    if (u < d.hk) { dst = p.qn + u * 128 + l16 * 4; stride = (int64_t)d.hk * 128; }
    else if (!is_v) { dst = p.kn + (u - d.hk) * 128 + l16 * 4; stride = (int64_t)d.hk * 128; }
    else { dst = p.vc + (u - 2 * d.hk) * 128 + l16 * 4; stride = (int64_t)d.hv * 128; }

    auto token = [&](int i) {
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
        if (active) store8_split_nt(dst + (s0 + t0 + i) * stride, s);
    };
    if (nt == TW) {
#pragma unroll
        for (int i = 0; i < TW; ++i) token(i);
    } else {
#pragma unroll
        for (int i = 0; i < TW; ++i)
            if (i < nt) token(i);  // uniform across the wave
    }

    // ---- history carry (the sequence's first wave only; see header) -----
    if (t0 == 0 && active) {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
            const int64_t xi = T_n + r;  // row of X that becomes history row r
            Raw8<TI> v;
            if (xi == 0) v = win[0];
            else if (xi == 1) v = win[1];
            else if (xi == 2) v = win[2];
            else v.load_split(qkv + (s0 + xi - 3) * C + c0);
            v.store_split(hist + ((int64_t)n * 3 + r) * C + c0);
        }
    }
}

template <typename TI, int TW>
static hipError_t launch_pre_t(const gdn_shape &s, const PreArgs &a, hipStream_t st)
{
    PreDims d;
    d.hk = s.hk;
    d.hv = s.hv;
    d.C = 2 * s.hk * 128 + s.hv * 128;
    d.U = d.C / 128;
    d.n_ug = (d.U + 3) / 4;
    d.tiles_per_seq = (int)((s.max_T + 4 * TW - 1) / (4 * TW));
    d.n_tiles = (int64_t)s.n_seq * d.tiles_per_seq;
    d.eps = s.eps_l2;
    if (d.n_tiles == 0) return hipSuccess;
    const unsigned gy = (unsigned)(d.n_tiles < 65535 ? d.n_tiles : 65535);
    const unsigned gz = (unsigned)((d.n_tiles + gy - 1) / gy);
    const dim3 grid((unsigned)(d.n_ug + 1), gy, gz);
    hipLaunchKernelGGL((pre_kernel<TI, TW>), grid, dim3(256), 0, st, a, d);
    return hipGetLastError();
}

hipError_t launch_pre(const gdn_shape &s, const PreArgs &a, hipStream_t st)
{
    if (s.io_dtype == GDN_F16) return launch_pre_t<_Float16, PRE_WAVE_TOKENS>(s, a, st);
    return launch_pre_t<float, PRE_WAVE_TOKENS>(s, a, st);
}

} // namespace gdn
