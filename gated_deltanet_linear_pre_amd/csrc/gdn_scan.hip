// gdn_scan.hip -- the gated delta rule on an fp32 state, in 16-token chunks on
// fp16 MFMA with split (hi + lo) operands.
//
// "Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1
// (gdn_scan_r findings): one state per value head, updated token by token in
// the same pass that forms the dot products against the old state; section 2:
// a token-blocked run must equal the single pass.
//
// The recurrence, per value head h (key head j = h / G), state S (dv x dk):
//   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
//   o_t = S_t q_t / sqrt(dk),  alpha_t = exp(g_t).
// Over a chunk of 16 tokens starting from state S0, with
//   D[t][s] = exp(g_{s+1} + ... + g_t)    (decay from just after s to t, <= 1)
//   Lam_t   = exp(g_0 + ... + g_t)        (decay from the chunk start)
// the writes u_t = beta_t (v_t - alpha_t S_{t-1} k_t) solve a unit lower
// triangular system, and the outputs and the next state follow:
//   (I + A) U = diag(beta) (V - diag(Lam) P),  A[t][s] = beta_t D[t][s] k_t.k_s (s<t)
//   O  = (diag(Lam) R + M U) / sqrt(dk),       M[t][s] = D[t][s] q_t.k_s     (s<=t)
//   S' = Lam_last S0 + sum_s D[last][s] u_s k_s^T
// with P = K S0^T, R = Q S0^T (tokens x value channels).  This is exact
// algebra of the recurrence (unroll S_t = Lam_t S0 + sum_{s<=t} D[t][s] u_s k_s^T).
// Every decay is formed as exp of a sum of at most 16 log decays, never as a
// ratio of two cumulative products, so nothing overflows or cancels.
//
// Precision.  Every product of the chunk step runs on fp16 MFMA with fp32
// accumulation, each fp32 operand x split into hi = fp16(x) and
// lo = fp16(x - hi): x*y ~ hi_x hi_y + hi_x lo_y + lo_x hi_y, good to about
// 2^-21 relative per product (the dropped lo_x lo_y term and the rounding of
// lo).  k, q and the state are scaled by 16 (exactly); the state stays fp32
// in the MFMA accumulators.  The low halves of the operands whose scale
// follows the data (state, B, U w, U) are carried x 2^10 in products of their
// own (see LO_SCALE), so the split stays accurate for small values too.
// Range: |16 state|, |B|, |U w| and |U| below 65504; past it a scaled low half
// overflows and the results turn to inf/NaN.
//
// gfx950 mapping.
// * gdn_scan_prep (parallel over sequence x chunk x key head):
//   - k.k and q.k of the chunk on fp32 MFMA, once per key head;
//   - K, Q (16 tokens x 128 keys) and K^T split into hi/lo fp16 and laid out
//     in the exact per-lane operand order of the chunk kernel's MFMAs
//     ("key-head slot", 24 KB per chunk);
//   - per value head: the decays, T = (I + A)^-1 by forward substitution
//     (one column per lane, in registers), M, Lam, beta and the last-row
//     decays, T and M split and laid out as MFMA operands ("value-head slot").
// * gdn_scan_chunk (sequential over chunks): a block owns 32 value channels
//   of one (sequence, value head) in two row groups of 16; each row group's
//   state (16 channels x 128 keys) is split by key halves over a pair of
//   compute waves, each holding its 16 x 64 quarter in MFMA accumulator
//   layout (16 VGPRs/lane).  Per chunk and compute wave:
//     K S^T, Q S^T     6 + 6    v_mfma_f32_16x16x32_f16 (3 split terms x 2 key steps)
//     U = T B          1 + 1    16x16x32 (hi.hi + lo.hi) + 16x16x16 (hi.lo)
//     S' = Lam_last S + K^T (D U)  4 + 4  same, per key block
//   (over the 16 tokens of a chunk, two split terms share one 16x16x32 product:
//   its contraction runs over the pair (term, token)).  The two waves of a
//   pair add their partial K S^T through LDS in the same order, so both form
//   the same U; this exchange and one barrier per chunk are the only
//   synchronisation on the recurrence.
//   Every product consumes the accumulator layout the previous one produced
//   (the contraction index is permuted consistently, and the prep kernel packs
//   K, Q and K^T in that order), so the state never leaves registers.
//   A copy wave moves the chunk operands from global memory into LDS three
//   chunks ahead (four LDS copies).  An output wave forms O = Lam R + M U
//   (1 + 1 products per row group) one step behind, from the partial Q S^T,
//   U, Lam and M the compute waves leave in LDS, so the outputs stay off the
//   recurrence's path.  In the layer path with fp16 inputs a v wave forms v
//   of the block's channels from the raw qkv rows the copy wave brings (conv
//   with the history, SiLU: the pre stage's expressions) and carries their
//   history, so the fp32 v never goes through memory.
// * Block order: longest sequence first (its chain of chunk steps is the
//   critical path of a packed batch), and XCD-aware: blocks are dealt
//   round-robin to the 8 XCDs, so inside each sequence's range the index is
//   permuted to give each XCD whole key-head groups, whose key-head slots are
//   then shared in one L2.
//
// Determinism: fixed-order MFMA chains, no atomics.  Splitting a sequence at a
// multiple of 16 tokens gives bit-identical results; other split points agree
// within rounding (the chunk grid moves).
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int CT = 16;           // tokens per chunk
constexpr int KS = 132;          // LDS row stride of the fp32 K/Q chunk in prep
constexpr float KQ_SCALE = 16.f; // k and q scale before the fp16 split (exact)
constexpr float SCALE = 0.08838834764831845f;  // 1 / sqrt(128)

// key-head slot, in fp16 elements
constexpr int KH_KP = 0;     // [4 key steps][2 hi/lo][64 lanes][8]  K for K S^T
constexpr int KH_QP = 4096;  // same for Q
constexpr int KH_KT = 8192;  // [8 key blocks][64 lanes][hi 4, lo 4]  K^T for the update
static_assert(SCAN_KH_FLOATS * 2 == 12288, "key-head slot size");
// value-head slot, in floats
constexpr int VH_TP = 0;       // [64 lanes][hi 4, lo 4] fp16  T   (256 floats)
constexpr int VH_MP = 256;     // [64 lanes][hi 4, lo 4] fp16  M   (256 floats)
constexpr int VH_LAM = 512;    // Lam_t / 256 (k, q and the state each carry a factor 16)
constexpr int VH_BETA = 528;   // beta_t (0 past the chunk's end)
constexpr int VH_W = 544;      // D[last][s] (0 past the end)
constexpr int VH_LAST = 560;   // Lam_last
static_assert(SCAN_SLOT_FLOATS >= 564 && SCAN_SLOT_FLOATS % 4 == 0, "value-head slot size");

__device__ __forceinline__ f4 mfma_f32(float a, float b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// D += A B, 16x16x16: lane l supplies A[l%16][4(l/16)+e] and B[4(l/16)+e][l%16];
// D[4(l/16)+r][l%16] comes back in component r.
// A product never takes the result of a product of the other shape as its
// accumulator: the compiler leaves too few wait states between a 16x16x32
// and a 16x16x16 that reads its result as C on gfx950 (measured: stale rows
// in the result).  Chains stay within one shape; the two shapes meet only
// through a VALU add, or the 16-deep term runs as a zero-padded 16x16x32.
__device__ __forceinline__ f4 mfma_k16(h4 a, h4 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// 16x16x32: A[l%16][8(l/16)+e], B[8(l/16)+e][l%16], same D layout.
__device__ __forceinline__ f4 mfma_k32(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// x = hi + lo + O(2^-22 |x|): hi = fp16(x) rounded toward zero, lo = fp16(x - hi)
// rounded to nearest (|lo| < ulp(hi), so lo keeps 11 more bits of x).
// x - hi is exact in fp32 and is formed by one mixed-precision multiply-add
// (v_fma_mix takes the fp16 hi as it is); m1 = -1 comes in at run time so
// that the compiler keeps that form instead of converting hi back first.
// hi comes from the conversion intrinsic, which the compiler neither fuses
// with the product that made x nor recomputes: both uses of hi (the MFMA
// operand and the lo) see one value, and the pair sums to x.  (A plain
// fp16 cast may be fused with a preceding multiply into one rounding in one
// use and not in the other.)  Plain compiler-visible code on purpose: these
// values feed MFMA operands, and the compiler inserts the VALU/MFMA hazard
// waits only for code it sees.
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t hi_pair(float x0, float x1)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
}
__device__ __forceinline__ uint32_t lo_pair(uint32_t hi2, float x0, float x1, float m1)
{
    const h2 h = __builtin_bit_cast(h2, hi2);
    const h2 r = {(_Float16)__builtin_fmaf((float)h[0], m1, x0),
                  (_Float16)__builtin_fmaf((float)h[1], m1, x1)};
    return __builtin_bit_cast(uint32_t, r);
}
// For operands whose scale follows the data (the state, B = beta (v - Lam P),
// U w, U) the low half is carried multiplied by LO_SCALE = 2^10 and enters
// its own product, which is scaled back (exactly) by 2^-10 when it is added:
// lo stays a normal fp16 number down to |x| ~ 2^-13 instead of 2^-3, so the
// split keeps ~22 bits over 29 binades of magnitude, and past the top of the
// fp16 range (|x| > 65504 + 2^6) the scaled low half overflows to inf, which
// the results show.  ms = -LO_SCALE at run time (see lo_pair).
constexpr float LO_SCALE = 1024.f;
constexpr float LO_UNSCALE = 1.f / 1024.f;
__device__ __forceinline__ uint32_t lo_pair_s(uint32_t hi2, float x0, float x1, float ms)
{
    const h2 h = __builtin_bit_cast(h2, hi2);
    const h2 r = {(_Float16)__builtin_fmaf((float)h[0], ms, x0 * LO_SCALE),
                  (_Float16)__builtin_fmaf((float)h[1], ms, x1 * LO_SCALE)};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ void split4s(const f4 x, h4 &hi, h4 &lo, float ms)
{
    u2 h, l;
    h[0] = hi_pair(x[0], x[1]);
    h[1] = hi_pair(x[2], x[3]);
    l[0] = lo_pair_s(h[0], x[0], x[1], ms);
    l[1] = lo_pair_s(h[1], x[2], x[3], ms);
    hi = __builtin_bit_cast(h4, h);
    lo = __builtin_bit_cast(h4, l);
}
__device__ __forceinline__ void split8s(const f4 a, const f4 b, h8 &hi, h8 &lo, float ms)
{
    u4 h, l;
    h[0] = hi_pair(a[0], a[1]);
    h[1] = hi_pair(a[2], a[3]);
    h[2] = hi_pair(b[0], b[1]);
    h[3] = hi_pair(b[2], b[3]);
    l[0] = lo_pair_s(h[0], a[0], a[1], ms);
    l[1] = lo_pair_s(h[1], a[2], a[3], ms);
    l[2] = lo_pair_s(h[2], b[0], b[1], ms);
    l[3] = lo_pair_s(h[3], b[2], b[3], ms);
    hi = __builtin_bit_cast(h8, h);
    lo = __builtin_bit_cast(h8, l);
}
__device__ __forceinline__ void split4(const f4 x, h4 &hi, h4 &lo, float m1)
{
    u2 h, l;
    h[0] = hi_pair(x[0], x[1]);
    h[1] = hi_pair(x[2], x[3]);
    l[0] = lo_pair(h[0], x[0], x[1], m1);
    l[1] = lo_pair(h[1], x[2], x[3], m1);
    hi = __builtin_bit_cast(h4, h);
    lo = __builtin_bit_cast(h4, l);
}
__device__ __forceinline__ void split8(const f4 a, const f4 b, h8 &hi, h8 &lo, float m1)
{
    u4 h, l;
    h[0] = hi_pair(a[0], a[1]);
    h[1] = hi_pair(a[2], a[3]);
    h[2] = hi_pair(b[0], b[1]);
    h[3] = hi_pair(b[2], b[3]);
    l[0] = lo_pair(h[0], a[0], a[1], m1);
    l[1] = lo_pair(h[1], a[2], a[3], m1);
    l[2] = lo_pair(h[2], b[0], b[1], m1);
    l[3] = lo_pair(h[3], b[2], b[3], m1);
    hi = __builtin_bit_cast(h8, h);
    lo = __builtin_bit_cast(h8, l);
}

// (a, b) as one 8-element operand: in a 16x16x32 product the contraction
// positions 8(l/16) + e take a for e < 4 and b for e >= 4, so
// mfma_k32(cat(x1, x2), cat(y1, y2)) = x1 y1 + x2 y2 over 16-deep halves.
__device__ __forceinline__ h8 cat(h4 a, h4 b)
{
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ h4 lo_half(h8 a) { return __builtin_shufflevector(a, a, 0, 1, 2, 3); }

// Slot of chunk c of sequence n (cu0 = cu[n]); injective, and below
// total_T / 16 + n_seq.
__device__ __forceinline__ int64_t chunk_slot(int cu0, int n, int c)
{
    return (int64_t)(cu0 >> 4) + c + n;
}

struct PrepDims {
    int hk, hv, G, n_chunk_max;
    float m1;         // -1 (see lo_pair)
    int64_t vh_base;  // float offset of the value-head slots in the workspace
    int C;            // channels of a qkv row (fused layer prep)
    float eps_l2;     // (fused layer prep)
};

// LDS of the prep step of one (chunk, key head)
struct PrepShared {
    float sK[CT][KS];           // k and q of the chunk (zero past the end)
    float sQ[CT][KS];
    f4 sPart[2][4][64];         // per-wave partial K K^T, K Q^T
    float sA[4][CT][CT + 1];
    float sTm[4][CT][CT + 1];
    float sGB[4][2][CT];
};

// Everything after k and q of the chunk are in LDS: the key-head slot and the
// value-head slots.  load_gb(gh, g, b) gives lane t % 16 the g and beta of
// token t of value head gh of the group (0 past the end); g_next, b_next
// already hold those of this wave's first head.
template <class GB>
__device__ __forceinline__ void prep_body(PrepShared &sm, float *ws, const PrepDims &d, int j,
                                          int64_t slot, int nv, float g_next, float b_next,
                                          GB load_gb)
{
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, kk = lane >> 4;
    const int hk = d.hk, hv = d.hv;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};
    auto &sK = sm.sK;
    auto &sQ = sm.sQ;
    auto &sPart = sm.sPart;
    auto &sA = sm.sA;
    auto &sTm = sm.sTm;
    auto &sGB = sm.sGB;
    struct {
        float *ws;
    } p{ws};

    // ---- key-head slot: K, Q and K^T split and packed in operand order ----
    _Float16 *kh = reinterpret_cast<_Float16 *>(p.ws + (slot * hk + j) * SCAN_KH_FLOATS);
    {
        // K S^T step s, lane L = 16 kk + t holds keys 32 s + 16 (e / 4) + 4 kk + e % 4
        const int s = wave, L = lane, t = l16;
        f4 ka, kb, qa, qb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ka[e] = KQ_SCALE * sK[t][32 * s + 4 * kk + e];
            kb[e] = KQ_SCALE * sK[t][32 * s + 16 + 4 * kk + e];
            qa[e] = KQ_SCALE * sQ[t][32 * s + 4 * kk + e];
            qb[e] = KQ_SCALE * sQ[t][32 * s + 16 + 4 * kk + e];
        }
        h8 khi, klo, qhi, qlo;
        split8(ka, kb, khi, klo, d.m1);
        *reinterpret_cast<h8 *>(kh + KH_KP + ((s * 2 + 0) * 64 + L) * 8) = khi;
        *reinterpret_cast<h8 *>(kh + KH_KP + ((s * 2 + 1) * 64 + L) * 8) = klo;
        split8(qa, qb, qhi, qlo, d.m1);
        *reinterpret_cast<h8 *>(kh + KH_QP + ((s * 2 + 0) * 64 + L) * 8) = qhi;
        *reinterpret_cast<h8 *>(kh + KH_QP + ((s * 2 + 1) * 64 + L) * 8) = qlo;
        // this wave's 32 keys of K K^T and K Q^T (x256) from the same split
        // operands: as A and as B operand, lane (t, kk) holds the same K[t][keys]
        sPart[0][wave][lane] = (mfma_k32(khi, khi, z4) + mfma_k32(khi, klo, z4)) + mfma_k32(klo, khi, z4);
        sPart[1][wave][lane] = (mfma_k32(khi, qhi, z4) + mfma_k32(khi, qlo, z4)) + mfma_k32(klo, qhi, z4);
        // K^T block b, lane L = 16 kk + m holds K[4 kk + e][16 b + m]
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            const int b = 2 * wave + m2;
            f4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = KQ_SCALE * sK[4 * kk + e][16 * b + l16];
            h4 h, l;
            split4(x, h, l, d.m1);
            *reinterpret_cast<h8 *>(kh + KH_KT + (b * 64 + L) * 8) = cat(h, l);
        }
    }

    __syncthreads();
    // k_t.k_u and k_t.q_u summed over the four key steps in one order by every
    // wave; lane (u = l16, kk) holds component r = (t - 4 kk): KK4[r] =
    // k_{4 kk + r}.k_{l16} and KQ4[r] = k_{4 kk + r}.q_{l16}
    f4 KK4, KQ4;
    {
        const float unscale = 1.f / (KQ_SCALE * KQ_SCALE);
        KK4 = (((sPart[0][0][lane] + sPart[0][1][lane]) + sPart[0][2][lane]) + sPart[0][3][lane]) * unscale;
        KQ4 = (((sPart[1][0][lane] + sPart[1][1][lane]) + sPart[1][2][lane]) + sPart[1][3][lane]) * unscale;
    }

    // ---- value-head slots ------------------------------------------------
    for (int gh = wave; gh < d.G; gh += 4) {
        const int h = j * d.G + gh;
        float *vs = p.ws + d.vh_base + (slot * hv + h) * SCAN_SLOT_FLOATS;
        // the head's 16 g and beta, uniform across the wave (0 past the end)
        const float g_own = g_next, b_own = b_next;
        if (gh + 4 < d.G) load_gb(gh + 4, g_next, b_next);
        // the 16 g and beta through this wave's LDS row: every lane reads the
        // g row as uniform VGPRs, and its own 4-token pieces of g and beta
        if (lane < CT) {
            sGB[wave][0][lane] = g_own;
            sGB[wave][1][lane] = b_own;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float gv[CT];
#pragma unroll
        for (int i = 0; i < CT / 4; ++i) {
            const f4 x = *reinterpret_cast<const f4 *>(&sGB[wave][0][4 * i]);
            gv[4 * i] = x[0]; gv[4 * i + 1] = x[1]; gv[4 * i + 2] = x[2]; gv[4 * i + 3] = x[3];
        }
        const f4 g4 = *reinterpret_cast<const f4 *>(&sGB[wave][0][4 * kk]);  // g[4 kk + i]
        const f4 b4 = *reinterpret_cast<const f4 *>(&sGB[wave][1][4 * kk]);  // beta[4 kk + i]
        // Every decay is the exp of a direct sum of the log decays it spans.
        // A[t][s] = beta_t D[t][s] k_t.k_s (s < t): lane (s = l16, kk) takes
        // t = 4 kk .. 4 kk + 3, summing g over (s, 4 kk] once and then one
        // term per t.
        {
            const int s0 = l16;
            float acc = 0.f;
#pragma unroll
            for (int r = 1; r < CT; ++r) acc += (r > s0 && r <= 4 * kk) ? gv[r] : 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * kk + i;
                if (i > 0) acc += t > s0 ? g4[i] : 0.f;
                sA[wave][t][s0] = (t < nv && s0 < t) ? b4[i] * exp_fast(acc) * KK4[i] : 0.f;
            }
        }
        // M[t][s] = D[t][s] q_t.k_s (s <= t) in operand order: lane L = 16 kk + t
        // holds s = 4 kk + e; the sum over (4 kk + 3, t] first, then one term
        // per step down in s
        {
            const int t = l16;
            float acc = 0.f;
#pragma unroll
            for (int r = 1; r < CT; ++r) acc += (r >= 4 * kk + 4 && r <= t) ? gv[r] : 0.f;
            f4 mv;
#pragma unroll
            for (int e = 3; e >= 0; --e) {
                const int s0 = 4 * kk + e;
                if (e < 3) acc += (s0 + 1 <= t) ? g4[e + 1] : 0.f;
                mv[e] = (t < nv && s0 <= t) ? exp_fast(acc) * KQ4[e] : 0.f;
            }
            h4 hi, lo;
            split4(mv, hi, lo, d.m1);
            *reinterpret_cast<h8 *>(reinterpret_cast<_Float16 *>(vs + VH_MP) + lane * 8) = cat(hi, lo);
        }
        if (lane < CT) {
            const int t = lane;
            float lam = 0.f, wdec = 0.f;
#pragma unroll
            for (int r = 0; r < CT; ++r) {
                lam += r <= t ? gv[r] : 0.f;
                wdec += (r > t && r < nv) ? gv[r] : 0.f;
            }
            // Lam_t and D[last][t] weight this chunk's terms only; Lam_last
            // multiplies the whole state every chunk, so it takes the
            // correctly rounded exp
            vs[VH_LAM + t] = t < nv ? exp_fast(lam) * (1.f / (KQ_SCALE * KQ_SCALE)) : 0.f;
            vs[VH_BETA + t] = b_own;
            vs[VH_W + t] = t < nv ? exp_fast(wdec) : 0.f;
            if (t == nv - 1) vs[VH_LAST] = expf(lam);
        }
        // the wave's A writes must land before its lanes read them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < CT) {
            // T = (I + A)^-1 by forward substitution; lane s keeps column s
            const int s = lane;
            float Tc[CT];
#pragma unroll
            for (int t = 0; t < CT; ++t) {
                // four interleaved partial sums shorten the dependent chain
                float acc[4] = {(t == s) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int r = 0; r < t; ++r) acc[r & 3] = fmaf(-sA[wave][t][r], Tc[r], acc[r & 3]);
                Tc[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            }
#pragma unroll
            for (int t = 0; t < CT; ++t) sTm[wave][t][s] = Tc[t];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
            // T in operand order: lane L = 16 kk + t holds T[t][4 kk + e]
            f4 tv;
#pragma unroll
            for (int e = 0; e < 4; ++e) tv[e] = sTm[wave][l16][4 * kk + e];
            h4 hi, lo;
            split4(tv, hi, lo, d.m1);
            *reinterpret_cast<h8 *>(reinterpret_cast<_Float16 *>(vs + VH_TP) + lane * 8) = cat(hi, lo);
        }
        __builtin_amdgcn_wave_barrier();
    }
}

constexpr int CHUNK_PREP_THREADS = 256;

__global__ __launch_bounds__(256) void scan_prep_kernel(ScanArgs p, PrepDims d)
{
    __shared__ __attribute__((aligned(16))) PrepShared sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15;
    const int n = blockIdx.x / d.n_chunk_max;
    const int c = blockIdx.x - n * d.n_chunk_max;
    const int j = blockIdx.y;
    const int cu0 = p.cu[n];
    const int T_n = p.cu[n + 1] - cu0;
    if (c * CT >= T_n) return;
    const int nv = min(CT, T_n - c * CT);
    const int64_t tb = (int64_t)cu0 + c * CT;
    const int hk = d.hk, hv = d.hv;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};

    // g and beta of this wave's first value head, lane t % 16 holding token t
    // (requested first, so their latency overlaps the staging below)
    auto load_gb = [&](int gh, float &gl, float &bl) {
        const int64_t e = (tb + min(l16, nv - 1)) * hv + j * d.G + gh;
        gl = l16 < nv ? p.g[e] : 0.f;
        bl = l16 < nv ? p.beta[e] : 0.f;
    };
    float g_next = 0.f, b_next = 0.f;
    if (wave < d.G) load_gb(wave, g_next, b_next);

    // stage the chunk's k and q rows of key head j (zero past the end)
#pragma unroll
    for (int f2 = 0; f2 < 2; ++f2) {
        const int f = tid + 256 * f2;
        const int t = f >> 5, col = (f & 31) * 4;
        const int tc = min(t, nv - 1);
        const int64_t off = ((tb + tc) * hk + j) * 128 + col;
        const f4 kv = *reinterpret_cast<const f4 *>(p.kn + off);
        const f4 qv = *reinterpret_cast<const f4 *>(p.qn + off);
        *reinterpret_cast<f4 *>(&sm.sK[t][col]) = t < nv ? kv : z4;
        *reinterpret_cast<f4 *>(&sm.sQ[t][col]) = t < nv ? qv : z4;
    }
    __syncthreads();
    prep_body(sm, p.ws, d, j, chunk_slot(cu0, n, c), nv, g_next, b_next, load_gb);
}

struct ChunkDims {
    int hk, hv, G, n_seq;
    float m1;         // -1 (see lo_pair)
    float ms;         // -LO_SCALE (see lo_pair_s)
    int64_t vh_base;
};

// The sequence of rank r when the sequences are sorted by decreasing length
// (ties by index).  Lane l < n_seq takes sequence l and counts the sequences
// that come before it; every wave computes the same answer.
constexpr int SEQ_RANK_MAX = 64;
__device__ __forceinline__ int seq_of_rank(const int32_t *cu, int n_seq, int r)
{
    const int lane = threadIdx.x & 63;
    const int len = lane < n_seq ? cu[lane + 1] - cu[lane] : -1;
    int before = 0;
    for (int m = 0; m < n_seq; ++m) {
        const int lm = __shfl(len, m);
        before += (lm > len || (lm == len && m < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(lane < n_seq && before == r);
    return hit ? __builtin_ctzll(hit) : r;
}

// A block owns 32 value channels of one (sequence, value head): two row groups
// of 16 channels, and each row group is shared by a pair of waves, one per half
// of the 128 keys; each of these four compute waves holds its 16 x 64 quarter
// of the block's state.  A fifth wave only copies operands into LDS, and a
// sixth forms the outputs from what the compute waves leave in LDS.  With
// RAW_V a seventh wave forms v of the block's channels from the raw fp16 qkv
// rows (conv with the history, SiLU) instead of the copy wave bringing vc.
constexpr int CHUNK_WAVES = 4;                       // compute waves: 2 row groups x 2 key halves
constexpr int chunk_threads(bool raw_v) { return 64 * (CHUNK_WAVES + 2 + (raw_v ? 1 : 0)); }
constexpr int CHUNK_ROWS = 32;                       // value channels per block
constexpr int NBUF = 4;                              // LDS copies of a chunk's operands

// Block-wide barrier ordering LDS only: global copies in flight stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The copy and output waves' side of the same barrier.  They write LDS only
// through the copies, whose completion the copy wave waits for explicitly
// (vmcnt) before arriving; their own LDS reads are waited for here.  The
// empty asm statements keep the compiler from moving memory operations
// across the barrier.  (The fenced form above would also wait for global
// stores and loads in flight, which the compute waves do not need.)
__device__ __forceinline__ void side_barrier()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

template <bool RAW_V>
__global__ __launch_bounds__(chunk_threads(RAW_V)) void scan_chunk_kernel(ScanArgs p, ChunkDims d,
                                                                         VRawArgs vr)
{
    // operands of four chunks in flight: key-head slot, value-head slot, v
    __shared__ __attribute__((aligned(16))) float sKH[NBUF][SCAN_KH_FLOATS];
    __shared__ __attribute__((aligned(16))) float sVH[NBUF][SCAN_SLOT_FLOATS];
    __shared__ __attribute__((aligned(16))) float sV[NBUF][CT][CHUNK_ROWS];
    // RAW_V: raw fp16 qkv rows of the block's value channels, per chunk, and
    // the old history rows of those channels
    constexpr int RAW_BUF = RAW_V ? NBUF : 1;
    __shared__ __attribute__((aligned(16))) _Float16 sRaw[RAW_BUF][CT][CHUNK_ROWS];
    __shared__ __attribute__((aligned(16))) _Float16 sRawH[3][CHUNK_ROWS];
    // partial K S^T and Q S^T of every compute wave, and U of each row group
    __shared__ __attribute__((aligned(16))) f4 sXP[2][CHUNK_WAVES][64];
    __shared__ __attribute__((aligned(16))) f4 sXR[2][CHUNK_WAVES][64];
    __shared__ __attribute__((aligned(16))) f4 sU[2][CHUNK_WAVES / 2][64];
    // Lam and M of the chunk, passed on to the copy wave
    __shared__ __attribute__((aligned(16))) f4 sLam[2][64];
    __shared__ __attribute__((aligned(16))) h8 sMp[2][64];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, kk = lane >> 4;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};

    // block -> (sequence n, value head h, channel block rb): the sequences'
    // ranges of hv * RB blocks in order of decreasing length, so the longest
    // recurrence starts first (up to SEQ_RANK_MAX sequences; beyond that in
    // index order); inside a range (a multiple of 8 blocks when hv is even)
    // the XCD-aware permutation
    constexpr int RB = 128 / CHUNK_ROWS;
    const int per_seq = d.hv * RB;
    const int rank = (int)blockIdx.x / per_seq;
    int w = (int)blockIdx.x - rank * per_seq;
    if ((per_seq & 7) == 0) w = (w & 7) * (per_seq >> 3) + (w >> 3);
    const int rb = w % RB;
    const int h = w / RB;
    const int n = d.n_seq <= SEQ_RANK_MAX ? seq_of_rank(p.cu, d.n_seq, rank) : rank;
    const int j = h / d.G;
    const int hk = d.hk, hv = d.hv;

    const int cu0 = p.cu[n];
    const int T_n = p.cu[n + 1] - cu0;
    if (T_n <= 0) return;
    const int n_chunks = (T_n + CT - 1) / CT;
    const uint32_t vstride = (uint32_t)hv * 128;

    if (wave == CHUNK_WAVES) {
        // ---- copy wave: global -> LDS, three chunks ahead of the compute --
        // global_load_lds_dwordx4 moves 1 KB per instruction (lane i lands at
        // 16 i past the piece's LDS base) without passing through registers.
        typedef const void __attribute__((address_space(1))) *gptr_t;
        typedef void __attribute__((address_space(3))) *lptr_t;
        constexpr int KH_PIECES = SCAN_KH_FLOATS * 4 / 1024;                       // 24
        constexpr int VH_PIECES = (SCAN_SLOT_FLOATS * 4 + 1023) / 1024;             // 3
        // the last value-head piece is 256 bytes: one dword per lane
        static_assert(SCAN_SLOT_FLOATS * 4 - (VH_PIECES - 1) * 1024 == 256, "value-head tail");
        // v: 2 copies of vc, or (RAW_V) 1 copy of the raw fp16 rows, which the
        // v wave turns into v
        constexpr int V_PIECES = RAW_V ? 1 : CT * CHUNK_ROWS * 4 / 1024;
        constexpr int V_LANES = CHUNK_ROWS / 4;                                     // lanes per token
        constexpr int PER_CHUNK = KH_PIECES + VH_PIECES + V_PIECES;                 // copies per chunk
        static_assert(RAW_V ? CT * CHUNK_ROWS * 2 == 1024 : V_PIECES * 1024 == CT * CHUNK_ROWS * 4,
                      "v pieces");
        static_assert(2 * PER_CHUNK <= 63, "vmcnt range");
        auto copy16 = [](const float *src, float *lds_piece) {
            __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_piece, 16, 0, 0);
        };
        auto copy4 = [](const float *src, float *lds_piece) {
            __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_piece, 4, 0, 0);
        };
        // Rows past the sequence's end read its last token (valid memory); the
        // slots give them zero weight (beta = Lam = 0, identity rows of T, zero
        // k and q), so they add exactly nothing.
        auto issue = [&](int c) {
            const int b = c & (NBUF - 1);
            const int64_t tb = (int64_t)cu0 + (int64_t)c * CT;
            const int nv = min(CT, T_n - c * CT);
            const int64_t slot = chunk_slot(cu0, n, c);
            const float *khs = p.ws + (slot * hk + j) * SCAN_KH_FLOATS + lane * 4;
#pragma unroll
            for (int m = 0; m < KH_PIECES; ++m) copy16(khs + m * 256, &sKH[b][m * 256]);
            const float *vhs = p.ws + d.vh_base + (slot * hv + h) * SCAN_SLOT_FLOATS;
#pragma unroll
            for (int m = 0; m < VH_PIECES - 1; ++m) copy16(vhs + m * 256 + lane * 4, &sVH[b][m * 256]);
            copy4(vhs + (VH_PIECES - 1) * 256 + lane, &sVH[b][(VH_PIECES - 1) * 256]);
            if constexpr (RAW_V) {
                // lane l: token l / 4, raw channels 8 (l % 4) .. + 7 of the block's
                // 32, landing at sRaw[b][l / 4][8 (l % 4)]
                const _Float16 *src = static_cast<const _Float16 *>(vr.qkv) +
                                      (tb + min(lane >> 2, nv - 1)) * vr.C + (2 * hk + h) * 128 +
                                      rb * CHUNK_ROWS + (lane & 3) * 8;
                __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)&sRaw[b][0][0], 16, 0, 0);
            } else {
                const float *vb = p.vc + (tb * hv + h) * 128 + rb * CHUNK_ROWS + (lane % V_LANES) * 4;
#pragma unroll
                for (int m = 0; m < V_PIECES; ++m) {
                    const int t = m * (64 / V_LANES) + lane / V_LANES;
                    copy16(vb + (uint32_t)min(t, nv - 1) * vstride, &sV[b][m * (64 / V_LANES)][0]);
                }
            }
        };
        // Chunk c sits in LDS copy c % 4.  It is issued after the barrier of
        // step c - 3 (the compute waves are then done with chunk c - 4) and
        // waited for before the barrier of step c - 1; step c reads it.
        for (int c = 0; c < 3 && c < n_chunks; ++c) issue(c);
        if (n_chunks > 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_CHUNK));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        side_barrier();
        for (int c = 0; c < n_chunks; ++c) {
            side_barrier();
            if (c + 3 < n_chunks) {
                issue(c + 3);
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(PER_CHUNK));  // chunk c + 2 has landed
            } else {
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            }
        }
        side_barrier();
        return;
    }
    if (wave == CHUNK_WAVES + 1) {
        // ---- output wave: O = (Lam R + M U) / sqrt(dk) of chunk c for both
        // row groups, after the barrier of step c + 1.  R, U, Lam and M come
        // from the compute waves through LDS: written after the barrier of
        // step c, overwritten (for chunk c + 2) only after that of step c + 2.
        // None of them is an LDS target of the copies.  A wave of its own, as
        // the copy wave spends most of a step issuing the copies.
        auto o_store = [&](int c) {
            const int x = c & 1;
            const int nv = min(CT, T_n - c * CT);
            const int64_t tb = (int64_t)cu0 + (int64_t)c * CT;
            const f4 lam = sLam[x][lane];
            const h8 mp = sMp[x][lane];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const f4 R = sXR[x][2 * g][lane] + sXR[x][2 * g + 1][lane];
                const f4 U = sU[x][g][lane];
                h4 uh, ul;
                split4s(U, uh, ul, d.ms);
                // (M_hi + M_lo) U_hi, then M_hi U_lo scaled back
                const f4 O = (mfma_k32(mp, cat(uh, uh), lam * R) +
                              mfma_k16(lo_half(mp), ul, z4) * LO_UNSCALE) * SCALE;
                char *ob = reinterpret_cast<char *>(p.o + (tb * hv + h) * 128 + rb * CHUNK_ROWS + g * 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 4 * kk + r;
                    if (t < nv) *reinterpret_cast<float *>(ob + ((uint32_t)t * vstride + l16) * 4u) = O[r];
                }
            }
        };
        side_barrier();
        for (int c = 0; c < n_chunks; ++c) {
            side_barrier();
            if (c > 0) o_store(c - 1);
        }
        side_barrier();
        o_store(n_chunks - 1);
        return;
    }

    if constexpr (RAW_V) {
        if (wave == CHUNK_WAVES + 2) {
            // ---- v wave: v of chunk c between the barriers of steps c - 1 and
            // c (the first: the initial barrier), into sV, from the raw rows the
            // copy wave brings with the chunk's other operands (in LDS from the
            // barrier of step c - 1 on).  Lane l takes token l / 4 of the chunk
            // and value channels 8 (l % 4) .. + 7 of the block's 32.  The
            // arithmetic is gdn_pre's (conv4, silu_fast), so v is bit for bit
            // the staged path's.
            const _Float16 *qkv = static_cast<const _Float16 *>(vr.qkv);
            const _Float16 *cw = static_cast<const _Float16 *>(vr.conv_w);
            _Float16 *hist = static_cast<_Float16 *>(vr.hist) + (int64_t)n * 3 * vr.C;
            const int C = vr.C;
            const int cv = (2 * hk + h) * 128 + rb * CHUNK_ROWS;  // the block's first raw channel
            const int t = lane >> 2, g8 = (lane & 3) * 8;
            float w[8][4];
            {
                float tw[4][8];
#pragma unroll
                for (int k = 0; k < 4; ++k) load8(cw + (int64_t)(cv + g8) * 4 + k * 8, tw[k]);
#pragma unroll
                for (int k = 0; k < 4; ++k)
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[(k * 8 + e) >> 2][(k * 8 + e) & 3] = tw[k][e];
            }
            // the old history rows of the block's channels (lanes 0..11)
            Raw8<_Float16> hrow;
            if (lane < 12) hrow.load(hist + (int64_t)(lane >> 2) * C + cv + g8);
            wait_vmem_all();
            if (lane < 12) *reinterpret_cast<h8 *>(&sRawH[lane >> 2][g8]) = hrow.v;
            // taps of token t: raw rows t - 3 .. t, reaching into the previous
            // chunk's rows (or the history, for chunk 0)
            auto conv_chunk = [&](int c) {
                const int b = c & (NBUF - 1), pb = (c - 1) & (NBUF - 1), rbuf = b;
                Raw8<_Float16> x[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int r = t + m - 3;
                    const _Float16 *rp = r >= 0 ? &sRaw[rbuf][r][g8]
                                       : c == 0 ? &sRawH[3 + r][g8] : &sRaw[pb][CT + r][g8];
                    x[m].v = *reinterpret_cast<const h8 *>(rp);
                }
                f4 s0, s1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float acc = conv4(w[e][0], w[e][1], w[e][2], w[e][3], x[0].get(e), x[1].get(e),
                                            x[2].get(e), x[3].get(e));
                    (e < 4 ? s0 : s1)[e & 3] = silu_fast(acc);
                }
                *reinterpret_cast<f4 *>(&sV[b][t][g8]) = s0;
                *reinterpret_cast<f4 *>(&sV[b][t][g8 + 4]) = s1;
            };
            side_barrier();
            conv_chunk(0);
            for (int c = 0; c < n_chunks; ++c) {
                side_barrier();
                if (c + 1 < n_chunks) conv_chunk(c + 1);
            }
            side_barrier();
            // the new history of the block's channels: X rows T_n .. T_n + 2 of
            // X = [old history; the sequence's rows]
            if (lane < 12) {
                const int r = lane >> 2;
                const int64_t xi = (int64_t)T_n + r;
                Raw8<_Float16> v;
                if (xi < 3) v.v = *reinterpret_cast<const h8 *>(&sRawH[xi][g8]);
                else v.load(qkv + ((int64_t)cu0 + xi - 3) * C + cv + g8);
                v.store(hist + (int64_t)r * C + cv + g8);
            }
            return;
        }
    }

    // ---- compute waves ---------------------------------------------------
    const int grp = wave >> 1;    // row group
    const int kh = wave & 1;      // key half: keys 64 kh .. 64 kh + 63
    const int partner = wave ^ 1;
    const int row = rb * CHUNK_ROWS + grp * 16 + l16;

    // state x 16 (exact), accumulator layout: S4[b][r] = 16 S[row][64 kh + 16 b + 4 kk + r].
    // With k and q also x16, every split operand and product stays well above
    // the fp16 subnormal range; Lam carries the 1/256 back.
    float *Srow = p.state + (((int64_t)n * hv + h) * 128 + row) * 128 + 64 * kh + 4 * kk;
    f4 S4[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) S4[b] = *reinterpret_cast<const f4 *>(Srow + 16 * b) * KQ_SCALE;

    // this wave's two 32-key steps of K (or Q) of chunk c, hi and lo
    auto key_ops = [&](int c, int off, h8 (&hi)[2], h8 (&lo)[2]) {
        const _Float16 *khp = reinterpret_cast<const _Float16 *>(sKH[c & (NBUF - 1)]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int s = 2 * kh + i;
            hi[i] = *reinterpret_cast<const h8 *>(khp + off + ((s * 2 + 0) * 64 + lane) * 8);
            lo[i] = *reinterpret_cast<const h8 *>(khp + off + ((s * 2 + 1) * 64 + lane) * 8);
        }
    };

    // K of chunk c + 1 is read from LDS during step c (it landed before the
    // barrier of step c), and the partial R of chunk c is formed after the
    // state update of step c: neither is on the path from the barrier of one
    // step to that of the next.
    lds_barrier();  // chunks 0 and 1 are in LDS
    h8 kph[2], kpl[2];
    key_ops(0, KH_KP, kph, kpl);
    for (int c = 0; c < n_chunks; ++c) {
        const int b = c & (NBUF - 1), x = c & 1;
        const _Float16 *khp = reinterpret_cast<const _Float16 *>(sKH[b]);
        const float *vh = sVH[b];
        // partial P = K S^T (x256) over this wave's 64 keys
        h8 sh[2], sl[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) split8s(S4[2 * i], S4[2 * i + 1], sh[i], sl[i], d.ms);
        f4 Phh = {0.f, 0.f, 0.f, 0.f}, Phl = Phh, Plh = Phh;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            Phh = mfma_k32(kph[i], sh[i], Phh);
            Phl = mfma_k32(kph[i], sl[i], Phl);   // x LO_SCALE
            Plh = mfma_k32(kpl[i], sh[i], Plh);
        }
        const f4 Pp = (Phh + Plh) + Phl * LO_UNSCALE;
        sXP[x][wave][lane] = Pp;
        lds_barrier();  // partials visible; every wave is past chunk c - 1
        __builtin_amdgcn_sched_barrier(0);  // nothing below moves up before the barrier

        // the partner's partial P first, then this chunk's value-head
        // operands, its Q and K^T, and K of the next chunk
        const f4 Po = sXP[x][partner][lane];
        const h8 tp = *reinterpret_cast<const h8 *>(reinterpret_cast<const _Float16 *>(vh + VH_TP) + lane * 8);
        const f4 lam = *reinterpret_cast<const f4 *>(vh + VH_LAM + 4 * kk);
        const f4 bet = *reinterpret_cast<const f4 *>(vh + VH_BETA + 4 * kk);
        const f4 wu = *reinterpret_cast<const f4 *>(vh + VH_W + 4 * kk);
        const float last = vh[VH_LAST];
        f4 vv;
#pragma unroll
        for (int r = 0; r < 4; ++r) vv[r] = sV[b][4 * kk + r][grp * 16 + l16];
        h8 kt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) kt[i] = *reinterpret_cast<const h8 *>(khp + KH_KT + ((4 * kh + i) * 64 + lane) * 8);
        h8 qph[2], qpl[2];
        key_ops(c, KH_QP, qph, qpl);
        if (c + 1 < n_chunks) key_ops(c + 1, KH_KP, kph, kpl);
        __builtin_amdgcn_sched_barrier(0);  // the reads go out before the work below

        // the full P, summed in the same order by both waves of the pair
        const f4 P = kh == 0 ? Pp + Po : Po + Pp;
        // B = beta (V - Lam P), component r is token 4 kk + r, channel l16
        f4 Bm;
#pragma unroll
        for (int r = 0; r < 4; ++r) Bm[r] = bet[r] * __builtin_fmaf(-lam[r], P[r], vv[r]);
        h4 bh, bl;
        split4s(Bm, bh, bl, d.ms);
        // U = T B: (T_hi B_hi + T_lo B_hi) + T_hi B_lo (the last scaled back)
        const f4 U = mfma_k32(tp, cat(bh, bh), z4) + mfma_k16(lo_half(tp), bl, z4) * LO_UNSCALE;
        if (kh == 0) sU[x][grp][lane] = U;
        if (wave == 1) {
            sLam[x][lane] = lam;
            sMp[x][lane] = *reinterpret_cast<const h8 *>(reinterpret_cast<const _Float16 *>(vh + VH_MP) + lane * 8);
        }
        h4 uwh, uwl;
        split4s(U * wu, uwh, uwl, d.ms);
        const h8 uww = cat(uwh, uwh);
        // 16 S' = Lam_last (16 S) + (16 K)^T (D[last] U): this wave's 4 key blocks;
        // (K_hi + K_lo)^T (U w)_hi accumulates onto Lam_last S, and the
        // K_hi^T (U w)_lo product (x LO_SCALE) is scaled back and added
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f4 C = mfma_k32(kt[i], uww, S4[i] * last);
            S4[i] = C + mfma_k16(lo_half(kt[i]), uwl, z4) * LO_UNSCALE;
        }
        // partial R = Q S^T (x256) of this chunk from the split of the state
        // before the update; the output wave reads it after the next barrier
        f4 Rhh = z4, Rhl = z4, Rlh = z4;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            Rhh = mfma_k32(qph[i], sh[i], Rhh);
            Rhl = mfma_k32(qph[i], sl[i], Rhl);   // x LO_SCALE
            Rlh = mfma_k32(qpl[i], sh[i], Rlh);
        }
        sXR[x][wave][lane] = (Rhh + Rlh) + Rhl * LO_UNSCALE;
    }
    lds_barrier();  // R and U of the last chunk are visible to the output wave
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f4 *>(Srow + 16 * i) = S4[i] * (1.f / KQ_SCALE);
}

static int64_t scan_slots(const gdn_shape &s)
{
    return s.total_T / CT + (int64_t)s.n_seq + 1;
}

// ---- the layer's pre stage fused into the prep step ------------------------
//
// With fp32 io, one block per (chunk, key head j) computes, for the chunk's
// 16 tokens, the pre stage of exactly the channels the prep step needs: q and
// k of key head j (conv, SiLU, L2 norm) straight into LDS, the group's gates,
// and v of the group's value heads (conv, SiLU) to the vc buffer the chunk
// kernel reads; then it builds the slots like scan_prep_kernel.  (With fp16
// io, layer_prep_pair_kernel below does the same for q, k and the gates of two
// chunks per block, and the chunk kernel forms v from the raw rows.)  The normalised q and k and the gates never go
// through memory.  The arithmetic is that of gdn_pre (the same per-element
// expressions), so the layer's results equal the staged path's bit for bit.
// History carry without a race: only the chunk-0 blocks read the old history,
// each for its own channels, and the same block writes the new history of
// those channels after a barrier.
template <typename TI>
__global__ __launch_bounds__(256) void layer_prep_kernel(LayerPrepArgs p, PrepDims d)
{
    __shared__ __attribute__((aligned(16))) PrepShared sm;
    __shared__ float sGate[LAYER_G_MAX][2][CT];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15;
    const int n = blockIdx.x / d.n_chunk_max;
    const int c = blockIdx.x - n * d.n_chunk_max;
    const int j = blockIdx.y;
    const int cu0 = p.cu[n];
    const int T_n = p.cu[n + 1] - cu0;
    if (c * CT >= T_n) return;
    const int nv = min(CT, T_n - c * CT);
    const int64_t tb = (int64_t)cu0 + c * CT;
    const int hk = d.hk, hv = d.hv, G = d.G, C = d.C;
    const TI *qkv = static_cast<const TI *>(p.qkv);
    const TI *cw = static_cast<const TI *>(p.conv_w);
    TI *hist = static_cast<TI *>(p.hist) + (int64_t)n * 3 * C;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};

    // Tasks (unit u, token part) of up to 8 tokens x 128 channels, one per
    // 16-lane row: u = 0 q of key head j, u = 1 its k, u = 2 + gh v of value
    // head j G + gh.  Each unit's 16 tokens are cut into P parts, P as large as
    // keeps the units x P tasks within the block's 16 rows (production: 5
    // units x 3 parts of 5, 5 and 6 tokens on 15 rows).  Lane l16 of the row
    // takes channels 4 l16 .. + 3 and 64 + 4 l16 .. + 3 of the unit (every
    // memory instruction covers whole 64-channel runs).  A task issues its
    // weight loads and the rows of X its tokens read, all unconditional (rows
    // past the chunk's end repeat its last row), waits for them once, and then
    // walks its tokens with no load behind a store.
    const int units = 2 + G;
    const int P = units > 8 ? 2 : CT / units;
    auto unit_base = [&](int u) {
        return u == 0 ? j * 128 : u == 1 ? (hk + j) * 128 : (2 * hk + j * G + (u - 2)) * 128;
    };
    // row xi of X = [history (3 rows); the sequence's tokens]
    auto xrow_ptr = [&](int64_t xi, int ch) {
        return xi < 3 ? hist + xi * C + ch : qkv + (cu0 + xi - 3) * C + ch;
    };
    const int ntask = units * P;
    for (int task = wave * 4 + (lane >> 4); task < ntask; task += 16) {  // uniform per 16-lane row
        const int u = task / P, part = task - u * P;
        const int ch = unit_base(u) + l16 * 4;
        const int t0 = CT * part / P;
        const int ntok = CT * (part + 1) / P - t0;  // tokens of this task (at most 8)
        const int nt = max(0, min(ntok, nv - t0));  // valid ones
        float w[8][4];
        {
            float tw[4][8];
#pragma unroll
            for (int k = 0; k < 4; ++k) load8(cw + (int64_t)(ch + 64 * (k >> 1)) * 4 + (k & 1) * 8, tw[k]);
#pragma unroll
            for (int k = 0; k < 4; ++k)
#pragma unroll
                for (int e = 0; e < 8; ++e) w[(k * 8 + e) >> 2][(k * 8 + e) & 3] = tw[k][e];
        }
        const int64_t xb = (int64_t)c * CT + t0;          // X row of tap 0 of the first token
        const int64_t x_last = (int64_t)c * CT + nv + 2;  // tap 3 of the chunk's last token
        Raw8<TI> x[11];
#pragma unroll
        for (int i = 0; i < 11; ++i) x[i].load_split(xrow_ptr(min(xb + min(i, ntok + 2), x_last), ch));
        wait_vmem_all();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i >= ntok) break;  // uniform per 16-lane row
            const int t = t0 + i;
            float sv[8];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float acc = conv4(w[e][0], w[e][1], w[e][2], w[e][3], x[i].get(e),
                                        x[i + 1].get(e), x[i + 2].get(e), x[i + 3].get(e));
                sv[e] = silu_fast(acc);
                ss = fmaf(sv[e], sv[e], ss);
            }
            if (u < 2) {
                ss = row_sum16(ss);
                const float sc = rsqrt_fast(ss + d.eps_l2);
                float *dst = u == 0 ? &sm.sQ[t][l16 * 4] : &sm.sK[t][l16 * 4];
                *reinterpret_cast<f4 *>(dst) =
                    i < nt ? f4{sv[0] * sc, sv[1] * sc, sv[2] * sc, sv[3] * sc} : z4;
                *reinterpret_cast<f4 *>(dst + 64) =
                    i < nt ? f4{sv[4] * sc, sv[5] * sc, sv[6] * sc, sv[7] * sc} : z4;
            } else if (i < nt) {
                store8_split_nt(p.vc + ((tb + t) * hv + j * G + (u - 2)) * 128 + l16 * 4, sv);
            }
        }
    }

    // gates of the group's value heads, token t of head gh at sGate[gh][.][t]
    // (the last wave, which has the fewest tasks above)
    if (wave == CHUNK_PREP_THREADS / 64 - 1) {
        for (int i = lane; i < G * CT; i += 64) {
            const int gh = i / CT, t = i - gh * CT, h = j * G + gh;
            float g = 0.f, bt = 0.f;
            if (t < nv) {
                const int64_t e = (tb + t) * hv + h;
                gates(ld1(static_cast<const TI *>(p.a) + e), ld1(static_cast<const TI *>(p.dt_bias) + h),
                      ld1(static_cast<const TI *>(p.A_log) + h), ld1(static_cast<const TI *>(p.b) + e), g,
                      bt);
            }
            sGate[gh][0][t] = g;
            sGate[gh][1][t] = bt;
        }
    }
    __syncthreads();

    // the new history of this block's channels (chunk 0 only)
    if (c == 0 && tid < units * 16) {
        const int ch = unit_base(tid >> 4) + l16 * 4;
        Raw8<TI> v[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) v[r].load_split(xrow_ptr((int64_t)T_n + r, ch));
        // X row T_n + r; for T_n + r < 3 it is old history row T_n + r > r,
        // not yet overwritten: all three are read before the first write
        wait_vmem_all();
#pragma unroll
        for (int r = 0; r < 3; ++r) v[r].store_split(hist + (int64_t)r * C + ch);
    }

    auto load_gb = [&](int gh, float &gl, float &bl) {
        gl = sGate[gh][0][l16];
        bl = sGate[gh][1][l16];
    };
    float g_next = 0.f, b_next = 0.f;
    if (wave < G) load_gb(wave, g_next, b_next);
    prep_body(sm, p.ws, d, j, chunk_slot(cu0, n, c), nv, g_next, b_next, load_gb);
}

// The fp16 layer path's prep step: what layer_prep_kernel does for one
// chunk, without v (the chunk kernel forms it), for two consecutive chunks
// per block.  Each 16-lane row has one task per chunk, q or k of key head j
// for two of its tokens; both chunks' rows are requested up front, so those
// of the second are in flight while the block builds the first chunk's slots,
// and with half as many blocks all of them are resident at once.  Same
// per-element arithmetic as gdn_pre, so the results equal the staged path's
// bit for bit.
__global__ __launch_bounds__(256) void layer_prep_pair_kernel(LayerPrepArgs p, PrepDims d)
{
    __shared__ __attribute__((aligned(16))) PrepShared sm;
    __shared__ float sGate[2][LAYER_G_MAX][2][CT];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15;
    const int per_seq = (d.n_chunk_max + 1) >> 1;
    const int n = blockIdx.x / per_seq;
    const int c0 = 2 * (int)(blockIdx.x - n * per_seq);
    const int j = blockIdx.y;
    const int cu0 = p.cu[n];
    const int T_n = p.cu[n + 1] - cu0;
    if (c0 * CT >= T_n) return;
    const bool two = (c0 + 1) * CT < T_n;  // uniform per block
    const int nv0 = min(CT, T_n - c0 * CT);
    const int nv1 = two ? min(CT, T_n - (c0 + 1) * CT) : 0;
    const int hk = d.hk, hv = d.hv, G = d.G, C = d.C;
    const _Float16 *qkv = static_cast<const _Float16 *>(p.qkv);
    const _Float16 *cw = static_cast<const _Float16 *>(p.conv_w);
    _Float16 *hist = static_cast<_Float16 *>(p.hist) + (int64_t)n * 3 * C;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};

    // task of this row: unit u (0: q, 1: k of key head j), tokens t0, t0 + 1
    // of each chunk; lane l16 takes channels 4 l16 .. + 3 and 64 + 4 l16 .. + 3
    const int task = wave * 4 + (lane >> 4);
    const int u = task >> 3, t0 = 2 * (task & 7);
    const int ch = (u == 0 ? j : hk + j) * 128 + l16 * 4;
    // row xi of X = [history (3 rows); the sequence's tokens], channel c
    auto xrow = [&](int64_t xi, int c) { return xi < 3 ? hist + xi * C + c : qkv + (cu0 + xi - 3) * C + c; };
    // weights (fp16, element (4 m + tap) of the lane's channel m = 0..7), then
    // the five X rows of the task's two tokens in each chunk; rows past a
    // chunk's end repeat its last row (valid memory, results unused)
    Raw8<_Float16> wr[4], xa[5], xb[5];
    auto load_w = [&]() {
#pragma unroll
        for (int k = 0; k < 4; ++k) wr[k].load(cw + (int64_t)(ch + 64 * (k >> 1)) * 4 + (k & 1) * 8);
    };
    load_w();
#pragma unroll
    for (int i = 0; i < 5; ++i)
        xa[i].load_split(xrow(min((int64_t)c0 * CT + t0 + i, (int64_t)c0 * CT + nv0 + 2), ch));
    if (two) {
#pragma unroll
        for (int i = 0; i < 5; ++i)
            xb[i].load_split(xrow(min((int64_t)(c0 + 1) * CT + t0 + i, (int64_t)(c0 + 1) * CT + nv1 + 2), ch));
    }
    // conv, SiLU and the L2 norm of the task's tokens of one chunk, into sQ / sK
    auto conv = [&](const Raw8<_Float16> (&x)[5], int nv) {
        const int nt = max(0, min(2, nv - t0));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = t0 + i;
            float sv[8];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float acc = conv4(wr[e >> 1].get((e & 1) * 4 + 0), wr[e >> 1].get((e & 1) * 4 + 1),
                                        wr[e >> 1].get((e & 1) * 4 + 2), wr[e >> 1].get((e & 1) * 4 + 3),
                                        x[i].get(e), x[i + 1].get(e), x[i + 2].get(e), x[i + 3].get(e));
                sv[e] = silu_fast(acc);
                ss = fmaf(sv[e], sv[e], ss);
            }
            ss = row_sum16(ss);
            const float sc = rsqrt_fast(ss + d.eps_l2);
            float *dst = u == 0 ? &sm.sQ[t][l16 * 4] : &sm.sK[t][l16 * 4];
            *reinterpret_cast<f4 *>(dst) = i < nt ? f4{sv[0] * sc, sv[1] * sc, sv[2] * sc, sv[3] * sc} : z4;
            *reinterpret_cast<f4 *>(dst + 64) = i < nt ? f4{sv[4] * sc, sv[5] * sc, sv[6] * sc, sv[7] * sc} : z4;
        }
    };
    conv(xa, nv0);

    // gates of the group's value heads for both chunks, token t of head gh of
    // chunk k at sGate[k][gh][.][t] (zero past the end)
    if (wave == CHUNK_PREP_THREADS / 64 - 1) {
        for (int i = lane; i < 2 * G * CT; i += 64) {
            const int k = i / (G * CT), r = i - k * G * CT;
            const int gh = r / CT, t = r - gh * CT, h = j * G + gh;
            float g = 0.f, bt = 0.f;
            if (t < (k == 0 ? nv0 : nv1)) {
                const int64_t e = ((int64_t)cu0 + (c0 + k) * CT + t) * hv + h;
                gates(ld1(static_cast<const _Float16 *>(p.a) + e), ld1(static_cast<const _Float16 *>(p.dt_bias) + h),
                      ld1(static_cast<const _Float16 *>(p.A_log) + h), ld1(static_cast<const _Float16 *>(p.b) + e),
                      g, bt);
            }
            sGate[k][gh][0][t] = g;
            sGate[k][gh][1][t] = bt;
        }
    }
    __syncthreads();

    // the new history of q and k of key head j (the block of chunk 0): X rows
    // T_n .. T_n + 2; for T_n + r < 3 that is old history row T_n + r > r,
    // not yet overwritten: all three are read before the first write
    if (c0 == 0 && tid < 32) {
        const int hc = ((tid >> 4) == 0 ? j : hk + j) * 128 + l16 * 4;
        Raw8<_Float16> v[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) v[r].load_split(xrow((int64_t)T_n + r, hc));
        wait_vmem_all();
#pragma unroll
        for (int r = 0; r < 3; ++r) v[r].store_split(hist + (int64_t)r * C + hc);
    }

    float g_next = 0.f, b_next = 0.f;
    auto load_gb0 = [&](int gh, float &gl, float &bl) {
        gl = sGate[0][gh][0][l16];
        bl = sGate[0][gh][1][l16];
    };
    if (wave < G) load_gb0(wave, g_next, b_next);
    prep_body(sm, p.ws, d, j, chunk_slot(cu0, n, c0), nv0, g_next, b_next, load_gb0);
    if (!two) return;

    load_w();  // (again: not held across the first chunk's slots)
    __syncthreads();  // every wave is done with the first chunk's LDS
    conv(xb, nv1);
    __syncthreads();
    auto load_gb1 = [&](int gh, float &gl, float &bl) {
        gl = sGate[1][gh][0][l16];
        bl = sGate[1][gh][1][l16];
    };
    g_next = 0.f;
    b_next = 0.f;
    if (wave < G) load_gb1(wave, g_next, b_next);
    prep_body(sm, p.ws, d, j, chunk_slot(cu0, n, c0 + 1), nv1, g_next, b_next, load_gb1);
}

static PrepDims prep_dims(const gdn_shape &s)
{
    PrepDims pd;
    pd.hk = s.hk;
    pd.hv = s.hv;
    pd.G = s.hv / s.hk;
    pd.n_chunk_max = (int)((s.max_T + CT - 1) / CT);
    pd.vh_base = scan_slots(s) * s.hk * SCAN_KH_FLOATS;
    pd.m1 = -1.f;
    pd.C = 2 * s.hk * 128 + s.hv * 128;
    pd.eps_l2 = s.eps_l2;
    return pd;
}

static hipError_t launch_chunk(const gdn_shape &s, const ScanArgs &a, hipStream_t st,
                               const VRawArgs *vr = nullptr)
{
    ChunkDims cd;
    cd.hk = s.hk;
    cd.hv = s.hv;
    cd.G = s.hv / s.hk;
    cd.n_seq = s.n_seq;
    cd.vh_base = scan_slots(s) * s.hk * SCAN_KH_FLOATS;
    cd.m1 = -1.f;
    cd.ms = -LO_SCALE;
    const int64_t blocks = (int64_t)s.n_seq * s.hv * (128 / CHUNK_ROWS);
    if (vr)
        hipLaunchKernelGGL(scan_chunk_kernel<true>, dim3((unsigned)blocks), dim3(chunk_threads(true)), 0,
                           st, a, cd, *vr);
    else
        hipLaunchKernelGGL(scan_chunk_kernel<false>, dim3((unsigned)blocks), dim3(chunk_threads(false)), 0,
                           st, a, cd, VRawArgs{});
    return hipGetLastError();
}

hipError_t launch_scan(const gdn_shape &s, const ScanArgs &a, hipStream_t st)
{
    const PrepDims pd = prep_dims(s);
    hipLaunchKernelGGL(scan_prep_kernel, dim3((unsigned)(s.n_seq * (int64_t)pd.n_chunk_max), s.hk),
                       dim3(CHUNK_PREP_THREADS), 0, st, a, pd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_chunk(s, a, st);
}

hipError_t launch_layer_scan(const gdn_shape &s, const LayerPrepArgs &lp, const ScanArgs &a,
                             hipStream_t st)
{
    const PrepDims pd = prep_dims(s);
    const dim3 grid((unsigned)(s.n_seq * (int64_t)pd.n_chunk_max), s.hk);
    if (s.io_dtype == GDN_F16) {
        // v of the value heads is formed in the chunk kernel (VRawArgs)
        const dim3 pgrid((unsigned)(s.n_seq * (int64_t)((pd.n_chunk_max + 1) / 2)), s.hk);
        hipLaunchKernelGGL(layer_prep_pair_kernel, pgrid, dim3(CHUNK_PREP_THREADS), 0, st, lp, pd);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const VRawArgs vr{lp.qkv, lp.conv_w, lp.hist, pd.C};
        return launch_chunk(s, a, st, &vr);
    }
    hipLaunchKernelGGL(layer_prep_kernel<float>, grid, dim3(CHUNK_PREP_THREADS), 0, st, lp, pd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_chunk(s, a, st);
}

size_t scan_workspace_bytes(const gdn_shape &s)
{
    return (size_t)scan_slots(s) * ((size_t)s.hk * SCAN_KH_FLOATS + (size_t)s.hv * SCAN_SLOT_FLOATS) *
           sizeof(float);
}

} // namespace gdn
