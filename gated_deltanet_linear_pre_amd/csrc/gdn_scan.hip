// gdn_scan.hip -- the gated delta rule on an fp32 state, in 32-token chunks on
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
// Over a chunk of 32 tokens starting from state S0, with
//   D[t][s] = exp(g_{s+1} + ... + g_t)    (decay from just after s to t, <= 1)
//   Lam_t   = exp(g_0 + ... + g_t)        (decay from the chunk start)
// the writes u_t = beta_t (v_t - alpha_t S_{t-1} k_t) solve a unit lower
// triangular system, and the outputs and the next state follow:
//   (I + A) U = diag(beta) (V - diag(Lam) P),  A[t][s] = beta_t D[t][s] k_t.k_s (s<t)
//   O  = (diag(Lam) R + M U) / sqrt(dk),       M[t][s] = D[t][s] q_t.k_s     (s<=t)
//   S' = Lam_last S0 + sum_s D[last][s] u_s k_s^T
// with P = K S0^T, R = Q S0^T (tokens x value channels).  This is exact
// algebra of the recurrence (unroll S_t = Lam_t S0 + sum_{s<=t} D[t][s] u_s k_s^T).
// Every decay is formed as exp of a sum of at most 16 log decays (one half of
// the chunk), or as the product of two such decays (both <= 1) when it spans
// both halves; never as a ratio of two cumulative products, so nothing
// overflows or cancels.
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
// * prep (parallel over sequence x chunk x key head):
//   - K and Q of the chunk (32 tokens x 128 keys) split into hi/lo fp16 and
//     laid out in the exact per-lane operand order of the chunk kernel's
//     MFMAs ("key-head slot", 32 KB per chunk); the same split operands give
//     the chunk's k.k and k.q tiles on MFMA, once per key head;
//   - per value head: the decays, T = (I + A)^-1 (its two diagonal blocks by
//     forward substitution, one column per lane, and the off-diagonal block
//     as a product), M, Lam, beta and the last-row decays, T and M
//     split and laid out as MFMA operands ("value-head slot", 6.5 KB).
// * chunk kernel (sequential over chunks): a block owns 32 value channels
//   of one (sequence, value head) in two row groups of 16; each row group's
//   state (16 channels x 128 keys) is split by key halves over a pair of
//   compute waves, each holding its 16 x 64 quarter in MFMA accumulator
//   layout (16 VGPRs/lane).  Per chunk and compute wave (v_mfma_f32_16x16x32_f16):
//     P = K S^T, R = Q S^T   12 + 12  (2 token tiles x 2 key steps x 3 split terms)
//     U = T B                2 + 3    (token tile 0: 16-deep; tile 1: 32-deep)
//     S' = Lam_last S + K^T (D U)  12 (4 key blocks x 3 split terms)
//   A 32-deep contraction over the chunk's tokens runs over a permuted token
//   order (position 8 (l/16) + e is token 16 (e/4) + 4 (l/16) + e % 4), so
//   the accumulator layout of the two 16-token tiles of B, U and U w is
//   directly the B operand.  K^T for the update is read from K's LDS copy
//   with gfx950's transposing LDS read (ds_read_b64_tr_b16), so the key-head
//   slot holds K and Q only.  The two waves of a pair add their partial
//   K S^T through LDS in the same order, so both form the same U; this
//   exchange and one barrier per chunk are the only synchronisation on the
//   recurrence.  Every product consumes the layout the previous one produced,
//   so the state never leaves registers.
//   A copy wave moves the chunk operands from global memory into LDS a step
//   ahead (K two steps ahead: the compute waves read it one step early); Q
//   goes from the workspace straight into the compute waves' registers.  Two
//   output waves (one per row group) form O = Lam R + M U one step behind,
//   from the partial Q S^T and U the compute waves leave in LDS, so the
//   outputs stay off the recurrence's path.  In the layer path with fp16 inputs a v wave forms v
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
// multiple of 32 tokens gives bit-identical results; other split points agree
// within rounding (the chunk grid moves).
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
// the operand type of the transposing LDS read builtin
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_t lds_h4;

constexpr int CT = 32;           // tokens per chunk (two 16-token tiles)
constexpr int KS = 132;          // LDS row stride of the fp32 K/Q chunk in prep
constexpr int AS = 36;           // LDS row stride of A and T in prep (rows 16-byte aligned)
constexpr float KQ_SCALE = 16.f; // k and q scale before the fp16 split (exact)
constexpr float SCALE = 0.08838834764831845f;  // 1 / sqrt(128)

// key-head slot, in fp16 elements: K, then Q, each
// [2 token tiles][4 key steps][2 hi/lo][64 positions][8]; lane 16 kk + t of
// tile tau, key step s holds keys 32 s + 16 (e / 4) + 4 kk + e % 4 of token
// 16 tau + t, at position lane in Q and kpos(lane) in K.
constexpr int KH_KP = 0;
constexpr int KH_QP = 8192;
static_assert(SCAN_KH_FLOATS * 2 == 16384, "key-head slot size");
__host__ __device__ constexpr int kp_off(int tau, int s, int hl) { return ((tau * 4 + s) * 2 + hl) * 512; }
// K's positions are swizzled for the transposing K^T read, whose 16 lanes of
// a group address four tokens of all four key quads kk: unswizzled those sit
// 256 bytes apart, on the same LDS banks (measured: 6 conflict cycles per
// read).  Position 16 kk + (t ^ 4 x(kk)), x = (0, 3, 2, 1), spreads each
// half-wave's 32 addresses over every 16-byte bank group twice (2 cycles,
// the least for 8-byte reads that all take the same half of a 16-byte
// piece), and keeps the 16-byte operand reads free of conflicts (measured;
// the plain x(kk) = kk is not).
__host__ __device__ constexpr int kpos(int lane)
{
    return lane ^ (4 * ((lane >> 4) ^ (((lane >> 4) & 1) << 1)));
}
// value-head slot, in floats
constexpr int VH_TP = 0;       // [3][64 lanes][8] fp16: T00 (hi 4 | lo 4), T1 hi, T1 lo
constexpr int VH_MP = 768;     // the same for M
constexpr int VH_LAM = 1536;   // [32] Lam_t / 256 (k, q and the state each carry a factor 16)
constexpr int VH_BETA = 1568;  // [32] beta_t (0 past the chunk's end)
constexpr int VH_W = 1600;     // [32] D[last][s] (0 past the end)
constexpr int VH_LAST = 1632;  // Lam_last
static_assert(SCAN_SLOT_FLOATS >= 1633 && SCAN_SLOT_FLOATS * 4 == 6 * 1024 + 512, "value-head slot size");

// D += A B, 16x16x16: lane l supplies A[l%16][4(l/16)+e] and B[4(l/16)+e][l%16];
// D[4(l/16)+r][l%16] comes back in component r.
// A product never takes the result of a product of the other shape as its
// accumulator: the compiler leaves too few wait states between a 16x16x32
// and a 16x16x16 that reads its result as C on gfx950 (measured: stale rows
// in the result).  The chunk step uses 16x16x32 only; a 16-deep term runs as
// a zero-padded one.
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
// its own product, whose other operand is scaled by 2^-10 (or whose result
// is, when it is added): lo stays a normal fp16 number down to |x| ~ 2^-13
// instead of 2^-3, so the split keeps ~22 bits over 29 binades of
// magnitude, and past the top of the fp16 range (|x| > 65504 + 2^6) the
// scaled low half overflows to inf, which the results show.  2^10 is the
// largest scale that keeps that top: lo <= ulp(hi) 2^10 < 2^15 for every
// finite hi.  ms = -LO_SCALE at run time (see lo_pair).
constexpr float LO_SCALE = 1024.f;
constexpr float LO_UNSCALE = 1.f / 1024.f;
__device__ __forceinline__ uint32_t lo_pair_s(uint32_t hi2, float x0, float x1, float ms)
{
    const h2 h = __builtin_bit_cast(h2, hi2);
    const h2 r = {(_Float16)__builtin_fmaf((float)h[0], ms, x0 * LO_SCALE),
                  (_Float16)__builtin_fmaf((float)h[1], ms, x1 * LO_SCALE)};
    return __builtin_bit_cast(uint32_t, r);
}
template <bool SCALED>
__device__ __forceinline__ void split4(const f4 x, h4 &hi, h4 &lo, float m)
{
    u2 h, l;
    h[0] = hi_pair(x[0], x[1]);
    h[1] = hi_pair(x[2], x[3]);
    if constexpr (SCALED) {
        l[0] = lo_pair_s(h[0], x[0], x[1], m);
        l[1] = lo_pair_s(h[1], x[2], x[3], m);
    } else {
        l[0] = lo_pair(h[0], x[0], x[1], m);
        l[1] = lo_pair(h[1], x[2], x[3], m);
    }
    hi = __builtin_bit_cast(h4, h);
    lo = __builtin_bit_cast(h4, l);
}
template <bool SCALED>
__device__ __forceinline__ void split8(const f4 a, const f4 b, h8 &hi, h8 &lo, float m)
{
    h4 ha, la, hb, lb;
    split4<SCALED>(a, ha, la, m);
    split4<SCALED>(b, hb, lb, m);
    hi = __builtin_shufflevector(ha, hb, 0, 1, 2, 3, 4, 5, 6, 7);
    lo = __builtin_shufflevector(la, lb, 0, 1, 2, 3, 4, 5, 6, 7);
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
// total_T / 32 + n_seq.
__device__ __forceinline__ int64_t chunk_slot(int cu0, int n, int c)
{
    return (int64_t)(cu0 >> 5) + c + n;
}

// A 16-byte store of a prep slot that writes through the L2 (the buffer
// store's sc1 cache-policy bit): only the next launch reads the slots, and a
// launch that leaves fewer dirty L2 lines behind hands over to the next one
// sooner (36-layer prefill +0.6%).  base is the same for the whole wave.
__device__ __forceinline__ void store_slot(_Float16 *base, int off_halves, h8 v)
{
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, 0x7fffffff, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), r, off_halves * 2, 0, 16);
}

struct PrepDims {
    int hk, hv, G, n_chunk_max;
    float m1;         // -1 (see lo_pair)
    int64_t vh_base;  // float offset of the value-head slots in the workspace
    int C;            // channels of a qkv row (fused layer prep)
    float eps_l2;     // (fused layer prep)
};

// LDS of the prep step of one (chunk, key head).  Its three phases use it one
// after another: k and q of the chunk; the per-wave partial k.k and k.q
// tiles; A and T of each wave's value head.
struct PrepShared {
    union {
        struct {
            float sK[CT][KS];           // k and q of the chunk (zero past the end)
            float sQ[CT][KS];
        } kq;
        f4 sPart[6][4][64];             // per-wave partial tiles
        struct {
            float sA[4][CT][AS];
            float sT[4][CT][AS];
        } at;
    } u;
    float sGB[4][2][CT];
};

// Everything after k and q of the chunk are in LDS: the key-head slot and the
// value-head slots.  load_gb(gh, g, b) gives lane l the g and beta of token
// l % 32 of value head gh of the group (0 past the end); g_next, b_next
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

    // ---- key-head slot: K and Q split and packed in operand order, and this
    // wave's 32 keys (key step s = wave) of the k.k and k.q tiles ------------
    _Float16 *kh = reinterpret_cast<_Float16 *>(ws + (slot * hk + j) * SCAN_KH_FLOATS);
    // tiles in accumulator layout (component r of lane (l16, kk) is row 4 kk
    // + r, column l16), K0 / K1 = tokens 0-15 / 16-31: 0: K0 K0^T, 1: K1 K0^T,
    // 2: K1 K1^T, 3: K0 Q0^T, 4: K0 Q1^T, 5: K1 Q1^T
    f4 part[6];
    {
        const int s = wave;
        h8 khi[2], klo[2], qhi[2], qlo[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const int t = 16 * tau + l16;
            f4 ka, kb, qa, qb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ka[e] = KQ_SCALE * sm.u.kq.sK[t][32 * s + 4 * kk + e];
                kb[e] = KQ_SCALE * sm.u.kq.sK[t][32 * s + 16 + 4 * kk + e];
                qa[e] = KQ_SCALE * sm.u.kq.sQ[t][32 * s + 4 * kk + e];
                qb[e] = KQ_SCALE * sm.u.kq.sQ[t][32 * s + 16 + 4 * kk + e];
            }
            split8<false>(ka, kb, khi[tau], klo[tau], d.m1);
            split8<false>(qa, qb, qhi[tau], qlo[tau], d.m1);
            store_slot(kh, KH_KP + kp_off(tau, s, 0) + kpos(lane) * 8, khi[tau]);
            store_slot(kh, KH_KP + kp_off(tau, s, 1) + kpos(lane) * 8, klo[tau]);
            store_slot(kh, KH_QP + kp_off(tau, s, 0) + lane * 8, qhi[tau]);
            store_slot(kh, KH_QP + kp_off(tau, s, 1) + lane * 8, qlo[tau]);
        }
        // as A and as B operand, lane (t, kk) holds the same row of keys, so
        // the product is X Y^T over this key step (x 256)
        auto mm = [&](h8 ah, h8 al, h8 bh, h8 bl) {
            return (mfma_k32(ah, bh, z4) + mfma_k32(ah, bl, z4)) + mfma_k32(al, bh, z4);
        };
        part[0] = mm(khi[0], klo[0], khi[0], klo[0]);
        part[1] = mm(khi[1], klo[1], khi[0], klo[0]);
        part[2] = mm(khi[1], klo[1], khi[1], klo[1]);
        part[3] = mm(khi[0], klo[0], qhi[0], qlo[0]);
        part[4] = mm(khi[0], klo[0], qhi[1], qlo[1]);
        part[5] = mm(khi[1], klo[1], qhi[1], qlo[1]);
    }
    __syncthreads();  // every wave is done with k and q in LDS
#pragma unroll
    for (int i = 0; i < 6; ++i) sm.u.sPart[i][wave][lane] = part[i];
    __syncthreads();
    // the four key steps summed in one order by every wave
    f4 tl[6];
    {
        const float unscale = 1.f / (KQ_SCALE * KQ_SCALE);
#pragma unroll
        for (int i = 0; i < 6; ++i)
            tl[i] = (((sm.u.sPart[i][0][lane] + sm.u.sPart[i][1][lane]) + sm.u.sPart[i][2][lane]) +
                     sm.u.sPart[i][3][lane]) * unscale;
    }
    __syncthreads();  // the partials are read before A and T overwrite them

    // ---- value-head slots ------------------------------------------------
    auto &sA = sm.u.at.sA[wave];
    auto &sT = sm.u.at.sT[wave];
    for (int gh = wave; gh < d.G; gh += 4) {
        // lane index and chunk length made opaque to the compiler here, so
        // that the many comparisons below are formed next to their use in
        // every iteration rather than hoisted out of the loop and kept live
        // (which spilled scalar registers)
        int lane_o = lane, nv_o = nv;
        __asm__ volatile("" : "+v"(lane_o), "+s"(nv_o));
        const int l16 = lane_o & 15, kk = lane_o >> 4;
        const int h = j * d.G + gh;
        float *vs = ws + d.vh_base + (slot * hv + h) * SCAN_SLOT_FLOATS;
        const float g_own = g_next, b_own = b_next;
        if (gh + 4 < d.G) load_gb(gh + 4, g_next, b_next);
        // the 32 g and beta through this wave's LDS rows: every lane reads the
        // g row as uniform VGPRs, and its own 4-token pieces of g and beta
        if (lane < CT) {
            sm.sGB[wave][0][lane] = g_own;
            sm.sGB[wave][1][lane] = b_own;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float gv[CT];
#pragma unroll
        for (int i = 0; i < CT / 4; ++i) {
            const f4 x = *reinterpret_cast<const f4 *>(&sm.sGB[wave][0][4 * i]);
            gv[4 * i] = x[0]; gv[4 * i + 1] = x[1]; gv[4 * i + 2] = x[2]; gv[4 * i + 3] = x[3];
        }
        // beta of tokens 4 kk .. 4 kk + 3 and 16 + 4 kk .. 16 + 4 kk + 3
        const f4 b4a = *reinterpret_cast<const f4 *>(&sm.sGB[wave][1][4 * kk]);
        const f4 b4b = *reinterpret_cast<const f4 *>(&sm.sGB[wave][1][16 + 4 * kk]);
        // Every decay is the exp of a sum of the log decays it spans, each
        // sum taken in token order within one 16-token half of the chunk.
        // The walk covers the two diagonal blocks at once in 16 steps: lane
        // s < 16 walks column s over tokens 0..15 and lane 16 + s' column
        // 16 + s' over tokens 16..31, D[t][s] = exp(g_{s+1} + ... + g_t) for
        // t > s (0 above the diagonal, 1 on it, written after the walk), into
        // sT (free until T is formed).  Lanes 32 and 33 take the sums from
        // the chunk start over tokens 0..15 (Lam_t = exp of it in column 32,
        // the sum in column 33), lanes 34 and 35 those from token 16 over
        // tokens 16..31 (exp of it, D[t][15], in column 15, the sum in column
        // 34).  The walk has no comparison: whether token t counts for a lane
        // is the sign of its start column minus t.  Then the block below the
        // diagonal ones is D[t][s] = D[t][15] D[15][s] (t >= 16 > s; both
        // factors <= 1), and Lam_t for t >= 16 is exp(S_15 + sum_{16..t}).
        {
            const bool second = (lane_o >= 16 && lane_o < 32) || lane_o >= 34;
            const int s0 = lane_o < 32 ? (lane_o & 31) : (lane_o < 34 ? -1 : 15);
            // column each lane writes: its own, 32/33, 15/34; lanes past 35
            // (and their unused results) go to padding column 35
            const int colw = lane_o < 32 ? lane_o : lane_o == 32 ? 32 : lane_o == 33 ? 33
                           : lane_o == 34 ? 15 : lane_o == 35 ? 34 : 35;
            const bool wsum = lane_o == 33 || lane_o == 35;
            const int tb = second ? CT / 2 : 0;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < CT / 2; ++i) {
                const int t = tb + i;
                const float gi = second ? gv[CT / 2 + i] : gv[i];
                const uint32_t m = (uint32_t)((s0 - t) >> 31);  // all ones if t counts
                acc += __uint_as_float(__float_as_uint(gi) & m);
                const float e = exp_fast(acc);
                sT[t][colw] = __uint_as_float(__float_as_uint(wsum ? acc : e) & m);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            {
                // rows 16 + (lane % 16), columns 4 (lane / 16) .. + 3 (but 15)
                const int t = CT / 2 + l16, sb = 4 * kk;
                const float dt = sT[t][15];
                const f4 d15 = *reinterpret_cast<const f4 *>(&sT[15][sb]);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (sb + k < 15) sT[t][sb + k] = dt * d15[k];
                if (lane_o < CT) sT[lane_o][lane_o] = 1.f;
                if (lane_o >= CT / 2 && lane_o < CT) {
                    const float st = sT[15][33] + sT[lane_o][34];
                    sT[lane_o][33] = st;
                    sT[lane_o][32] = exp_fast(st);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane_o < CT) {
                const int s = lane_o;
                // Lam_t and D[last][t] weight this chunk's terms only
                vs[VH_LAM + s] = s < nv_o ? sT[s][32] * (1.f / (KQ_SCALE * KQ_SCALE)) : 0.f;
                vs[VH_BETA + s] = b_own;
                vs[VH_W + s] = s < nv_o ? sT[nv_o - 1][s] : 0.f;
            }
            // Lam_last multiplies the whole state every chunk, so it takes
            // the correctly rounded exp
            if (lane_o == 32) vs[VH_LAST] = expf(sT[nv_o - 1][33]);
        }
        // A[t][s] = beta_t D[t][s] k_t.k_s (s < t), by tiles: lane (l16, kk)
        // takes column s = l16 (+ 16) and rows t = 4 kk + i (+ 16)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t0 = 4 * kk + i, t1 = 16 + 4 * kk + i;
            sA[t0][l16] = (t0 < nv_o && l16 < t0) ? b4a[i] * sT[t0][l16] * tl[0][i] : 0.f;
            sA[t1][l16] = t1 < nv_o ? b4b[i] * sT[t1][l16] * tl[1][i] : 0.f;
            sA[t1][16 + l16] = (t1 < nv_o && 16 + l16 < t1) ? b4b[i] * sT[t1][16 + l16] * tl[2][i] : 0.f;
        }
        // M[t][s] = D[t][s] q_t.k_s (s <= t) in operand order, lane L = 16 kk + t':
        //   M00: t = t', s = 4 kk + e;  M1: t = 16 + t', s = 16 (e / 4) + 4 kk + e % 4
        {
            const int tp = l16;
            const f4 d00 = *reinterpret_cast<const f4 *>(&sT[tp][4 * kk]);
            const f4 d1a = *reinterpret_cast<const f4 *>(&sT[16 + tp][4 * kk]);
            const f4 d1b = *reinterpret_cast<const f4 *>(&sT[16 + tp][16 + 4 * kk]);
            f4 m00, m1a, m1b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                m00[e] = tp < nv_o ? d00[e] * tl[3][e] : 0.f;
                m1a[e] = 16 + tp < nv_o ? d1a[e] * tl[4][e] : 0.f;
                m1b[e] = 16 + tp < nv_o ? d1b[e] * tl[5][e] : 0.f;
            }
            h4 hi, lo;
            split4<false>(m00, hi, lo, d.m1);
            _Float16 *mp = reinterpret_cast<_Float16 *>(vs + VH_MP);
            store_slot(mp, lane * 8, cat(hi, lo));
            h8 h1, l1;
            split8<false>(m1a, m1b, h1, l1, d.m1);
            store_slot(mp, 512 + lane * 8, h1);
            store_slot(mp, 1024 + lane * 8, l1);
        }
        // the wave's A writes must land before its lanes read them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        {
            // T = (I + A)^-1 by blocks: T00 = (I + A00)^-1 and T11 = (I + A11)^-1
            // by forward substitution at once (lane s < 16 keeps column s of
            // T00, lane 16 + s column s of T11; rows of A read four entries at
            // a time, entries at or right of the diagonal unused), then
            // T10 = -T11 A10 T00.
            if (lane < CT) {
                const int o = lane & 16, s = lane & 15;
                float Tc[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    float acc[4] = {(t == s) ? 1.f : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int r4 = 0; r4 < t; r4 += 4) {
                        const f4 a = *reinterpret_cast<const f4 *>(&sA[o + t][o + r4]);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            if (r4 + q < t) acc[q] = fmaf(-a[q], Tc[r4 + q], acc[q]);
                    }
                    Tc[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                }
#pragma unroll
                for (int t = 0; t < 16; ++t) sT[o + t][o + s] = Tc[t];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // fp32 MFMA 16x16x4 (lane (l16, kk) gives A[l16][kk], B[kk][l16] per
            // 4-deep step i), over the contraction order k = 4 kk + i so that
            // the first product's accumulator layout (W[4 kk + r][l16] in
            // component r) is the second's B operand as it stands:
            //   W = A10 T00,  T10 = -(T11 W)
            // (every operand read before the first product: a read issued while
            // a product is in flight may be given the registers of its operands)
            float wa[4], wb[4], ta[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                wa[i] = sA[16 + l16][4 * kk + i];
                wb[i] = sT[4 * kk + i][l16];
                ta[i] = sT[16 + l16][16 + 4 * kk + i];
            }
            __builtin_amdgcn_sched_barrier(0);
            f4 W = z4;
#pragma unroll
            for (int i = 0; i < 4; ++i) W = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[i], wb[i], W, 0, 0, 0);
            f4 T10 = z4;
#pragma unroll
            for (int i = 0; i < 4; ++i) T10 = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[i], W[i], T10, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) sT[16 + 4 * kk + r][l16] = -T10[r];
        }
        {
            // T in operand order, lane L = 16 kk + t':
            //   T00 (hi | lo): T[t'][4 kk + e];  T1: T[16 + t'][16 (e / 4) + 4 kk + e % 4]
            const f4 t00 = *reinterpret_cast<const f4 *>(&sT[l16][4 * kk]);
            const f4 t1a = *reinterpret_cast<const f4 *>(&sT[16 + l16][4 * kk]);
            const f4 t1b = *reinterpret_cast<const f4 *>(&sT[16 + l16][16 + 4 * kk]);
            h4 hi, lo;
            split4<false>(t00, hi, lo, d.m1);
            _Float16 *tp = reinterpret_cast<_Float16 *>(vs + VH_TP);
            store_slot(tp, lane * 8, cat(hi, lo));
            h8 h1, l1;
            split8<false>(t1a, t1b, h1, l1, d.m1);
            store_slot(tp, 512 + lane * 8, h1);
            store_slot(tp, 1024 + lane * 8, l1);
        }
        // every lane is done with A and T before the next head overwrites them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

constexpr int CHUNK_PREP_THREADS = 256;

__global__ __launch_bounds__(256) void scan_prep_kernel(ScanArgs p, PrepDims d)
{
    __shared__ __attribute__((aligned(16))) PrepShared sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
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

    // g and beta of this wave's first value head, lane l holding token l % 32
    // (requested first, so their latency overlaps the staging below)
    auto load_gb = [&](int gh, float &gl, float &bl) {
        const int t = lane & (CT - 1);
        const int64_t e = (tb + min(t, nv - 1)) * hv + j * d.G + gh;
        gl = t < nv ? p.g[e] : 0.f;
        bl = t < nv ? p.beta[e] : 0.f;
    };
    float g_next = 0.f, b_next = 0.f;
    if (wave < d.G) load_gb(wave, g_next, b_next);

    // stage the chunk's k and q rows of key head j (zero past the end)
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
        const int f = tid + 256 * k4;
        const int t = f >> 5, col = (f & 31) * 4;
        const int tc = min(t, nv - 1);
        const int64_t off = ((tb + tc) * hk + j) * 128 + col;
        const f4 kv = *reinterpret_cast<const f4 *>(p.kn + off);
        const f4 qv = *reinterpret_cast<const f4 *>(p.qn + off);
        *reinterpret_cast<f4 *>(&sm.u.kq.sK[t][col]) = t < nv ? kv : z4;
        *reinterpret_cast<f4 *>(&sm.u.kq.sQ[t][col]) = t < nv ? qv : z4;
    }
    __syncthreads();
    prep_body(sm, p.ws, d, j, chunk_slot(cu0, n, c), nv, g_next, b_next, load_gb);
}

struct ChunkDims {
    int hk, hv, G, n_seq;
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
// of the 128 keys; each of these four compute waves (0-3) holds its 16 x 64
// quarter of the block's state.  Wave 4 only copies operands into LDS; waves
// 5 and 6 form the outputs of row group 0 and 1 from what the compute waves
// leave in LDS.  With RAW_V wave 7 forms v of the block's channels from the
// raw fp16 qkv rows (conv with the history, SiLU) instead of the copy wave
// bringing vc.  Waves are dealt to the CU's four SIMDs in turn, so each SIMD
// holds one compute wave and at most one helper (the v wave, with the most
// arithmetic, on the SIMD of compute wave 3).
constexpr int CHUNK_WAVES = 4;                       // compute waves: 2 row groups x 2 key halves
constexpr int COPY_WAVE = 4, OUT_WAVE = 5, V_WAVE = 7;
constexpr int chunk_threads(bool raw_v) { return 64 * (raw_v ? 8 : 7); }
constexpr int CHUNK_ROWS = 32;                       // value channels per block
constexpr int KH_HALF_FLOATS = SCAN_KH_FLOATS / 2;   // K (or Q) of one key-head slot, in floats

// Block-wide barrier ordering LDS only: global copies in flight stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The copy, output and v waves' side of the same barrier.  They write LDS
// only through the copies, whose completion the copy wave waits for
// explicitly (vmcnt) before arriving, or with their own LDS stores, waited
// for here with their LDS reads.  The empty asm statements keep the compiler
// from moving memory operations across the barrier.  (The fenced form above
// would also wait for global stores and loads in flight, which the compute
// waves do not need.)
__device__ __forceinline__ void side_barrier()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// LDS rings: chunk c's K in sKP[c % 3] (read a step ahead for K S^T, and as
// K^T in step c); its value-head slot in sVH[c % 2]; with RAW_V its raw
// fp16 v rows in sRaw[c % 3]; its fp32 v in sV[c % 2].  Every member's size
// is a multiple of 256 bytes but the last.
template <bool RAW_V>
struct __attribute__((aligned(16))) ChunkShared {
    float sKP[3][KH_HALF_FLOATS];
    float sVH[2][SCAN_SLOT_FLOATS];
    _Float16 sRaw[RAW_V ? 3 : 1][CT][CHUNK_ROWS];
    float sV[2][CT][CHUNK_ROWS];
    // partial K S^T and Q S^T of every compute wave per token tile, and U of
    // each row group
    f4 sXP[2][CHUNK_WAVES][2][64];
    f4 sXR[2][CHUNK_WAVES][2][64];
    f4 sU[2][CHUNK_WAVES / 2][2][64];
    _Float16 sRawH[3][CHUNK_ROWS];
};

// With SIGNAL (the layer step that runs post in the same launch, one
// sequence), the output waves store o with device-scope stores and, once the
// stores of chunk c have completed, add 1 to the counter of (c, h): the eight
// output waves of value head h (four channel blocks, two row groups) take it
// to 8, after which every value of o of chunk c and head h is visible to a
// device-scope load anywhere on the device.  Each counter has a 256-byte line
// of its own (COUNT_STRIDE words): packed, the post waves' polls of a few
// lines slowed the whole chip (by ~30 us per layer).
struct OutSignal {
    uint32_t *count;
};
constexpr uint32_t O_WRITERS = 2 * (128 / CHUNK_ROWS);  // output waves per value head
constexpr int COUNT_STRIDE = 64;
__host__ __device__ __forceinline__ int64_t count_index(int c, int hv, int h)
{
    return ((int64_t)c * hv + h) * COUNT_STRIDE;
}

template <bool RAW_V, bool SIGNAL>
__device__ __forceinline__ void chunk_body(ChunkShared<RAW_V> &L, const ScanArgs &p, const ChunkDims &d,
                                           const VRawArgs &vr, const int bid, const OutSignal &sig)
{
    auto &sKP = L.sKP;
    auto &sVH = L.sVH;
    auto &sRaw = L.sRaw;
    auto &sRawH = L.sRawH;
    auto &sV = L.sV;
    auto &sXP = L.sXP;
    auto &sXR = L.sXR;
    auto &sU = L.sU;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, kk = lane >> 4;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};
    const h4 zh = {};

    // block -> (sequence n, value head h, channel block rb): the sequences'
    // ranges of hv * RB blocks in order of decreasing length, so the longest
    // recurrence starts first (up to SEQ_RANK_MAX sequences; beyond that in
    // index order); inside a range (a multiple of 8 blocks when hv is even)
    // the XCD-aware permutation
    constexpr int RB = 128 / CHUNK_ROWS;
    const int per_seq = d.hv * RB;
    const int rank = bid / per_seq;
    int w = bid - rank * per_seq;
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

    if (wave == COPY_WAVE) {
        // ---- copy wave: global -> LDS -----------------------------------
        // global_load_lds_dwordx4 moves 1 KB per instruction (lane i lands at
        // 16 i past the piece's LDS base) without passing through registers.
        typedef const void __attribute__((address_space(1))) *gptr_t;
        typedef void __attribute__((address_space(3))) *lptr_t;
        constexpr int K_PIECES = KH_HALF_FLOATS * 4 / 1024;                        // 16
        constexpr int VH_PIECES = SCAN_SLOT_FLOATS * 4 / 1024;                      // 6 (+ 512 B)
        // load instructions per issue_vh and issue_raw
        constexpr int VH_COPIES = VH_PIECES + 2 + (RAW_V ? 0 : 4);
        constexpr int RAW_COPIES = RAW_V ? 2 : 0;
        auto copy16 = [](const void *src, void *lds_piece) {
            __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_piece, 16, 0, 0);
        };
        auto copy4 = [](const void *src, void *lds_piece) {
            __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_piece, 4, 0, 0);
        };
        // Rows past the sequence's end read its last token (valid memory); the
        // slots give them zero weight (beta = Lam = 0, identity rows of T, zero
        // k and q), so they add exactly nothing.
        auto kh_src = [&](int c) {
            return p.ws + (chunk_slot(cu0, n, c) * hk + j) * SCAN_KH_FLOATS;
        };
        auto issue_k = [&](int c) {
            const float *src = kh_src(c) + lane * 4;
            float *dst = sKP[c % 3];
#pragma unroll
            for (int m = 0; m < K_PIECES; ++m) copy16(src + m * 256, dst + m * 256);
        };
        auto issue_vh = [&](int c) {
            const int b = c & 1;
            const float *vhs = p.ws + d.vh_base + (chunk_slot(cu0, n, c) * hv + h) * SCAN_SLOT_FLOATS;
#pragma unroll
            for (int m = 0; m < VH_PIECES; ++m)
                copy16(vhs + m * 256 + lane * 4, &sVH[b][m * 256]);
            // the last 512 bytes: two dword copies
            copy4(vhs + VH_PIECES * 256 + lane, &sVH[b][VH_PIECES * 256]);
            copy4(vhs + VH_PIECES * 256 + 64 + lane, &sVH[b][VH_PIECES * 256 + 64]);
            if constexpr (!RAW_V) {
                // fp32 v: lane l takes token 8 m + l / 8, channels 4 (l % 8) .. + 3
                const int64_t tb = (int64_t)cu0 + (int64_t)c * CT;
                const int nv = min(CT, T_n - c * CT);
                const float *vb = p.vc + (tb * hv + h) * 128 + rb * CHUNK_ROWS + (lane & 7) * 4;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int t = 8 * m + (lane >> 3);
                    copy16(vb + (uint32_t)min(t, nv - 1) * vstride, &sV[b][8 * m][0]);
                }
            }
        };
        auto issue_raw = [&](int c) {
            if constexpr (RAW_V) {
                // lane l: token 16 m + l / 4, raw channels 8 (l % 4) .. + 7 of
                // the block's 32, landing at sRaw[c % 3][16 m + l / 4][8 (l % 4)]
                const int64_t tb = (int64_t)cu0 + (int64_t)c * CT;
                const int nv = min(CT, T_n - c * CT);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int t = 16 * m + (lane >> 2);
                    const _Float16 *src = static_cast<const _Float16 *>(vr.qkv) +
                                          (tb + min(t, nv - 1)) * vr.C + (2 * hk + h) * 128 +
                                          rb * CHUNK_ROWS + (lane & 3) * 8;
                    copy16(src, &sRaw[c % 3][16 * m][0]);
                }
            }
        };
        // Issued after the barrier of step c (the compute waves are then done
        // with chunk c - 1), waited for before that of step c + 1: chunk
        // c + 2's K (read during step c + 1), chunk c + 1's value-head slot
        // and fp32 v, and with RAW_V chunk c + 2's raw rows (the v wave turns
        // them into v between the barriers of steps c + 1 and c + 2).
        // what is read before the barrier of step 0 first (chunk 0's K for
        // the compute waves' first products, its raw rows for the v wave),
        // then what is read after it
        issue_k(0);
        issue_raw(0);
        issue_vh(0);
        if (n_chunks > 1) {
            issue_k(1);
            issue_raw(1);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(K_PIECES + VH_COPIES + RAW_COPIES));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(VH_COPIES));
        }
        side_barrier();
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        for (int c = 0; c < n_chunks; ++c) {
            side_barrier();
            if (c + 2 < n_chunks) issue_k(c + 2);
            if (c + 1 < n_chunks) issue_vh(c + 1);
            if (c + 2 < n_chunks) issue_raw(c + 2);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        side_barrier();
        return;
    }
    if (wave == OUT_WAVE || wave == OUT_WAVE + 1) {
        // ---- output waves: O = (Lam R + M U) / sqrt(dk) of chunk c for row
        // group g, after the barrier of step c + 1.  R and U come from the
        // compute waves through LDS: written after the barrier of step c,
        // overwritten (for chunk c + 2) only after that of step c + 2.  Lam and
        // M are read from chunk c's value-head slot during step c (before the
        // copy of chunk c + 2 may replace it) and kept in registers.
        const int g = wave - OUT_WAVE;
        f4 lam0 = z4, lam1 = z4;
        h8 m0 = {}, m1h = {}, m1l = {};
        auto take_lam_m = [&](int c) {
            const float *vh = sVH[c & 1];
            lam0 = *reinterpret_cast<const f4 *>(vh + VH_LAM + 4 * kk);
            lam1 = *reinterpret_cast<const f4 *>(vh + VH_LAM + 16 + 4 * kk);
            const _Float16 *mp = reinterpret_cast<const _Float16 *>(vh + VH_MP);
            m0 = *reinterpret_cast<const h8 *>(mp + lane * 8);
            m1h = *reinterpret_cast<const h8 *>(mp + 512 + lane * 8);
            m1l = *reinterpret_cast<const h8 *>(mp + 1024 + lane * 8);
        };
        auto o_store = [&](int c) {
            const int x = c & 1;
            const int nv = min(CT, T_n - c * CT);
            const int64_t tb = (int64_t)cu0 + (int64_t)c * CT;
            const f4 R0 = sXR[x][2 * g][0][lane] + sXR[x][2 * g + 1][0][lane];
            const f4 R1 = sXR[x][2 * g][1][lane] + sXR[x][2 * g + 1][1][lane];
            h4 uh0, ul0, uh1, ul1;
            split4<true>(sU[x][g][0][lane], uh0, ul0, d.ms);
            split4<true>(sU[x][g][1][lane], uh1, ul1, d.ms);
            // M_hi x 2^-10 for the products with the scaled low half of U
            const h8 m0s = cat(lo_half(m0) * (_Float16)LO_UNSCALE, zh);
            const h8 m1hs = m1h * (_Float16)LO_UNSCALE;
            // tile 0: (M_hi + M_lo) U_hi over 16 tokens, then M_hi U_lo
            // (zero-padded to the same shape)
            f4 O0 = mfma_k32(m0, cat(uh0, uh0), lam0 * R0);
            O0 = mfma_k32(m0s, cat(ul0, zh), O0) * SCALE;
            // tile 1: 32-deep, the three split terms chained
            f4 O1 = mfma_k32(m1h, cat(uh0, uh1), lam1 * R1);
            O1 = mfma_k32(m1l, cat(uh0, uh1), O1);
            O1 = mfma_k32(m1hs, cat(ul0, ul1), O1) * SCALE;
            // straight from the accumulators: lane (l16, kk) writes channel l16
            // of tokens 4 kk + r and 16 + 4 kk + r (each store instruction
            // covers 64 contiguous bytes of four token rows)
            float *ob = p.o + (tb * hv + h) * 128 + rb * CHUNK_ROWS + g * 16 + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t0 = 4 * kk + r, t1 = 16 + 4 * kk + r;
                if constexpr (SIGNAL) {
                    if (t0 < nv)
                        __hip_atomic_store(ob + (uint32_t)t0 * vstride, O0[r], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    if (t1 < nv)
                        __hip_atomic_store(ob + (uint32_t)t1 * vstride, O1[r], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    if (t0 < nv) ob[(uint32_t)t0 * vstride] = O0[r];
                    if (t1 < nv) ob[(uint32_t)t1 * vstride] = O1[r];
                }
            }
        };
        auto count_chunk = [&](int c) {
            if (lane == 0)
                __hip_atomic_fetch_add(sig.count + count_index(c, hv, h), 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        };
        side_barrier();
        for (int c = 0; c < n_chunks; ++c) {
            side_barrier();
            // let the compute waves' reads that the recurrence waits for
            // reach the LDS first (~256 cycles)
            __builtin_amdgcn_s_sleep(4);
            if (c > 0) o_store(c - 1);
            if constexpr (SIGNAL) {
                if (c > 2) {
                    // Chunk c - 3 is counted once its stores have completed.
                    // The 16 stores of chunks c - 2 and c - 1 (full chunks:
                    // each o_store issues 8 store instructions) followed
                    // them, and vector-memory operations complete in order,
                    // so at most 16 outstanding means those are done; the
                    // stores were issued two steps ago, so the wait is
                    // normally over already.  The empty asm statements keep
                    // the compiler from moving memory operations across it.
                    __asm__ volatile("" ::: "memory");
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * 8));
                    __asm__ volatile("" ::: "memory");
                    count_chunk(c - 3);
                }
            }
            take_lam_m(c);
        }
        side_barrier();
        o_store(n_chunks - 1);
        if constexpr (SIGNAL) {
            wait_vmem_all();
            for (int c = max(0, n_chunks - 3); c < n_chunks; ++c) count_chunk(c);
        }
        return;
    }

    if constexpr (RAW_V) {
        if (wave == V_WAVE) {
            // ---- v wave: v of chunk c between the barriers of steps c - 1 and
            // c (the first: the initial barrier), into sV, from the raw rows the
            // copy wave brings (in LDS from the barrier of step c - 1 on).
            // Lane l takes tokens l / 4 and 16 + l / 4 of the chunk and value
            // channels 8 (l % 4) .. + 7 of the block's 32.  The arithmetic is
            // gdn_pre's (conv4, silu_fast), so v is bit for bit the staged
            // path's.
            const _Float16 *qkv = static_cast<const _Float16 *>(vr.qkv);
            const _Float16 *cw = static_cast<const _Float16 *>(vr.conv_w);
            _Float16 *hist = static_cast<_Float16 *>(vr.hist) + (int64_t)n * 3 * vr.C;
            const int C = vr.C;
            const int cv = (2 * hk + h) * 128 + rb * CHUNK_ROWS;  // the block's first raw channel
            const int tq = lane >> 2, g8 = (lane & 3) * 8;
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
            // taps of token t: raw rows t - 3 .. t, reaching into the previous
            // chunk's rows (or the history, for chunk 0)
            auto conv_chunk = [&](int c) {
                const int b = c % 3, pb = (c + 2) % 3, vb = c & 1;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int t = 16 * half + tq;
                    Raw8<_Float16> x[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int r = t + m - 3;
                        const _Float16 *rp = r >= 0 ? &sRaw[b][r][g8]
                                           : c == 0 ? &sRawH[3 + r][g8] : &sRaw[pb][CT + r][g8];
                        x[m].v = *reinterpret_cast<const h8 *>(rp);
                    }
                    f4 s0, s1;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float acc = conv4(w[e][0], w[e][1], w[e][2], w[e][3], x[0].get(e),
                                                x[1].get(e), x[2].get(e), x[3].get(e));
                        (e < 4 ? s0 : s1)[e & 3] = silu_fast(acc);
                    }
                    *reinterpret_cast<f4 *>(&sV[vb][t][g8]) = s0;
                    *reinterpret_cast<f4 *>(&sV[vb][t][g8 + 4]) = s1;
                }
            };
            // the weights and history rows arrive while the other waves
            // wait for chunk 0's operands (sRawH is this wave's own)
            side_barrier();
            wait_vmem_all();
            if (lane < 12) *reinterpret_cast<h8 *>(&sRawH[lane >> 2][g8]) = hrow.v;
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

    // this wave's two 32-key steps of K of both token tiles, hi and lo (at
    // positions pos = kpos(lane))
    auto key_ops = [&](const float *base, int pos, h8 (&hi)[2][2], h8 (&lo)[2][2]) {
        const _Float16 *kb = reinterpret_cast<const _Float16 *>(base);
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int s = 2 * kh + i;
                hi[tau][i] = *reinterpret_cast<const h8 *>(kb + kp_off(tau, s, 0) + pos * 8);
                lo[tau][i] = *reinterpret_cast<const h8 *>(kb + kp_off(tau, s, 1) + pos * 8);
            }
    };
    // K^T of key block b' = 4 kh + b (keys 16 b' .. + 15) from K's LDS copy
    // with the transposing read: in each 16-lane group kk, lane i gets short
    // i % 4 of the 8 bytes lane 4 jj + i / 4 addresses, for jj = 0..3, and
    // lane 4 jj + q addresses keys 16 b' + 4 q .. + 3 of token 16 tau + 4 kk +
    // jj, so lane (m, kk) receives K[16 tau + 4 kk + jj][16 b' + m]: the
    // update's A operand in the permuted token order.
    const int tr_off = kpos(16 * (l16 & 3) + 4 * kk + (l16 >> 2)) * 8;
    auto kt_half = [&](const float *base, int b, int hl, int tau) -> h4 {
        const int bp = 4 * kh + b;
        const _Float16 *q = reinterpret_cast<const _Float16 *>(base) + kp_off(tau, bp >> 1, hl) + tr_off +
                            4 * (bp & 1);
        return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4 *)q));
    };

    // K of chunk c + 1 is read from LDS during step c (it landed before the
    // barrier of step c).  The partial R = Q S^T of chunk c is formed at the
    // start of step c + 1, its products beside the split of the updated
    // state, from the split of the state before the update (kept) and Q of
    // chunk c; it reaches LDS before the barrier of step c + 1, after which
    // the output waves take it.  Q does not pass through LDS: each compute wave
    // loads its Q operands of chunk c + 1 from the key-head slot in global
    // memory (an L2 hit: twelve blocks share a slot) just before the barrier
    // of step c, where no product is in flight, into the register set of
    // chunk c - 1, whose R has been formed; sets alternate by chunk parity.
    lds_barrier();  // chunk 0's operands and chunk 1's K are in LDS
    h8 kph[2][2], kpl[2][2];
    key_ops(sKP[0], kpos(lane), kph, kpl);
    const _Float16 *qslot0 = reinterpret_cast<const _Float16 *>(p.ws + (int64_t)j * SCAN_KH_FLOATS) + KH_QP;
    // this wave's Q operands of chunk cq (the positions they have in the slot)
    auto q_load = [&](int cq, h8 (&qh)[2][2], h8 (&ql)[2][2]) {
        const _Float16 *qb = qslot0 + chunk_slot(cu0, n, cq) * hk * (int64_t)(2 * SCAN_KH_FLOATS);
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int s = 2 * kh + i;
                qh[tau][i] = *reinterpret_cast<const h8 *>(qb + kp_off(tau, s, 0) + lane * 8);
                ql[tau][i] = *reinterpret_cast<const h8 *>(qb + kp_off(tau, s, 1) + lane * 8);
            }
    };
    // chunk 0's Q in set A; set B holds zeros for the R of "chunk -1" that
    // step 0 stores into the exchange slot of chunk 1 (rewritten before
    // anything reads it)
    h8 qphA[2][2], qplA[2][2], qphB[2][2], qplB[2][2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 2; ++i) qphB[tau][i] = qplB[tau][i] = h8{};
    q_load(0, qphA, qplA);
    // partial R = Q S^T (x256) of chunk cr from the split (shp, slp) of the
    // state before its update
    auto r_partial = [&](int cr, const h8 (&shp)[2], const h8 (&slp)[2], const h8 (&qph)[2][2],
                         const h8 (&qpl)[2][2]) {
        const int xr = cr & 1;
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            // the two unscaled terms share one chain, the scaled one has its own
            f4 Rh = z4, Rl = z4;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                Rh = mfma_k32(qph[tau][i], shp[i], Rh);
                Rl = mfma_k32(qph[tau][i], slp[i], Rl);   // x LO_SCALE
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) Rh = mfma_k32(qpl[tau][i], shp[i], Rh);
            sXR[xr][wave][tau][lane] = Rh + Rl * LO_UNSCALE;
        }
    };
    int kb_cur = 0;  // ring slot of this chunk's K (c % 3)
    // one chunk step: (sh, sl) receive the split of this chunk's state,
    // (shp, slp) hold the previous chunk's
    auto step = [&](int c, h8 (&sh)[2], h8 (&sl)[2], const h8 (&shp)[2], const h8 (&slp)[2],
                    h8 (&qph)[2][2], h8 (&qpl)[2][2]) {
        const int x = c & 1;
        const int kb_next = kb_cur == 2 ? 0 : kb_cur + 1;
        const float *vh = sVH[x];
        // partial P = K S^T (x256) over this wave's 64 keys, per token tile
#pragma unroll
        for (int i = 0; i < 2; ++i) split8<true>(S4[2 * i], S4[2 * i + 1], sh[i], sl[i], d.ms);
        // K^T of this chunk for the update, read now while the LDS is quiet
        // (K landed before the previous barrier); after the split, which has
        // taken the last products' results, so no product is in flight
        __builtin_amdgcn_sched_barrier(0);
        h4 kt[4][2][2];  // [key block][hi/lo][token tile]
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                for (int tau = 0; tau < 2; ++tau) kt[b][hl][tau] = kt_half(sKP[kb_cur], b, hl, tau);
        __builtin_amdgcn_sched_barrier(0);
        // the previous chunk's partial R
        r_partial(c - 1, shp, slp, qph, qpl);
        f4 Pp[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            f4 Ph = z4, Pl = z4;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                Ph = mfma_k32(kph[tau][i], sh[i], Ph);
                Pl = mfma_k32(kph[tau][i], sl[i], Pl);   // x LO_SCALE
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) Ph = mfma_k32(kpl[tau][i], sh[i], Ph);
            Pp[tau] = Ph + Pl * LO_UNSCALE;
            sXP[x][wave][tau][lane] = Pp[tau];
        }
        // chunk c + 1's Q into the set R of chunk c - 1 has just used (the
        // products' results are stored, so none is in flight)
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 < n_chunks) q_load(c + 1, qph, qpl);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();  // partials visible; every wave is past chunk c - 1
        __builtin_amdgcn_sched_barrier(0);  // nothing below moves up before the barrier

        // Reads in the order they are needed, since each wave's LDS reads
        // complete in order and four waves read at once after the barrier:
        // what B needs (the partner's partial P, Lam, beta, v); then T and
        // the last-row decays; the next chunk's K once U is formed.
        const f4 Po0 = sXP[x][partner][0][lane];
        const f4 Po1 = sXP[x][partner][1][lane];
        const f4 lam0 = *reinterpret_cast<const f4 *>(vh + VH_LAM + 4 * kk);
        const f4 lam1 = *reinterpret_cast<const f4 *>(vh + VH_LAM + 16 + 4 * kk);
        const f4 bet0 = *reinterpret_cast<const f4 *>(vh + VH_BETA + 4 * kk);
        const f4 bet1 = *reinterpret_cast<const f4 *>(vh + VH_BETA + 16 + 4 * kk);
        f4 vv0, vv1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            vv0[r] = sV[x][4 * kk + r][grp * 16 + l16];
            vv1[r] = sV[x][16 + 4 * kk + r][grp * 16 + l16];
        }
        __builtin_amdgcn_sched_barrier(0);
        // the full P, summed in the same order by both waves of the pair;
        // B = beta (V - Lam P), component r is token 16 tau + 4 kk + r, channel l16
        const f4 P0 = kh == 0 ? Pp[0] + Po0 : Po0 + Pp[0];
        const f4 P1 = kh == 0 ? Pp[1] + Po1 : Po1 + Pp[1];
        f4 B0, B1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            B0[r] = bet0[r] * __builtin_fmaf(-lam0[r], P0[r], vv0[r]);
            B1[r] = bet1[r] * __builtin_fmaf(-lam1[r], P1[r], vv1[r]);
        }
        const _Float16 *tpp = reinterpret_cast<const _Float16 *>(vh + VH_TP);
        const h8 tp0 = *reinterpret_cast<const h8 *>(tpp + lane * 8);
        const h8 tp1h = *reinterpret_cast<const h8 *>(tpp + 512 + lane * 8);
        const h8 tp1l = *reinterpret_cast<const h8 *>(tpp + 1024 + lane * 8);
        const f4 wu0 = *reinterpret_cast<const f4 *>(vh + VH_W + 4 * kk);
        const f4 wu1 = *reinterpret_cast<const f4 *>(vh + VH_W + 16 + 4 * kk);
        const float last = vh[VH_LAST];
        __builtin_amdgcn_sched_barrier(0);

        h4 bh0, bl0, bh1, bl1;
        split4<true>(B0, bh0, bl0, d.ms);
        split4<true>(B1, bh1, bl1, d.ms);
        // U = T B.  Tile 0 (16-deep): (T_hi + T_lo) B_hi, then T_hi B_lo with
        // T_hi x 2^-10 (zero-padded); tile 1 (32-deep over the permuted
        // tokens): T_hi B_hi, T_lo B_hi, (T_hi x 2^-10) B_lo, chained.
        const h8 t0s = cat(lo_half(tp0) * (_Float16)LO_UNSCALE, zh);
        const h8 t1s = tp1h * (_Float16)LO_UNSCALE;
        f4 U0 = mfma_k32(tp0, cat(bh0, bh0), z4);
        U0 = mfma_k32(t0s, cat(bl0, zh), U0);
        const h8 bhh = cat(bh0, bh1);
        f4 U1 = mfma_k32(tp1h, bhh, z4);
        U1 = mfma_k32(tp1l, bhh, U1);
        U1 = mfma_k32(t1s, cat(bl0, bl1), U1);
        if (kh == 0) {
            sU[x][grp][0][lane] = U0;
            sU[x][grp][1][lane] = U1;
        }
        h4 uwh0, uwl0, uwh1, uwl1;
        split4<true>(U0 * wu0, uwh0, uwl0, d.ms);
        split4<true>(U1 * wu1, uwh1, uwl1, d.ms);
        const h8 uwh = cat(uwh0, uwh1), uwl = cat(uwl0, uwl1);
        // (here no product of this step is in flight: a load issued while one
        // is may be given the registers of its operands, see tests/asm_hazards.py)
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 < n_chunks) key_ops(sKP[kb_next], kpos(lane), kph, kpl);
        __builtin_amdgcn_sched_barrier(0);
        // 16 S' = Lam_last (16 S) + (16 K)^T (D[last] U) over the 32 permuted
        // tokens: this wave's 4 key blocks, three split terms chained each
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const h8 kth = cat(kt[b][0][0], kt[b][0][1]);
            const h8 ktl = cat(kt[b][1][0], kt[b][1][1]);
            f4 C = mfma_k32(kth, uwh, S4[b] * last);
            C = mfma_k32(ktl, uwh, C);
            S4[b] = mfma_k32(kth * (_Float16)LO_UNSCALE, uwl, C);
        }
        kb_cur = kb_next;
    };
    // two steps per turn, so that the two splits alternate between register
    // sets instead of being copied
    h8 shA[2] = {}, slA[2] = {}, shB[2] = {}, slB[2] = {};
    int c = 0;
    for (; c + 1 < n_chunks; c += 2) {
        step(c, shA, slA, shB, slB, qphB, qplB);
        step(c + 1, shB, slB, shA, slA, qphA, qplA);
    }
    if (c < n_chunks) {
        step(c, shA, slA, shB, slB, qphB, qplB);
        r_partial(c, shA, slA, qphA, qplA);
    } else {
        r_partial(c - 1, shB, slB, qphB, qplB);
    }
    lds_barrier();  // R and U of the last chunk are visible to the output wave
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<f4 *>(Srow + 16 * i) = S4[i] * (1.f / KQ_SCALE);
}

template <bool RAW_V>
__global__ __launch_bounds__(chunk_threads(RAW_V)) void scan_chunk_kernel(ScanArgs p, ChunkDims d,
                                                                         VRawArgs vr)
{
    __shared__ ChunkShared<RAW_V> L;
    chunk_body<RAW_V, false>(L, p, d, vr, (int)blockIdx.x, OutSignal{nullptr});
}

static int64_t scan_slots(const gdn_shape &s)
{
    return s.total_T / CT + (int64_t)s.n_seq + 1;
}

// ---- the layer's pre stage fused into the prep step ------------------------
//
// With fp32 io, one block per (chunk, key head j) computes, for the chunk's
// 32 tokens, the pre stage of exactly the channels the prep step needs: q and
// k of key head j (conv, SiLU, L2 norm) straight into LDS, the group's gates,
// and v of the group's value heads (conv, SiLU) to the vc buffer the chunk
// kernel reads; then it builds the slots like scan_prep_kernel.  (With fp16
// io, layer_prep_f16_kernel below does the same for q, k and the gates, and
// the chunk kernel forms v from the raw rows.)  The normalised q and k and the
// gates never go through memory.  The arithmetic is that of gdn_pre (the same
// per-element expressions), so the layer's results equal the staged path's
// bit for bit.  History carry without a race: only the chunk-0 blocks read
// the old history, each for its own channels, and the same block writes the
// new history of those channels after a barrier.
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

    // Tasks (unit u, token part) of 8 tokens x 128 channels, one per 16-lane
    // row at a time: u = 0 q of key head j, u = 1 its k, u = 2 + gh v of
    // value head j G + gh; each unit's 32 tokens in 4 parts.  Lane l16 of the
    // row takes channels 4 l16 .. + 3 and 64 + 4 l16 .. + 3 of the unit (every
    // memory instruction covers whole 64-channel runs).  A task issues its
    // weight loads and the rows of X its tokens read, all unconditional (rows
    // past the chunk's end repeat its last row), waits for them once, and then
    // walks its tokens with no load behind a store.
    constexpr int P = CT / 8;
    const int units = 2 + G;
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
        const int t0 = 8 * part;
        const int nt = max(0, min(8, nv - t0));  // valid tokens of this task
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
        for (int i = 0; i < 11; ++i) x[i].load_split(xrow_ptr(min(xb + i, x_last), ch));
        wait_vmem_all();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
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
                float *dst = u == 0 ? &sm.u.kq.sQ[t][l16 * 4] : &sm.u.kq.sK[t][l16 * 4];
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
        gl = sGate[gh][0][lane & (CT - 1)];
        bl = sGate[gh][1][lane & (CT - 1)];
    };
    float g_next = 0.f, b_next = 0.f;
    if (wave < G) load_gb(wave, g_next, b_next);
    prep_body(sm, p.ws, d, j, chunk_slot(cu0, n, c), nv, g_next, b_next, load_gb);
}

// The fp16 layer path's prep step: what layer_prep_kernel does, without v
// (the chunk kernel forms it).  Each 16-lane row has one task, q or k of key
// head j for four of the chunk's tokens, with all its loads issued up front.
// Same per-element arithmetic as gdn_pre, so the results equal the staged
// path's bit for bit.
static_assert(LAYER_G_MAX * CT <= CHUNK_PREP_THREADS, "one gate pair per thread");
__global__ __launch_bounds__(256) void layer_prep_f16_kernel(LayerPrepArgs p, PrepDims d)
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
    const int hk = d.hk, hv = d.hv, G = d.G, C = d.C;
    if (p.sync) {
        // (one sequence) the counters of chunk c's value heads of this group,
        // and the status word, start at zero for the chunk kernel's post role
        if (tid < G) p.sync[count_index(c, hv, j * G + tid)] = 0;
        if (c == 0 && j == 0 && tid == 0) p.sync[count_index(d.n_chunk_max, hv, 0)] = 0;
    }
    const _Float16 *qkv = static_cast<const _Float16 *>(p.qkv);
    const _Float16 *cw = static_cast<const _Float16 *>(p.conv_w);
    _Float16 *hist = static_cast<_Float16 *>(p.hist) + (int64_t)n * 3 * C;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};

    // task of this row: unit u (0: q, 1: k of key head j), tokens t0 .. t0 + 3;
    // lane l16 takes channels 4 l16 .. + 3 and 64 + 4 l16 .. + 3
    const int task = wave * 4 + (lane >> 4);
    const int u = task >> 3, t0 = 4 * (task & 7);
    const int ch = (u == 0 ? j : hk + j) * 128 + l16 * 4;
    // row xi of X = [history (3 rows); the sequence's tokens], channel c
    auto xrow = [&](int64_t xi, int cc) { return xi < 3 ? hist + xi * C + cc : qkv + (cu0 + xi - 3) * C + cc; };
    // weights (fp16, element (4 m + tap) of the lane's channel m = 0..7), then
    // the seven X rows of the task's four tokens; rows past the chunk's end
    // repeat its last row (valid memory, results unused)
    Raw8<_Float16> wr[4], xa[7];
    // the gate inputs of pair tid = (value head gh of the group, token t),
    // requested with the rows so that their latency overlaps them (pairs
    // past the chunk's end, and threads past G * CT, load nothing)
    const int gh_t = tid / CT, gt_t = tid - gh_t * CT;
    const bool gate_t = tid < G * CT, gate_ld = gate_t && gt_t < nv;
    _Float16 ga = 0, gdt = 0, gal = 0, gb = 0;
    if (gate_ld) {
        const int h = j * G + gh_t;
        const int64_t e = ((int64_t)cu0 + c * CT + gt_t) * hv + h;
        ga = static_cast<const _Float16 *>(p.a)[e];
        gb = static_cast<const _Float16 *>(p.b)[e];
        gdt = static_cast<const _Float16 *>(p.dt_bias)[h];
        gal = static_cast<const _Float16 *>(p.A_log)[h];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) wr[k].load(cw + (int64_t)(ch + 64 * (k >> 1)) * 4 + (k & 1) * 8);
#pragma unroll
    for (int i = 0; i < 7; ++i)
        xa[i].load_split(xrow(min((int64_t)c * CT + t0 + i, (int64_t)c * CT + nv + 2), ch));
    {
        const int nt = max(0, min(4, nv - t0));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + i;
            float sv[8];
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float acc = conv4(wr[e >> 1].get((e & 1) * 4 + 0), wr[e >> 1].get((e & 1) * 4 + 1),
                                        wr[e >> 1].get((e & 1) * 4 + 2), wr[e >> 1].get((e & 1) * 4 + 3),
                                        xa[i].get(e), xa[i + 1].get(e), xa[i + 2].get(e), xa[i + 3].get(e));
                sv[e] = silu_fast(acc);
                ss = fmaf(sv[e], sv[e], ss);
            }
            ss = row_sum16(ss);
            const float sc = rsqrt_fast(ss + d.eps_l2);
            float *dst = u == 0 ? &sm.u.kq.sQ[t][l16 * 4] : &sm.u.kq.sK[t][l16 * 4];
            *reinterpret_cast<f4 *>(dst) = i < nt ? f4{sv[0] * sc, sv[1] * sc, sv[2] * sc, sv[3] * sc} : z4;
            *reinterpret_cast<f4 *>(dst + 64) = i < nt ? f4{sv[4] * sc, sv[5] * sc, sv[6] * sc, sv[7] * sc} : z4;
        }
    }

    // gates of the group's value heads, token t of head gh at sGate[gh][.][t]
    // (zero past the end)
    if (gate_t) {
        float g = 0.f, bt = 0.f;
        if (gate_ld) gates((float)ga, (float)gdt, (float)gal, (float)gb, g, bt);
        sGate[gh_t][0][gt_t] = g;
        sGate[gh_t][1][gt_t] = bt;
    }
    __syncthreads();

    // the new history of q and k of key head j (the block of chunk 0): X rows
    // T_n .. T_n + 2; for T_n + r < 3 that is old history row T_n + r > r,
    // not yet overwritten: all three are read before the first write
    if (c == 0 && tid < 32) {
        const int hc = ((tid >> 4) == 0 ? j : hk + j) * 128 + l16 * 4;
        Raw8<_Float16> v[3];
#pragma unroll
        for (int r = 0; r < 3; ++r) v[r].load_split(xrow((int64_t)T_n + r, hc));
        wait_vmem_all();
#pragma unroll
        for (int r = 0; r < 3; ++r) v[r].store_split(hist + (int64_t)r * C + hc);
    }

    auto load_gb = [&](int gh, float &gl, float &bl) {
        gl = sGate[gh][0][lane & (CT - 1)];
        bl = sGate[gh][1][lane & (CT - 1)];
    };
    float g_next = 0.f, b_next = 0.f;
    if (wave < G) load_gb(wave, g_next, b_next);
    prep_body(sm, p.ws, d, j, chunk_slot(cu0, n, c), nv, g_next, b_next, load_gb);
}

// ---- post in the chunk kernel's launch ------------------------------------
//
// The chunk kernel leaves CUs idle (one block per (value head, 32 channels):
// 192 blocks for 48 value heads on 256 CUs) and finishes o chunk by chunk,
// while post needs all 128 channels of a (token, value head) row, which four
// chunk blocks hold.  Here blocks past the chunk blocks run post: each wave
// takes units (chunk c, value head h) in chunk order, waits until the eight
// output waves of head h have counted chunk c (OutSignal), reads its 32 rows
// of o with device-scope loads and writes y (the post kernel's arithmetic,
// post_row).  The post blocks have the highest indices, so the chunk blocks,
// which wait for nothing, are dispatched first: the launch completes whatever
// the number of CUs.  A wait is bounded; past the bound the unit is computed
// from whatever o holds (the results are then undefined) and bit 0 of the
// status word is set.  Units of the value heads of XCD x run on XCD x (blocks
// are dealt to the 8 XCDs in turn; the chunk blocks' permutation puts the
// heads x hv / 8 .. there).
struct PostRoleArgs {
    const uint32_t *count;
    uint32_t *status;
    const _Float16 *z, *gamma;
    void *y;
    float eps;
    int chunk_blocks, np;  // chunk blocks, post blocks
    int T;                 // tokens of the one sequence
    int xcd_affine;
    int max_polls;         // polls before a wait gives up
};
// polls before a wait gives up: one sleeps ~0.8 us and waits for a load, so
// 2^15 of them take roughly 30-100 ms
constexpr int POST_WAIT_POLLS = 1 << 15;

template <typename TO>
__device__ __forceinline__ void post_role(const ScanArgs &p, const ChunkDims &d, const PostRoleArgs &pa)
{
    const int pb = (int)blockIdx.x - pa.chunk_blocks;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, l16 = lane & 15, rr = lane >> 4;
    const int hv = d.hv;
    const int n_chunks = (pa.T + CT - 1) / CT;
    float gm[8];
    load8_split(pa.gamma + l16 * 4, gm);
    // units of this wave: XCD x = block % 8 takes heads hx x .. hx x + hx - 1
    const int nw = pa.np * 8;  // post waves
    int first, step, per_xcd_heads = 0;
    if (pa.xcd_affine) {
        per_xcd_heads = hv >> 3;
        first = (pb >> 3) * 8 + wave;
        step = nw >> 3;
    } else {
        first = pb * 8 + wave;
        step = nw;
    }
    const int n_units = pa.xcd_affine ? n_chunks * per_xcd_heads : n_chunks * hv;
    bool gave_up = false;
    for (int u = first; u < n_units; u += step) {
        int c, h;
        if (pa.xcd_affine) {
            c = u / per_xcd_heads;
            h = (pb & 7) * per_xcd_heads + (u - c * per_xcd_heads);
        } else {
            c = u / hv;
            h = u - c * hv;
        }
        // z does not depend on the chunk step: requested before the wait
        const int nv = min(CT, pa.T - c * CT);
        const int64_t row0 = (int64_t)c * CT * hv + h;
        float zz[8][8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int tc = min(4 * i + rr, nv - 1);
            load8_split(pa.z + (row0 + (int64_t)tc * hv) * 128 + l16 * 4, zz[i]);
        }
        const uint32_t *cnt = pa.count + count_index(c, hv, h);
        for (int it = 0; !gave_up; ++it) {
            const uint32_t v = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (v >= O_WRITERS) break;
            if (it >= pa.max_polls) {
                gave_up = true;
                if (lane == 0) __hip_atomic_fetch_or(pa.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            // the last chunks: the launch ends with them, poll often
            if (c + 4 >= n_chunks) __builtin_amdgcn_s_sleep(2);
            else __builtin_amdgcn_s_sleep(30);
        }
        // rows (token 4 i + rr of the chunk), lane l16 takes channels 4 l16 ..
        // + 3 and 64 + 4 l16 .. + 3; o through a buffer descriptor based at the
        // unit's first row (offsets stay small), device-scope loads (sc1)
        __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(p.o + row0 * 128), (short)0, 0x7fffffff, 0x00020000);
        const uint32_t rstride = (uint32_t)hv * 128 * 4;  // bytes per token
        f4 oa[8], ob[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = 4 * i + rr;
            const int tc = min(t, nv - 1);  // rows past the end: the last row, unused
            const uint32_t off = (uint32_t)tc * rstride + (uint32_t)l16 * 16;
            oa[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 16));
            ob[i] = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(ro, off + 256, 0, 16));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = 4 * i + rr;
            const float x[8] = {oa[i][0], oa[i][1], oa[i][2], oa[i][3], ob[i][0], ob[i][1], ob[i][2], ob[i][3]};
            float out[8];
            post_row(x, zz[i], gm, pa.eps, out);
            if (t < nv) store8_split(static_cast<TO *>(pa.y) + (row0 + (int64_t)t * hv) * 128 + l16 * 4, out);
        }
    }
}

template <typename TO>
__global__ __launch_bounds__(chunk_threads(true)) void layer_chunk_post_kernel(ScanArgs p, ChunkDims d,
                                                                               VRawArgs vr, PostRoleArgs pa)
{
    __shared__ ChunkShared<true> L;
    if ((int)blockIdx.x < pa.chunk_blocks) {
        chunk_body<true, true>(L, p, d, vr, (int)blockIdx.x, OutSignal{const_cast<uint32_t *>(pa.count)});
        return;
    }
    post_role<TO>(p, d, pa);
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

static ChunkDims chunk_dims(const gdn_shape &s)
{
    ChunkDims cd;
    cd.hk = s.hk;
    cd.hv = s.hv;
    cd.G = s.hv / s.hk;
    cd.n_seq = s.n_seq;
    cd.vh_base = scan_slots(s) * s.hk * SCAN_KH_FLOATS;
    cd.ms = -LO_SCALE;
    return cd;
}

static int64_t chunk_blocks(const gdn_shape &s) { return (int64_t)s.n_seq * s.hv * (128 / CHUNK_ROWS); }

static hipError_t launch_chunk(const gdn_shape &s, const ScanArgs &a, hipStream_t st,
                               const VRawArgs *vr = nullptr)
{
    const ChunkDims cd = chunk_dims(s);
    const int64_t blocks = chunk_blocks(s);
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

// Compute units of the current device (0 if the runtime cannot say), looked
// up once per device.
static int device_cus()
{
    constexpr int kMaxDevices = 256;
    static std::atomic<int> cus[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Post blocks of the chunk launch for a shape (0: post runs as its own
// launch): one sequence of fp16 rows, and at least 32 CUs left by the chunk
// blocks (a multiple of 8, at most 64).  GDN_LAYER_POST_FUSED=0 in the
// environment selects the separate launch.
constexpr int POST_NP_MIN = 32, POST_NP_MAX = 64;
static int post_blocks(const gdn_shape &s)
{
    if (s.io_dtype != GDN_F16 || s.n_seq != 1) return 0;
    const char *e = getenv("GDN_LAYER_POST_FUSED");
    if (e && e[0] == '0') return 0;
    const int64_t free_cus = (int64_t)device_cus() - chunk_blocks(s);
    const int np = (int)(std::min<int64_t>(free_cus, POST_NP_MAX) & ~(int64_t)7);
    return np >= POST_NP_MIN ? np : 0;
}

// counters (one 256-byte line each) and the status word (a line of its own)
size_t layer_sync_bytes(const gdn_shape &s)
{
    return ((size_t)(s.max_T + CT - 1) / CT * s.hv + 1) * COUNT_STRIDE * sizeof(uint32_t);
}

template <typename TO>
static hipError_t launch_chunk_post(const gdn_shape &s, const ScanArgs &a, const VRawArgs &vr,
                                    const PostRoleArgs &pa, hipStream_t st)
{
    hipLaunchKernelGGL(layer_chunk_post_kernel<TO>, dim3((unsigned)(pa.chunk_blocks + pa.np)),
                       dim3(chunk_threads(true)), 0, st, a, chunk_dims(s), vr, pa);
    return hipGetLastError();
}

hipError_t launch_layer_scan(const gdn_shape &s, const LayerPrepArgs &lp0, const ScanArgs &a,
                             const PostArgs *post, bool *post_done, hipStream_t st)
{
    const PrepDims pd = prep_dims(s);
    const dim3 grid((unsigned)(s.n_seq * (int64_t)pd.n_chunk_max), s.hk);
    if (post_done) *post_done = false;
    if (s.io_dtype == GDN_F16) {
        const int np = post && post_done && lp0.sync ? post_blocks(s) : 0;
        LayerPrepArgs lp = lp0;
        if (np == 0) lp.sync = nullptr;
        // v of the value heads is formed in the chunk kernel (VRawArgs)
        hipLaunchKernelGGL(layer_prep_f16_kernel, grid, dim3(CHUNK_PREP_THREADS), 0, st, lp, pd);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const VRawArgs vr{lp.qkv, lp.conv_w, lp.hist, pd.C};
        if (np == 0) return launch_chunk(s, a, st, &vr);
        PostRoleArgs pa;
        pa.count = lp.sync;
        pa.status = lp.sync + count_index(pd.n_chunk_max, s.hv, 0);
        pa.z = static_cast<const _Float16 *>(post->z);
        pa.gamma = static_cast<const _Float16 *>(post->gamma);
        pa.y = post->y;
        pa.eps = s.eps_rms;
        pa.chunk_blocks = (int)chunk_blocks(s);
        pa.np = np;
        pa.T = (int)s.total_T;
        pa.xcd_affine = s.hv % 8 == 0 && pa.chunk_blocks % 8 == 0;
        // (GDN_POST_WAIT_POLLS in the environment lowers the bound, so that
        // a test can take the give-up path without anything going wrong)
        pa.max_polls = POST_WAIT_POLLS;
        if (const char *e = getenv("GDN_POST_WAIT_POLLS")) pa.max_polls = std::max(0, std::min(atoi(e), POST_WAIT_POLLS));
        e = s.out_dtype == GDN_F16 ? launch_chunk_post<_Float16>(s, a, vr, pa, st)
                                   : launch_chunk_post<float>(s, a, vr, pa, st);
        if (e == hipSuccess) *post_done = true;
        return e;
    }
    hipLaunchKernelGGL(layer_prep_kernel<float>, grid, dim3(CHUNK_PREP_THREADS), 0, st, lp0, pd);
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
