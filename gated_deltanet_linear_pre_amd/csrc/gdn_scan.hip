// gdn_scan.hip -- the gated delta rule on an fp32 state, in 16-token chunks on
// fp32 MFMA.
//
// "Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1
// (gdn_scan_r findings): one state per value head, updated token by token in
// the same pass that forms the dot products against the old state; section 2:
// a token-blocked run must equal the single pass.
//
// The recurrence, per value head h (key head j = h / G), state S (dv x dk):
//   S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
//   o_t = S_t q_t / sqrt(dk),  alpha_t = exp(g_t).
// Over a chunk of C = 16 tokens starting from state S0, with
//   D[t][s] = exp(g_{s+1} + ... + g_t)    (decay from just after s to t, <= 1)
//   Lam_t   = exp(g_0 + ... + g_t)        (decay from the chunk start)
// the writes u_t = beta_t (v_t - alpha_t S_{t-1} k_t) solve a unit lower
// triangular system, and the outputs and the next state follow:
//   (I + A) U = diag(beta) (V - diag(Lam) P),  A[t][s] = beta_t D[t][s] k_t.k_s (s<t)
//   O  = diag(Lam) R + M U,                     M[t][s] = D[t][s] q_t.k_s     (s<=t)
//   S' = Lam_last S0 + sum_s D[last][s] u_s k_s^T
// with P = K S0^T, R = Q S0^T (tokens x value channels).  This is exact
// algebra of the recurrence (unroll S_t = Lam_t S0 + sum_{s<=t} D[t][s] u_s k_s^T).
// Every decay is formed as exp of a sum of at most 16 log decays, never as a
// ratio of two cumulative products, so nothing overflows or cancels.
//
// gfx950 mapping.
// * gdn_scan_prep (fully parallel over sequence x chunk x key head): k.k and
//   q.k of the chunk on MFMA (once per key head, shared by its G value heads),
//   then per value head the decays, T = (I + A)^-1 by forward substitution (one
//   column per lane, in registers), M, Lam, beta and the last-row decays.  The
//   result goes to one slot per (chunk, value head) of the workspace.
// * gdn_scan_chunk (sequential over chunks): a block of 4 waves owns 32 value
//   channels of one (sequence, value head).  Each wave holds a 16-channel x
//   64-key quarter of the state in MFMA accumulator layout (16 VGPRs/lane).
//   Per chunk: K S0^T and Q S0^T over the wave's 64 keys (32 MFMA
//   16x16x4 f32), the partial sums of the two key halves exchanged through
//   LDS, U = T B (4 MFMA), O = Lam R + M U (4 MFMA, one wave per pair), and the
//   state update Lam_last S0 + (D K)^T U (16 MFMA).  The state never leaves
//   registers, and every product consumes the accumulator layout the previous
//   one produced: the contraction index is permuted consistently, so no
//   transposes are needed.
//   The next chunk's K, Q, V and prep slot are loaded into registers while the
//   current chunk computes.
// * Block order is XCD-aware (blocks are dealt round-robin to the 8 XCDs; the
//   index is permuted so each XCD gets whole heads and whole key-head groups,
//   sharing their K/Q stream in one L2).
//
// Determinism: fixed-order MFMA chains, no atomics; the two waves of a
// channel block add the key halves in the same order, so they agree bit for
// bit.  Splitting a sequence at a multiple of 16 tokens gives bit-identical
// results; other split points agree within rounding (the chunk grid moves).
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int CT = 16;    // tokens per chunk
constexpr int KS = 132;   // LDS row stride of the K/Q chunk (padded)
// prep slot layout (floats)
constexpr int OFF_T = 0;      // T = (I + A)^-1, [t][s]
constexpr int OFF_M = 256;    // M / sqrt(dk), [t][s]
constexpr int OFF_LAM = 512;  // Lam_t
constexpr int OFF_LAMS = 528; // Lam_t / sqrt(dk)
constexpr int OFF_BETA = 544; // beta_t (0 past the chunk's end)
constexpr int OFF_W = 560;    // D[last][s] (0 past the end)
constexpr int OFF_LAST = 576; // Lam_last
static_assert(SCAN_SLOT_FLOATS >= 580 && SCAN_SLOT_FLOATS % 4 == 0, "slot too small");

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c)
{
    // D[i][j] += sum_k A[i][k] B[k][j], 16x16x4: lane l supplies A[l%16][l/16]
    // and B[l/16][l%16]; D[4(l/16)+r][l%16] comes back in component r.
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Workspace slot of chunk c of sequence n (cu0 = cu[n]); injective, and
// below total_T / 16 + n_seq.
__device__ __forceinline__ int64_t chunk_slot(int cu0, int n, int c)
{
    return (int64_t)(cu0 >> 4) + c + n;
}

struct PrepDims {
    int hk, hv, G, n_chunk_max;
};

__global__ __launch_bounds__(256) void scan_prep_kernel(ScanArgs p, PrepDims d)
{
    __shared__ __attribute__((aligned(16))) float sK[CT][KS];
    __shared__ __attribute__((aligned(16))) float sQ[CT][KS];
    __shared__ float sKK[CT][CT + 1];
    __shared__ float sQK[CT][CT + 1];
    __shared__ float sA[4][CT][CT + 1];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, kk = lane >> 4;
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

    // stage the chunk's k and q rows of key head j (zero past the end)
#pragma unroll
    for (int f2 = 0; f2 < 2; ++f2) {
        const int f = tid + 256 * f2;
        const int t = f >> 5, col = (f & 31) * 4;
        const int tc = min(t, nv - 1);
        const int64_t off = ((tb + tc) * hk + j) * 128 + col;
        const f4 kv = *reinterpret_cast<const f4 *>(p.kn + off);
        const f4 qv = *reinterpret_cast<const f4 *>(p.qn + off);
        *reinterpret_cast<f4 *>(&sK[t][col]) = t < nv ? kv : z4;
        *reinterpret_cast<f4 *>(&sQ[t][col]) = t < nv ? qv : z4;
    }
    __syncthreads();

    // wave 0: K K^T, wave 1: Q K^T (16 x 16 over 128 keys, 32 MFMA each)
    if (wave < 2) {
        const float(*X)[KS] = wave == 0 ? sK : sQ;
        f4 acc = z4;
#pragma unroll
        for (int jb = 0; jb < 8; ++jb) {
            const f4 xa = *reinterpret_cast<const f4 *>(&X[l16][16 * jb + 4 * kk]);
            const f4 kb = *reinterpret_cast<const f4 *>(&sK[l16][16 * jb + 4 * kk]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc = mfma4(xa[r], kb[r], acc);
        }
        float(*O)[CT + 1] = wave == 0 ? sKK : sQK;
#pragma unroll
        for (int r = 0; r < 4; ++r) O[4 * kk + r][l16] = acc[r];
    }
    __syncthreads();

    const float scale = 0.08838834764831845f;  // 1 / sqrt(128)
    for (int gh = wave; gh < d.G; gh += 4) {
        const int h = j * d.G + gh;
        float *slot = p.ws + (chunk_slot(cu0, n, c) * hv + h) * SCAN_SLOT_FLOATS;
        float gv[CT], bv[CT];
#pragma unroll
        for (int t = 0; t < CT; ++t) {
            const int tc = min(t, nv - 1);
            const float gg = p.g[(tb + tc) * hv + h];
            const float bb = p.beta[(tb + tc) * hv + h];
            gv[t] = t < nv ? gg : 0.f;
            bv[t] = t < nv ? bb : 0.f;
        }
        // A (to LDS) and M (to the slot): entry (t, s), four per lane
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int e = lane + 64 * m;
            const int t = e >> 4, s = e & 15;
            float sum = 0.f;
#pragma unroll
            for (int r = 1; r < CT; ++r)
                if (r > s && r <= t) sum += gv[r];
            const float dec = expf(sum);
            const bool live = t < nv;
            sA[wave][t][s] = (live && s < t) ? bv[t] * dec * sKK[t][s] : 0.f;
            slot[OFF_M + e] = (live && s <= t) ? dec * sQK[t][s] * scale : 0.f;
        }
        if (lane < CT) {
            const int t = lane;
            float lam = 0.f, wdec = 0.f;
#pragma unroll
            for (int r = 0; r < CT; ++r) {
                if (r <= t) lam += gv[r];
                if (r > t && r < nv) wdec += gv[r];
            }
            const float L = t < nv ? expf(lam) : 0.f;
            slot[OFF_LAM + t] = L;
            slot[OFF_LAMS + t] = L * scale;
            slot[OFF_BETA + t] = bv[t];
            slot[OFF_W + t] = t < nv ? expf(wdec) : 0.f;
            if (t == nv - 1) slot[OFF_LAST] = L;
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
                float acc = (t == s) ? 1.f : 0.f;
#pragma unroll
                for (int r = 0; r < t; ++r) acc = fmaf(-sA[wave][t][r], Tc[r], acc);
                Tc[t] = acc;
            }
#pragma unroll
            for (int t = 0; t < CT; ++t) slot[OFF_T + t * CT + s] = Tc[t];
        }
        __builtin_amdgcn_wave_barrier();
    }
}

struct ChunkDims {
    int hk, hv, G;
};

// LDS strides (floats): rows padded so 16 lanes reading 16 rows hit distinct
// banks as far as a 16-byte read allows.
constexpr int TS_ = 20;   // T, M and V^T rows
constexpr int VEC = 80;   // Lam, Lam/sqrt(dk), beta, D[last][.], Lam_last

__global__ __launch_bounds__(256) void scan_chunk_kernel(ScanArgs p, ChunkDims d)
{
    // Staging buffers, indexed by chunk: K, V and the prep data are read after
    // the chunk's one barrier, so they rotate through 3 buffers; Q is read
    // only before it, so 2 suffice.  The partial sums rotate through 2.
    __shared__ __attribute__((aligned(16))) float sK[3][CT][KS];
    __shared__ __attribute__((aligned(16))) float sQ[2][CT][KS];
    __shared__ __attribute__((aligned(16))) float sV[3][32][TS_];   // v, [channel][token]
    __shared__ __attribute__((aligned(16))) float sT[3][CT][TS_];
    __shared__ __attribute__((aligned(16))) float sM[3][CT][TS_];
    __shared__ __attribute__((aligned(16))) float sVec[3][VEC];
    __shared__ __attribute__((aligned(16))) float sX[2][4][2][64][4];  // partial P, R

    const int tid = threadIdx.x;
    // wave index as a scalar: everything derived from it stays in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, kk = lane >> 4;

    // XCD-aware work index -> (sequence n, value head h, 32-channel block rb)
    const int nb = gridDim.x;
    int w = (int)blockIdx.x;
    if ((nb & 7) == 0) w = (w & 7) * (nb >> 3) + (w >> 3);
    const int rb = w & 3;
    w >>= 2;
    const int h = w % d.hv;
    const int n = w / d.hv;
    const int j = h / d.G;
    const int hk = d.hk, hv = d.hv;

    const int cu0 = p.cu[n];
    const int T_n = p.cu[n + 1] - cu0;
    if (T_n <= 0) return;

    const int rs = wave >> 1;  // 16-channel sub-block
    const int jh = wave & 1;   // key half: key blocks 4 jh .. 4 jh + 3
    const int row = rb * 32 + rs * 16 + l16;
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};

    // state quarter, accumulator layout: S4[b][r] = S[row][16 (4 jh + b) + 4 kk + r]
    float *Srow = p.state + (((int64_t)n * hv + h) * 128 + row) * 128 + 64 * jh + 4 * kk;
    f4 S4[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) S4[b] = *reinterpret_cast<const f4 *>(Srow + 16 * b);

    // Staging roles: k and q rows by all 256 threads (2 float4 each), v by
    // threads 0..127, the prep slot (T, M: 128 float4; the vectors: 20) by
    // threads 96..243.
    constexpr int SLOT_T0 = 96;
    const int tA = tid >> 5, tB = tA + 8, colK = (tid & 31) * 4;
    const int tV = tid >> 3, chV = (tid & 7) * 4;  // tid < 128
    const int fP = tid - SLOT_T0;                  // prep float4 index, 0..147
    f4 rkA = z4, rkB = z4, rqA = z4, rqB = z4, rv = z4, rp = z4;
    const int n_chunks = (T_n + CT - 1) / CT;
    const uint32_t kstride = (uint32_t)hk * 128;   // floats per token row of qn/kn
    const uint32_t vstride = (uint32_t)hv * 128;

    // Global loads only.  Rows past the sequence's end are read from its last
    // token instead (always valid memory) and then carry no weight: the prep
    // slot gives them beta = Lam = 0 and zero decay weights, and T is the
    // identity there, so they add exactly nothing to U, O or the state.
    // Addresses are a uniform base (SGPRs) plus a 32-bit byte offset per lane,
    // the form the global loads take directly.
    auto ld4 = [](const float *base, uint32_t byte_off) {
        return *reinterpret_cast<const f4 *>(reinterpret_cast<const char *>(base) + byte_off);
    };
    auto fetch = [&](int c) {
        const int64_t tb = (int64_t)cu0 + (int64_t)c * CT;
        const int nv = min(CT, T_n - c * CT);
        const float *kc = p.kn + (tb * hk + j) * 128;
        const float *qc = p.qn + (tb * hk + j) * 128;
        const uint32_t oA = ((uint32_t)min(tA, nv - 1) * kstride + colK) * 4u;
        const uint32_t oB = ((uint32_t)min(tB, nv - 1) * kstride + colK) * 4u;
        rkA = ld4(kc, oA);
        rqA = ld4(qc, oA);
        rkB = ld4(kc, oB);
        rqB = ld4(qc, oB);
        if (tid < 128)
            rv = ld4(p.vc + (tb * hv + h) * 128 + rb * 32,
                     ((uint32_t)min(tV, nv - 1) * vstride + chV) * 4u);
        if (fP >= 0 && fP < 148)
            rp = ld4(p.ws + (chunk_slot(cu0, n, c) * hv + h) * SCAN_SLOT_FLOATS, 16u * fP);
    };
    // registers -> the LDS buffers (b3, b2) of the chunk they hold
    auto stage = [&](auto b3c, auto b2c) {
        constexpr int b3 = decltype(b3c)::value, b2 = decltype(b2c)::value;
        *reinterpret_cast<f4 *>(&sK[b3][tA][colK]) = rkA;
        *reinterpret_cast<f4 *>(&sK[b3][tB][colK]) = rkB;
        *reinterpret_cast<f4 *>(&sQ[b2][tA][colK]) = rqA;
        *reinterpret_cast<f4 *>(&sQ[b2][tB][colK]) = rqB;
        if (tid < 128) {
            sV[b3][chV + 0][tV] = rv[0];
            sV[b3][chV + 1][tV] = rv[1];
            sV[b3][chV + 2][tV] = rv[2];
            sV[b3][chV + 3][tV] = rv[3];
        }
        if (fP >= 0 && fP < 64)
            *reinterpret_cast<f4 *>(&sT[b3][fP >> 2][(fP & 3) * 4]) = rp;
        else if (fP >= 64 && fP < 128)
            *reinterpret_cast<f4 *>(&sM[b3][(fP - 64) >> 2][(fP & 3) * 4]) = rp;
        else if (fP >= 128 && fP < 148)
            *reinterpret_cast<f4 *>(&sVec[b3][4 * (fP - 128)]) = rp;
    };

    // One chunk, with its LDS buffers (b3, b2) known at compile time.
    auto step = [&](auto b3c, auto b2c, int c) {
        constexpr int b3 = decltype(b3c)::value, b2 = decltype(b2c)::value;
        const int nv = min(CT, T_n - c * CT);
        const int64_t tb = (int64_t)cu0 + (int64_t)c * CT;
        // next chunk to LDS (its buffers were last read two chunks ago, before
        // the previous barrier), then start loading the one after
        if (c + 1 < n_chunks) {
            stage(std::integral_constant<int, (b3 + 1) % 3>{}, std::integral_constant<int, b2 ^ 1>{});
            if (c + 2 < n_chunks) fetch(c + 2);
        }

        // Every LDS operand of this chunk except the partner's partial sums is
        // in place already: read them all before the barrier, so that after it
        // only the exchange waits on LDS.
        f4 ka[4], qa[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = 16 * (4 * jh + b) + 4 * kk;
            ka[b] = *reinterpret_cast<const f4 *>(&sK[b3][l16][col]);
            qa[b] = *reinterpret_cast<const f4 *>(&sQ[b2][l16][col]);
        }
        const float *vec = sVec[b3];
        const f4 lam = *reinterpret_cast<const f4 *>(vec + 4 * kk);
        const f4 lams = *reinterpret_cast<const f4 *>(vec + 16 + 4 * kk);
        const f4 bet = *reinterpret_cast<const f4 *>(vec + 32 + 4 * kk);
        const f4 wv = *reinterpret_cast<const f4 *>(vec + 48 + 4 * kk);
        const float last = vec[64];
        const f4 vv = *reinterpret_cast<const f4 *>(&sV[b3][rs * 16 + l16][4 * kk]);
        const f4 trow = *reinterpret_cast<const f4 *>(&sT[b3][l16][4 * kk]);
        const f4 mrow = *reinterpret_cast<const f4 *>(&sM[b3][l16][4 * kk]);
        // A operand of the state update, K^T: key 16 (4 jh + b) + l16, token 4 kk + r
        float ak[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int b = 0; b < 4; ++b) ak[r][b] = sK[b3][4 * kk + r][16 * (4 * jh + b) + l16];
        }

        // partial P^T = K S0^T and R^T = Q S0^T over this wave's 64 keys
        f4 P = z4, R = z4;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                P = mfma4(ka[b][r], S4[b][r], P);
                R = mfma4(qa[b][r], S4[b][r], R);
            }
        }
        f4 C[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) C[b] = S4[b] * last;
        *reinterpret_cast<f4 *>(&sX[b2][wave][0][lane][0]) = P;
        *reinterpret_cast<f4 *>(&sX[b2][wave][1][lane][0]) = R;
        __syncthreads();  // the one barrier per chunk
        {
            // both waves of the pair add key half 0 + key half 1 (same bits)
            const f4 Po = *reinterpret_cast<const f4 *>(&sX[b2][wave ^ 1][0][lane][0]);
            const f4 Ro = *reinterpret_cast<const f4 *>(&sX[b2][wave ^ 1][1][lane][0]);
            P = jh == 0 ? P + Po : Po + P;
            R = jh == 0 ? R + Ro : Ro + R;
        }
        // B = beta (V - Lam P), component r is token 4 kk + r, channel l16
        f4 Bm;
#pragma unroll
        for (int r = 0; r < 4; ++r) Bm[r] = bet[r] * (vv[r] - lam[r] * P[r]);
        // U = T B
        f4 U = z4;
#pragma unroll
        for (int r = 0; r < 4; ++r) U = mfma4(trow[r], Bm[r], U);
        // S' = Lam_last S0 + K^T (D[last] U) on this wave's 64 keys
        const f4 Uw = U * wv;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int b = 0; b < 4; ++b) C[b] = mfma4(ak[r][b], Uw[r], C[b]);
        }
        if (jh == 0) {
            // O = Lam R + M U (both pre-scaled by 1/sqrt(dk))
            f4 O = lams * R;
#pragma unroll
            for (int r = 0; r < 4; ++r) O = mfma4(mrow[r], U[r], O);
            char *ob = reinterpret_cast<char *>(p.o + (tb * hv + h) * 128 + rb * 32 + rs * 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * kk + r;
                if (t < nv)
                    *reinterpret_cast<float *>(ob + ((uint32_t)t * vstride + l16) * 4u) = O[r];
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) S4[b] = C[b];
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    fetch(0);
    stage(I0{}, I0{});
    if (n_chunks > 1) fetch(1);
    __syncthreads();
    // unrolled by 6 = lcm(3, 2) so every buffer index is a constant
    for (int c = 0; c < n_chunks; c += 6) {
        step(I0{}, I0{}, c);
        if (c + 1 < n_chunks) step(I1{}, I1{}, c + 1);
        if (c + 2 < n_chunks) step(I2{}, I0{}, c + 2);
        if (c + 3 < n_chunks) step(I0{}, I1{}, c + 3);
        if (c + 4 < n_chunks) step(I1{}, I0{}, c + 4);
        if (c + 5 < n_chunks) step(I2{}, I1{}, c + 5);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) *reinterpret_cast<f4 *>(Srow + 16 * b) = S4[b];
}

hipError_t launch_scan(const gdn_shape &s, const ScanArgs &a, hipStream_t st)
{
    PrepDims pd;
    pd.hk = s.hk;
    pd.hv = s.hv;
    pd.G = s.hv / s.hk;
    pd.n_chunk_max = (int)((s.max_T + CT - 1) / CT);
    hipLaunchKernelGGL(scan_prep_kernel, dim3((unsigned)(s.n_seq * (int64_t)pd.n_chunk_max), s.hk),
                       dim3(256), 0, st, a, pd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ChunkDims cd;
    cd.hk = s.hk;
    cd.hv = s.hv;
    cd.G = s.hv / s.hk;
    const int64_t blocks = (int64_t)s.n_seq * s.hv * 4;
    hipLaunchKernelGGL(scan_chunk_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, cd);
    return hipGetLastError();
}

size_t scan_workspace_bytes(const gdn_shape &s)
{
    const size_t slots = (size_t)(s.total_T / CT) + (size_t)s.n_seq + 1;
    return slots * (size_t)s.hv * SCAN_SLOT_FLOATS * sizeof(float);
}

} // namespace gdn
