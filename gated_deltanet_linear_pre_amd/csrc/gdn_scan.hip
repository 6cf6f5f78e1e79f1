// gdn_scan.hip -- the gated delta rule, recurrent form, on an fp32 state.
//
// "Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1
// (gdn_scan_r findings): one state per value head, kept on chip and updated
// token by token in the same pass that forms the dot products against the old
// state; loads for the next tokens are issued before the per-token barrier.
// Section 2: a token-blocked run must equal the single pass.
//
// For value head h (key head j = h / G) and its dv x dk state S, per token:
//   alpha = exp(g),  p = S k,  r = S q                 (old state)
//   u = beta (v - alpha p)
//   S <- alpha S + u k^T
//   o = (alpha r + u (k . q)) / sqrt(dk)   (= S_new q / sqrt(dk))
// The last line is the plain o = S_t q / sqrt(dk), rewritten so that both dot
// products use the old state in one pass.
//
// gfx950 mapping.  Rows of S (value channels) evolve independently given the
// token's k, q, alpha, beta, so the state is split by rows across the whole
// chip.  A block of 4 waves owns 16 rows of one (sequence, value head).  A
// 16-lane DPP row holds one state row, 8 key columns per lane, in registers.
// The two row dot products are 8 FMAs per lane plus a 4-step DPP rotate-add,
// with no LDS round trip and no barrier per token.  Tokens are staged through
// LDS 16 at a time (k, q, the block's 16 v values, alpha, beta and k.q); the
// next chunk's global loads are issued before the current chunk is computed.
// So there are two barriers per 16 tokens rather than one per token.
// Outputs collect in LDS and leave as one 64-byte store per token.
//
// Block order is XCD-aware: blocks are dealt round-robin to the 8 XCDs, so the
// block index is permuted to give each XCD a contiguous run of
// (sequence, head, row block) work items.  The 8 row blocks of a head then
// share the key/query stream in one L2.
//
// Determinism: fixed-order FMAs and DPP trees, no atomics.  A sequence's
// result does not depend on how it is split across calls (the state is
// reloaded exactly as stored).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

constexpr int SCAN_CT = 16;  // tokens per LDS chunk
constexpr int SCAN_RB = 16;  // state rows per block

struct ScanDims {
    int hk, hv, G;
    int blocks_per_head;  // 128 / SCAN_RB
};

__global__ __launch_bounds__(256) void scan_kernel(ScanArgs p, ScanDims d)
{
    __shared__ __attribute__((aligned(16))) float sk[SCAN_CT][128];
    __shared__ __attribute__((aligned(16))) float sq[SCAN_CT][128];
    __shared__ __attribute__((aligned(16))) float sv[SCAN_CT][SCAN_RB];
    __shared__ __attribute__((aligned(16))) float so[SCAN_CT][SCAN_RB];
    __shared__ __attribute__((aligned(16))) float spar[SCAN_CT][4];  // alpha, beta, k.q, unused

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int l16 = lane & 15;

    // XCD-aware work index
    const int nb = gridDim.x;
    int w = (int)blockIdx.x;
    if ((nb & 7) == 0) w = (w & 7) * (nb >> 3) + (w >> 3);
    const int rb = w % d.blocks_per_head;
    w /= d.blocks_per_head;
    const int h = w % d.hv;
    const int n = w / d.hv;
    const int j = h / d.G;

    const int64_t s0 = p.cu[n];
    const int T_n = p.cu[n + 1] - p.cu[n];
    if (T_n <= 0) return;

    const int rl = (tid >> 6) * 4 + (lane >> 4);  // local row 0..15
    const int row = rb * SCAN_RB + rl;
    const int j0 = l16 * 8;
    const int hv = d.hv, hk = d.hk;
    const float scale = 0.08838834764831845f;  // 1 / sqrt(128)

    float S[8];
    float *Sp = p.state + (((int64_t)n * hv + h) * 128 + row) * 128 + j0;
    load8(Sp, S);

    // staging roles: float4 f = tid and tid + 256 of the chunk's k and q
    // (token f / 32, columns 4 (f % 32) ..); v: tid < 64 -> token tid / 4,
    // rows 4 (tid % 4) ..; alpha/beta: tid < 16 -> token tid.
    const int tokA = tid >> 5, tokB = tokA + 8;
    const int colK = (tid & 31) * 4;
    const int tokV = tid >> 2, colV = (tid & 3) * 4;
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 rkA = zero4, rkB = zero4, rqA = zero4, rqB = zero4, rv = zero4;
    float rg = 0.f, rbeta = 0.f;

#define GDN_SCAN_FETCH(c)                                                              \
    do {                                                                               \
        const int64_t tb_ = s0 + (int64_t)(c) * SCAN_CT;                               \
        const int nv_ = min(SCAN_CT, T_n - (c) * SCAN_CT);                             \
        const float *kb_ = p.kn + (tb_ * hk + j) * 128 + colK;                         \
        const float *qb_ = p.qn + (tb_ * hk + j) * 128 + colK;                         \
        const int64_t tstr_ = (int64_t)hk * 128;                                       \
        /* clamp to a valid token, then zero the value: no pointer select */         \
        const int ta_ = min(tokA, nv_ - 1), tb2_ = min(tokB, nv_ - 1);                 \
        const float4 ka_ = *reinterpret_cast<const float4 *>(kb_ + ta_ * tstr_);        \
        const float4 qa_ = *reinterpret_cast<const float4 *>(qb_ + ta_ * tstr_);        \
        const float4 kb2_ = *reinterpret_cast<const float4 *>(kb_ + tb2_ * tstr_);      \
        const float4 qb2_ = *reinterpret_cast<const float4 *>(qb_ + tb2_ * tstr_);      \
        rkA = tokA < nv_ ? ka_ : zero4;                                                \
        rqA = tokA < nv_ ? qa_ : zero4;                                                \
        rkB = tokB < nv_ ? kb2_ : zero4;                                               \
        rqB = tokB < nv_ ? qb2_ : zero4;                                               \
        if (tid < 64 && tokV < nv_)                                                    \
            rv = *reinterpret_cast<const float4 *>(p.vc + ((tb_ + tokV) * hv + h) * 128 + \
                                                   rb * SCAN_RB + colV);               \
        if (tid < nv_) {                                                               \
            rg = p.g[(tb_ + tid) * hv + h];                                            \
            rbeta = p.beta[(tb_ + tid) * hv + h];                                      \
        }                                                                              \
    } while (0)

#define GDN_SCAN_FLUSH(c)                                                              \
    do {                                                                               \
        const int64_t tb_ = s0 + (int64_t)(c) * SCAN_CT;                               \
        const int nv_ = min(SCAN_CT, T_n - (c) * SCAN_CT);                             \
        if (tid < 64 && tokV < nv_)                                                    \
            *reinterpret_cast<float4 *>(p.o + ((tb_ + tokV) * hv + h) * 128 +          \
                                        rb * SCAN_RB + colV) =                         \
                *reinterpret_cast<const float4 *>(&so[tokV][colV]);                    \
    } while (0)

    const int n_chunks = (T_n + SCAN_CT - 1) / SCAN_CT;
    GDN_SCAN_FETCH(0);
    for (int c = 0; c < n_chunks; ++c) {
        __syncthreads();  // previous chunk fully consumed
        if (c > 0) GDN_SCAN_FLUSH(c - 1);
        // registers -> LDS, plus k.q of each token (32 lanes per token)
        *reinterpret_cast<float4 *>(&sk[tokA][colK]) = rkA;
        *reinterpret_cast<float4 *>(&sq[tokA][colK]) = rqA;
        *reinterpret_cast<float4 *>(&sk[tokB][colK]) = rkB;
        *reinterpret_cast<float4 *>(&sq[tokB][colK]) = rqB;
        float kqA = rkA.x * rqA.x, kqB = rkB.x * rqB.x;
        kqA = fmaf(rkA.y, rqA.y, kqA);
        kqB = fmaf(rkB.y, rqB.y, kqB);
        kqA = fmaf(rkA.z, rqA.z, kqA);
        kqB = fmaf(rkB.z, rqB.z, kqB);
        kqA = fmaf(rkA.w, rqA.w, kqA);
        kqB = fmaf(rkB.w, rqB.w, kqB);
#pragma unroll
        for (int m = 16; m >= 1; m >>= 1) {
            kqA += __shfl_xor(kqA, m, 32);
            kqB += __shfl_xor(kqB, m, 32);
        }
        if ((tid & 31) == 0) {
            spar[tokA][2] = kqA;
            spar[tokB][2] = kqB;
        }
        if (tid < 64) *reinterpret_cast<float4 *>(&sv[tokV][colV]) = rv;
        if (tid < SCAN_CT) {
            spar[tid][0] = expf(rg);
            spar[tid][1] = rbeta;
        }
        if (c + 1 < n_chunks) GDN_SCAN_FETCH(c + 1);
        __syncthreads();

        const int nv = min(SCAN_CT, T_n - c * SCAN_CT);
#pragma unroll
        for (int i = 0; i < SCAN_CT; ++i) {
            if (i < nv) {  // uniform across the block
                const float4 k0 = *reinterpret_cast<const float4 *>(&sk[i][j0]);
                const float4 k1 = *reinterpret_cast<const float4 *>(&sk[i][j0 + 4]);
                const float4 q0 = *reinterpret_cast<const float4 *>(&sq[i][j0]);
                const float4 q1 = *reinterpret_cast<const float4 *>(&sq[i][j0 + 4]);
                const float4 par = *reinterpret_cast<const float4 *>(&spar[i][0]);
                const float v = sv[i][rl];
                const float k[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
                const float q[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
                float pk = S[0] * k[0], pq = S[0] * q[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) {
                    pk = fmaf(S[e], k[e], pk);
                    pq = fmaf(S[e], q[e], pq);
                }
                pk = row_sum16(pk);
                pq = row_sum16(pq);
                const float alpha = par.x, beta = par.y, kq = par.z;
                const float uu = beta * (v - alpha * pk);
                const float out = (alpha * pq + uu * kq) * scale;
#pragma unroll
                for (int e = 0; e < 8; ++e) S[e] = fmaf(uu, k[e], alpha * S[e]);
                if (l16 == 0) so[i][rl] = out;
            }
        }
    }
    __syncthreads();
    GDN_SCAN_FLUSH(n_chunks - 1);
#undef GDN_SCAN_FETCH
#undef GDN_SCAN_FLUSH
    store8(Sp, S);
}

hipError_t launch_scan(const gdn_shape &s, const ScanArgs &a, hipStream_t st)
{
    ScanDims d;
    d.hk = s.hk;
    d.hv = s.hv;
    d.G = s.hv / s.hk;
    d.blocks_per_head = 128 / SCAN_RB;
    const int64_t blocks = (int64_t)s.n_seq * s.hv * d.blocks_per_head;
    hipLaunchKernelGGL(scan_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, d);
    return hipGetLastError();
}

} // namespace gdn
