// gdn_post.hip -- per-(token, value head) RMSNorm with gamma, times SiLU(z).
//
// "Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", section 1
// (gdn_post): one sum of squares per row of dv values, gamma, fp16 or fp32
// output; "opus_r25_gdn -- round 25 track A", "shipped": the sigmoid gate.
//
//   y_i = o_i / sqrt(mean(o^2) + eps) * gamma_i * z_i * sigmoid(z_i)
//
// gfx950 mapping.  The stage moves 12 B (fp16 y) or 16 B (fp32 y) per element
// for about 10 flop, so it is bound by HBM bandwidth.  A 16-lane DPP row owns
// one row of 128 values: lane l takes values 4l..4l+3 and 64+4l..64+4l+3, so
// every load and store instruction covers whole 64-value runs of its four
// rows (whole cache lines; with 8 consecutive values per lane each fp32
// instruction filled half of every line it touched).  The sum of squares is a
// 4-step DPP rotate-add inside the row, with no LDS and no barrier.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void post_kernel(const float *__restrict__ o,
                                                   const TI *__restrict__ z,
                                                   const TI *__restrict__ gamma,
                                                   TO *__restrict__ y, int64_t n_rows,
                                                   float eps)
{
    const int l16 = threadIdx.x & 15;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    if (row >= n_rows) return;  // whole 16-lane rows leave together
    const int64_t base = row * 128 + l16 * 4;

    float x[8], zz[8], gm[8];
    load8_split(o + base, x);
    load8_split(z + base, zz);
    load8_split(gamma + l16 * 4, gm);

    float out[8];
    post_row(x, zz, gm, eps, out);
    store8_split(y + base, out);
}

template <typename TI, typename TO>
static hipError_t launch_post_t(const gdn_shape &s, const PostArgs &a, hipStream_t st)
{
    const int64_t n_rows = s.total_T * (int64_t)s.hv;
    const int64_t blocks = (n_rows + 15) / 16;
    hipLaunchKernelGGL((post_kernel<TI, TO>), dim3((unsigned)blocks), dim3(256), 0, st,
                       a.o, static_cast<const TI *>(a.z), static_cast<const TI *>(a.gamma),
                       static_cast<TO *>(a.y), n_rows, s.eps_rms);
    return hipGetLastError();
}

hipError_t launch_post(const gdn_shape &s, const PostArgs &a, hipStream_t st)
{
    if (s.io_dtype == GDN_F16)
        return s.out_dtype == GDN_F16 ? launch_post_t<_Float16, _Float16>(s, a, st)
                                      : launch_post_t<_Float16, float>(s, a, st);
    return s.out_dtype == GDN_F16 ? launch_post_t<float, _Float16>(s, a, st)
                                  : launch_post_t<float, float>(s, a, st);
}

} // namespace gdn
