// gdn_abi.hip -- the extern "C" entry points of include/gdn.h: argument
// checks (all before anything is enqueued), then the stage launchers.
#include <math.h>
#include <stdint.h>

#include "gdn_internal.h"

namespace {

using gdn::PreArgs;
using gdn::ScanArgs;
using gdn::PostArgs;
using gdn::StepArgs;

constexpr int64_t kMaxTokens = (int64_t)1 << 31;
constexpr int kMaxHeads = 1 << 12;
constexpr int kMaxSeqs = 1 << 20;

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool finite_nonneg(float x) { return isfinite(x) && x >= 0.f; }

} // namespace

// (also used by the no-allocation entry point)
int gdn::check_shape(const gdn_shape *s)
{
    if (!s) return GDN_E_NULL;
    if (s->io_dtype != GDN_F32 && s->io_dtype != GDN_F16) return GDN_E_DTYPE;
    if (s->out_dtype != GDN_F32 && s->out_dtype != GDN_F16) return GDN_E_DTYPE;
    if (s->dk != 128 || s->dv != 128) return GDN_E_SHAPE;
    if (s->hk < 1 || s->hv < 1 || s->hk > kMaxHeads || s->hv > kMaxHeads) return GDN_E_SHAPE;
    if (s->hv % s->hk != 0) return GDN_E_SHAPE;
    if (s->n_seq < 1 || s->n_seq > kMaxSeqs) return GDN_E_SHAPE;
    if (s->reserved != 0) return GDN_E_SHAPE;
    if (s->total_T < 0 || s->total_T >= kMaxTokens) return GDN_E_SHAPE;
    if (s->max_T < 0 || s->max_T > s->total_T) return GDN_E_SHAPE;
    if (s->total_T > 0 && s->max_T < 1) return GDN_E_SHAPE;
    if ((int64_t)s->n_seq * s->max_T < s->total_T) return GDN_E_SHAPE;
    if (!finite_nonneg(s->eps_l2) || !finite_nonneg(s->eps_rms)) return GDN_E_SHAPE;
    // launch-grid limits (pre: tiles of 8 tokens at worst; scan prep: 16)
    const int64_t pre_blocks = (int64_t)s->n_seq * ((s->max_T + 7) / 8);
    if (pre_blocks >= ((int64_t)1 << 31)) return GDN_E_SHAPE;
    if ((int64_t)s->n_seq * s->hv * 4 >= ((int64_t)1 << 31)) return GDN_E_SHAPE;
    return GDN_OK;
}

namespace {

using gdn::check_shape;

#define REQ(p)                                  \
    do {                                        \
        if (!(p)) return GDN_E_NULL;            \
    } while (0)
#define ALN(p, a)                               \
    do {                                        \
        if (!aligned((p), (a))) return GDN_E_ALIGN; \
    } while (0)

int check_pre(const gdn_shape *s, const int32_t *cu, const void *qkv, const void *conv_w,
              const void *a, const void *b, const void *A_log, const void *dt_bias,
              const void *hist, const float *qn, const float *kn, const float *vc,
              const float *g, const float *beta)
{
    REQ(cu); REQ(qkv); REQ(conv_w); REQ(a); REQ(b); REQ(A_log); REQ(dt_bias); REQ(hist);
    REQ(qn); REQ(kn); REQ(vc); REQ(g); REQ(beta);
    ALN(cu, 4); ALN(a, 4); ALN(b, 4); ALN(A_log, 4); ALN(dt_bias, 4); ALN(g, 4); ALN(beta, 4);
    ALN(qkv, 16); ALN(conv_w, 16); ALN(hist, 16); ALN(qn, 16); ALN(kn, 16); ALN(vc, 16);
    return GDN_OK;
}

int check_scan(const int32_t *cu, const float *qn, const float *kn, const float *vc,
               const float *g, const float *beta, const float *state, const float *o,
               const void *ws)
{
    REQ(cu); REQ(qn); REQ(kn); REQ(vc); REQ(g); REQ(beta); REQ(state); REQ(o); REQ(ws);
    ALN(cu, 4); ALN(g, 4); ALN(beta, 4);
    ALN(qn, 16); ALN(kn, 16); ALN(vc, 16); ALN(state, 16); ALN(o, 16); ALN(ws, 256);
    return GDN_OK;
}

int check_post(const float *o, const void *z, const void *gamma, const void *y)
{
    REQ(o); REQ(z); REQ(gamma); REQ(y);
    ALN(o, 16); ALN(z, 16); ALN(gamma, 16); ALN(y, 16);
    return GDN_OK;
}

} // namespace

// The caller's buffers of gdn_prefill_layer (everything but the workspace).
int gdn::check_layer_args(const int32_t *cu, const void *qkv, const void *conv_w, const void *a,
                          const void *b, const void *A_log, const void *dt_bias, const void *z,
                          const void *gamma, const void *hist, const float *state, const void *y)
{
    REQ(cu); REQ(qkv); REQ(conv_w); REQ(a); REQ(b); REQ(A_log); REQ(dt_bias); REQ(z); REQ(gamma);
    REQ(hist); REQ(state); REQ(y);
    ALN(cu, 4); ALN(a, 4); ALN(b, 4); ALN(A_log, 4); ALN(dt_bias, 4);
    ALN(qkv, 16); ALN(conv_w, 16); ALN(hist, 16); ALN(state, 16); ALN(z, 16); ALN(gamma, 16);
    ALN(y, 16);
    return GDN_OK;
}

namespace {

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carve {
    size_t qn, kn, vc, g, beta, o, scan, sync, total;
};

// Which path gdn_prefill_layer takes for a shape: the pre stage fused into the
// scan's prep step when a key head has at most LAYER_G_MAX value heads (with
// fp16 inputs v is formed inside the chunk kernel too), else the three stages.
enum class LayerPath { fused_f16, fused_f32, staged };

LayerPath layer_path(const gdn_shape *s)
{
    if (s->hv / s->hk > gdn::LAYER_G_MAX) return LayerPath::staged;
    return s->io_dtype == GDN_F16 ? LayerPath::fused_f16 : LayerPath::fused_f32;
}

// The layer workspace holds what the path writes and reads back: o and the
// scan scratch always; the fp32 v when the fused prep forms it (fp32 inputs);
// q, k, v and the gates only on the staged path; with fp16 inputs the
// counters of post run in the chunk kernel's launch.
Carve carve(const gdn_shape *s)
{
    const size_t T = (size_t)s->total_T;
    const LayerPath path = layer_path(s);
    const bool staged = path == LayerPath::staged;
    Carve c;
    size_t off = 0;
    c.qn = off; off += staged ? round256(T * s->hk * 128 * sizeof(float)) : 0;
    c.kn = off; off += staged ? round256(T * s->hk * 128 * sizeof(float)) : 0;
    c.vc = off; off += path != LayerPath::fused_f16 ? round256(T * s->hv * 128 * sizeof(float)) : 0;
    c.g = off; off += staged ? round256(T * s->hv * sizeof(float)) : 0;
    c.beta = off; off += staged ? round256(T * s->hv * sizeof(float)) : 0;
    c.o = off; off += round256(T * s->hv * 128 * sizeof(float));
    c.scan = off; off += round256(gdn::scan_workspace_bytes(*s));
    c.sync = off; off += path == LayerPath::fused_f16 ? round256(gdn::layer_sync_bytes(*s)) : 0;
    c.total = off;
    return c;
}

int launch_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_E_LAUNCH; }

} // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_str(int status)
{
    switch (status) {
    case GDN_OK: return "ok";
    case GDN_E_NULL: return "a required pointer is NULL";
    case GDN_E_SHAPE: return "unsupported or inconsistent sizes";
    case GDN_E_ALIGN: return "a pointer is not aligned as required";
    case GDN_E_WORKSPACE: return "workspace too small";
    case GDN_E_DTYPE: return "unknown dtype";
    case GDN_E_LAUNCH: return "the HIP runtime rejected a kernel launch or call";
    case GDN_E_TOO_LARGE: return "the shape needs more workspace than the library's static array holds";
    default: return "unknown status";
    }
}

int gdn_pre(const gdn_shape *shape, const int32_t *cu_seqlens, const void *qkv,
            const void *conv_w, const void *a, const void *b, const void *A_log,
            const void *dt_bias, void *hist, float *qn, float *kn, float *vc, float *g,
            float *beta, void *stream)
{
    int st = check_shape(shape);
    if (st) return st;
    if (shape->total_T == 0) return GDN_OK;
    st = check_pre(shape, cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, hist, qn, kn, vc, g, beta);
    if (st) return st;
    const PreArgs pa{cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, hist, qn, kn, vc, g, beta};
    return launch_status(gdn::launch_pre(*shape, pa, (hipStream_t)stream));
}

size_t gdn_scan_workspace_bytes(const gdn_shape *shape)
{
    if (check_shape(shape) != GDN_OK) return 0;
    return gdn::scan_workspace_bytes(*shape);
}

int gdn_scan(const gdn_shape *shape, const int32_t *cu_seqlens, const float *qn,
             const float *kn, const float *vc, const float *g, const float *beta,
             float *state, float *o, void *workspace, size_t workspace_bytes, void *stream)
{
    int st = check_shape(shape);
    if (st) return st;
    if (shape->total_T == 0) return GDN_OK;
    st = check_scan(cu_seqlens, qn, kn, vc, g, beta, state, o, workspace);
    if (st) return st;
    if (workspace_bytes < gdn::scan_workspace_bytes(*shape)) return GDN_E_WORKSPACE;
    const ScanArgs sa{cu_seqlens, qn, kn, vc, g, beta, state, o, static_cast<float *>(workspace)};
    return launch_status(gdn::launch_scan(*shape, sa, (hipStream_t)stream));
}

int gdn_post(const gdn_shape *shape, const float *o, const void *z, const void *gamma,
             void *y, void *stream)
{
    int st = check_shape(shape);
    if (st) return st;
    if (shape->total_T == 0) return GDN_OK;
    st = check_post(o, z, gamma, y);
    if (st) return st;
    const PostArgs pa{o, z, gamma, y};
    return launch_status(gdn::launch_post(*shape, pa, (hipStream_t)stream));
}

size_t gdn_prefill_workspace_bytes(const gdn_shape *shape)
{
    if (check_shape(shape) != GDN_OK) return 0;
    return carve(shape).total;
}

int gdn_prefill_layer(const gdn_shape *shape, const int32_t *cu_seqlens, const void *qkv,
                      const void *conv_w, const void *a, const void *b, const void *A_log,
                      const void *dt_bias, const void *z, const void *gamma, void *hist,
                      float *state, void *y, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    int st = check_shape(shape);
    if (st) return st;
    if (shape->total_T == 0) return GDN_OK;
    st = gdn::check_layer_args(cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, z, gamma, hist, state, y);
    if (st) return st;
    REQ(workspace);
    ALN(workspace, 256);
    const Carve c = carve(shape);
    if (workspace_bytes < c.total) return GDN_E_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    float *qn = reinterpret_cast<float *>(ws + c.qn);
    float *kn = reinterpret_cast<float *>(ws + c.kn);
    float *vc = reinterpret_cast<float *>(ws + c.vc);
    float *g = reinterpret_cast<float *>(ws + c.g);
    float *beta = reinterpret_cast<float *>(ws + c.beta);
    float *o = reinterpret_cast<float *>(ws + c.o);
    float *sws = reinterpret_cast<float *>(ws + c.scan);
    // (on the fused paths the unused intermediates have no room of their own:
    // their pointers alias the next region and are never dereferenced)
    st = check_pre(shape, cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, hist, qn, kn, vc, g, beta);
    if (st) return st;
    st = check_scan(cu_seqlens, qn, kn, vc, g, beta, state, o, sws);
    if (st) return st;
    st = check_post(o, z, gamma, y);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    const ScanArgs sa{cu_seqlens, qn, kn, vc, g, beta, state, o, sws};
    const PostArgs po{o, z, gamma, y};
    const LayerPath path = layer_path(shape);
    if (path != LayerPath::staged) {
        // pre fused into the scan's prep step: q, k and the gates stay on chip
        uint32_t *sync = path == LayerPath::fused_f16 ? reinterpret_cast<uint32_t *>(ws + c.sync) : nullptr;
        const gdn::LayerPrepArgs lp{cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, hist, vc, sws, sync};
        bool post_done = false;
        if (gdn::launch_layer_scan(*shape, lp, sa, &po, &post_done, s) != hipSuccess) return GDN_E_LAUNCH;
        if (post_done) return GDN_OK;
    } else {
        const PreArgs pa{cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, hist, qn, kn, vc, g, beta};
        if (gdn::launch_pre(*shape, pa, s) != hipSuccess) return GDN_E_LAUNCH;
        if (gdn::launch_scan(*shape, sa, s) != hipSuccess) return GDN_E_LAUNCH;
    }
    return launch_status(gdn::launch_post(*shape, po, s));
}

int gdn_step(const gdn_shape *shape, const void *qkv, const void *conv_w, const void *a,
             const void *b, const void *A_log, const void *dt_bias, const void *z,
             const void *gamma, void *hist, void *hist_out, float *state, void *y, void *stream)
{
    int st = check_shape(shape);
    if (st) return st;
    if (shape->total_T != shape->n_seq || shape->max_T != 1) return GDN_E_SHAPE;
    REQ(qkv); REQ(conv_w); REQ(a); REQ(b); REQ(A_log); REQ(dt_bias); REQ(z); REQ(gamma);
    REQ(hist); REQ(state); REQ(y);
    ALN(a, 4); ALN(b, 4); ALN(A_log, 4); ALN(dt_bias, 4);
    ALN(qkv, 16); ALN(conv_w, 16); ALN(z, 16); ALN(gamma, 16); ALN(hist, 16); ALN(state, 16);
    ALN(y, 16);
    if (hist_out == hist) hist_out = nullptr;  // in place
    if (hist_out) ALN(hist_out, 16);
    const StepArgs sa{qkv, conv_w, a, b, A_log, dt_bias, z, gamma, hist, hist_out, state, y};
    return launch_status(gdn::launch_step(*shape, sa, (hipStream_t)stream));
}

} // extern "C"
