// gdn_noalloc.hip -- gdn_prefill_layer_noalloc: the layer entry point with its
// workspace in a device array the library owns, for callers that cannot
// allocate device memory.
//
// `scratch` below is a file-scope device array.  In host code its name is only
// a host-side stand-in: the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// on the first call there, and that pointer is what reaches the kernels.
#include <mutex>

#include "gdn_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

int scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GDN_E_LAUNCH;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_E_LAUNCH;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return GDN_OK;
}

} // namespace

extern "C" int gdn_prefill_layer_noalloc(const gdn_shape *shape, const int32_t *cu_seqlens,
                                         const void *qkv, const void *conv_w, const void *a,
                                         const void *b, const void *A_log, const void *dt_bias,
                                         const void *z, const void *gamma, void *hist, float *state,
                                         void *y, void *stream)
{
    int st = gdn::check_shape(shape);
    if (st != GDN_OK) return st;
    if (shape->total_T == 0) return GDN_OK;
    st = gdn::check_layer_args(cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, z, gamma, hist, state, y);
    if (st != GDN_OK) return st;
    const size_t need = gdn_prefill_workspace_bytes(shape);
    if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_E_TOO_LARGE;
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != GDN_OK) return st;
    return gdn_prefill_layer(shape, cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, z, gamma, hist,
                             state, y, ws, (size_t)GDN_NOALLOC_SCRATCH_BYTES, stream);
}
