// gdn_internal.h -- launchers behind the C ABI (include/gdn.h).  Each one
// assumes its arguments were validated by the ABI layer and only enqueues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

struct PreArgs {
    const int32_t *cu;
    const void *qkv, *conv_w, *a, *b, *A_log, *dt_bias;
    void *hist;
    float *qn, *kn, *vc, *g, *beta;
};

struct ScanArgs {
    const int32_t *cu;
    const float *qn, *kn, *vc, *g, *beta;
    float *state, *o;
    float *ws;  // per-(chunk, value head) prep slots
};

// Scan workspace: per 32-token chunk, one key-head slot per key head (K and Q
// as split fp16 MFMA operands, 32 KB) and one value-head slot per value head
// (T, M as split fp16 operands plus the chunk's decay vectors, 6.5 KB).
constexpr int SCAN_KH_FLOATS = 8192;
constexpr int SCAN_SLOT_FLOATS = 1664;
size_t scan_workspace_bytes(const gdn_shape &s);

// The layer path with fp16 inputs forms v inside the chunk kernel, from the
// raw qkv rows of its value channels (4-tap conv with the history, SiLU), and
// carries the history of those channels there.
struct VRawArgs {
    const void *qkv, *conv_w;
    void *hist;
    int C;  // channels of a qkv row
};

// The layer path's fused pre + prep step: the pre-stage inputs, the history
// (in/out), and the two buffers the chunk kernel reads (vc and the slots).
struct LayerPrepArgs {
    const int32_t *cu;
    const void *qkv, *conv_w, *a, *b, *A_log, *dt_bias;
    void *hist;
    float *vc;
    float *ws;
    // fp16 io: room (layer_sync_bytes) for the counters and status word of
    // post run in the chunk kernel's launch (null: post is not fused)
    uint32_t *sync;
};
size_t layer_sync_bytes(const gdn_shape &s);
constexpr int LAYER_G_MAX = 8;  // value heads per key head the fused step handles

struct PostArgs {
    const float *o;
    const void *z, *gamma;
    void *y;
};

struct StepArgs {
    const void *qkv, *conv_w, *a, *b, *A_log, *dt_bias, *z, *gamma;
    void *hist;
    void *hist_out;  // NULL: hist is shifted in place by a second launch
    float *state;
    void *y;
};

// The shape checks every entry point runs first (GDN_OK or a gdn_status).
int check_shape(const gdn_shape *s);
// Null and alignment checks of gdn_prefill_layer's buffers other than the
// workspace (GDN_OK or a gdn_status).
int check_layer_args(const int32_t *cu, const void *qkv, const void *conv_w, const void *a,
                     const void *b, const void *A_log, const void *dt_bias, const void *z,
                     const void *gamma, const void *hist, const float *state, const void *y);

hipError_t launch_pre(const gdn_shape &s, const PreArgs &a, hipStream_t st);
hipError_t launch_scan(const gdn_shape &s, const ScanArgs &a, hipStream_t st);
// The layer's pre and scan; with post given, also post when it can run in the
// chunk kernel's launch (then *post_done is set, else the caller launches it).
hipError_t launch_layer_scan(const gdn_shape &s, const LayerPrepArgs &lp, const ScanArgs &a,
                             const PostArgs *post, bool *post_done, hipStream_t st);
hipError_t launch_post(const gdn_shape &s, const PostArgs &a, hipStream_t st);
hipError_t launch_step(const gdn_shape &s, const StepArgs &a, hipStream_t st);

// Grid-size limits the ABI checks before launching.
constexpr int PRE_WAVE_TOKENS = 4;  // tokens per pre wave; a pre block takes 4 waves' tokens

} // namespace gdn
