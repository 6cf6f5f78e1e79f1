/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet prefill path.
 *
 * Three stages, each a hand-written HIP kernel, plus the whole layer:
 *
 *   gdn_pre   4-tap causal depthwise conv over the packed q|k|v channels with
 *             a carried 3-token history, SiLU, per-key-head L2 norm of q and
 *             k, and the per-value-head decay and write-strength gates.
 *   gdn_scan  the gated delta rule on a per-value-head fp32 state.
 *   gdn_post  per-(token, value head) RMSNorm with gamma, times SiLU(z).
 *   gdn_prefill_layer  pre -> scan -> post with the intermediates in a
 *             caller-provided workspace.
 *   gdn_step  one decode token per sequence through the whole layer.
 *
 * The stage split, the buffer set (q, k, v, gates, history, o, state, y)
 * and the fp16/fp32 output switch are those of the audited Metal path:
 * "Round 30 Track C Audit: gdn_pre, gdn_post, and gdn_scanr_4", sections 1
 * and 2 (the ten buffers checked per stage).  The production widths (16 key
 * heads, 48 value heads, head dim 128, 10240 channels, eps 1e-6) are those of
 * "round 10 track b: gdn vectorization and scan", "source and execution".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers are DEVICE pointers on the current HIP device, except `shape`,
 * which is a host pointer read during the call only.  `stream` is a
 * hipStream_t passed as void* (NULL = the default stream).  Every function only
 * enqueues work on `stream`; none synchronises or allocates, and all but
 * gdn_prefill_layer_noalloc keep no state, so calls are re-entrant.  The
 * caller owns every buffer.
 *
 * Return value: GDN_OK (0), or a negative gdn_status.  All argument checks
 * run before anything is enqueued, so on an argument error nothing has been
 * launched.  GDN_E_LAUNCH is the exception: a call that enqueues several
 * kernels (gdn_scan, gdn_prefill_layer, gdn_step) returns it when the runtime
 * refuses one of them, and the kernels before it stay enqueued; hist and
 * state may then be partly overwritten and must be treated as undefined.
 * Errors of the asynchronous kernels themselves surface at the caller's next
 * synchronisation.  A call with total_T == 0 is a no-op that returns GDN_OK
 * (history and state unchanged).
 *
 * Layouts (row-major).  C = 2*hk*dk + hv*dv.  "io" = shape->io_dtype.
 *   cu_seqlens [n_seq+1] int32  sequence n owns tokens [cu[n], cu[n+1]);
 *                               cu[0] = 0, non-decreasing, cu[n_seq] = total_T,
 *                               and no sequence longer than max_T.  These
 *                               device contents cannot be checked without a
 *                               sync: they are a precondition.
 *   qkv     [total_T][C]      io   channel blocks q | k | v; head i of a block
 *                                  occupies channels [i*d, (i+1)*d)
 *   conv_w  [C][4]            io   tap 3 multiplies the current token, tap 0
 *                                  the token three steps back; no bias
 *   a, b    [total_T][hv]     io   decay and write-strength logits
 *   A_log, dt_bias [hv]       io
 *   hist    [n_seq][3][C]     io   carried conv history, oldest row first
 *   qn, kn  [total_T][hk][dk] fp32 normalised q, k
 *   vc      [total_T][hv][dv] fp32 SiLU(conv) of the value channels
 *   g, beta [total_T][hv]     fp32 log decay and write strength
 *   state   [n_seq][hv][dv][dk] fp32  row index = value channel
 *   o       [total_T][hv][dv] fp32 scan output
 *   z       [total_T][hv][dv] io   output-gate input
 *   gamma   [dv]              io   RMSNorm weight shared by all value heads
 *   y       [total_T][hv][dv] shape->out_dtype
 * Alignment: workspaces 256-byte; qkv, conv_w, hist, qn, kn, vc, state, o,
 * z, gamma and y 16-byte; a, b, A_log, dt_bias, g, beta and
 * cu_seqlens 4-byte aligned (GDN_E_ALIGN otherwise).
 * No two buffers may overlap, except where an argument is documented as
 * read-then-overwritten in place (hist, state).
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 5

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_E_NULL = -1,      /* a required pointer is NULL                        */
    GDN_E_SHAPE = -2,     /* unsupported or inconsistent sizes                 */
    GDN_E_ALIGN = -3,     /* a pointer is not aligned as required              */
    GDN_E_WORKSPACE = -4, /* workspace smaller than gdn_prefill_workspace_bytes */
    GDN_E_DTYPE = -5,     /* io_dtype or out_dtype not a gdn_dtype             */
    GDN_E_LAUNCH = -6,    /* the HIP runtime rejected a kernel launch or call  */
    GDN_E_TOO_LARGE = -7  /* the shape needs more than GDN_NOALLOC_SCRATCH_BYTES */
} gdn_status;

typedef enum gdn_dtype {
    GDN_F32 = 0,
    GDN_F16 = 1
} gdn_dtype;

/* Sizes of one call.  Supported: dk = dv = 128, hk >= 1, hv >= 1,
 * hv % hk == 0 (value head h reads key head h / (hv / hk)), n_seq >= 1,
 * 0 <= max_T <= total_T < 2^31, max_T >= 1 when total_T >= 1.
 * eps_l2 is added to the sum of squares inside the square root of the q/k
 * L2 norm; eps_rms to the mean square inside that of the RMSNorm
 * (both 1e-6 in the audited configuration; both must be finite and >= 0). */
typedef struct gdn_shape {
    int32_t hk, hv, dk, dv;
    int32_t n_seq;
    int32_t io_dtype;   /* gdn_dtype of qkv, conv_w, a, b, A_log, dt_bias, hist, z, gamma */
    int32_t out_dtype;  /* gdn_dtype of y */
    int32_t reserved;   /* must be 0 */
    int64_t total_T;    /* = cu_seqlens[n_seq] */
    int64_t max_T;      /* host copy of max_n (cu[n+1] - cu[n]) */
    float eps_l2;
    float eps_rms;
} gdn_shape;

/* ABI version this library implements (GDN_ABI_VERSION). */
int gdn_abi_version(void);

/* Static description of a status code; never NULL. */
const char *gdn_status_str(int status);

/*
 * gdn_pre -- "Round 30 Track C Audit", section 1 (gdn_pre): the 4-tap conv
 * loop with the history paths for the first three tokens, the history write
 * at the last token, and the per-key-head sums of squares; "round 10 track
 * b", "variants": four ordered multiply-adds per element and SiLU on the value
 * channels too.
 *
 * Per sequence n with T_n tokens let X = [hist[n]; qkv rows of n] ((3+T_n) x C):
 *   x~[t][c] = sum_{m=0..3} conv_w[c][m] * X[t+m][c]
 *   s = SiLU(x~) = x~ * sigmoid(x~)
 *   qn = s_q / sqrt(|s_q|^2 + eps_l2) per key head, kn likewise, vc = s_v
 *   g[t][h] = -exp(A_log[h]) * softplus(a[t][h] + dt_bias[h]); beta = sigmoid(b)
 *   hist[n] <- X[T_n .. T_n+2]  (for T_n < 3 this keeps 3-T_n old rows)
 * In:  cu_seqlens, qkv, conv_w, a, b, A_log, dt_bias, hist (read).
 * Out: qn, kn, vc, g, beta; hist (overwritten in place after it is read).
 */
int gdn_pre(const gdn_shape *shape, const int32_t *cu_seqlens,
            const void *qkv, const void *conv_w, const void *a, const void *b,
            const void *A_log, const void *dt_bias, void *hist,
            float *qn, float *kn, float *vc, float *g, float *beta,
            void *stream);

/*
 * gdn_scan -- "Round 30 Track C Audit", section 1 (gdn_scan_r findings): a
 * per-value-head state updated token by token in the loop that forms the dot
 * products against the old state; section 2: a token-blocked run must equal
 * the single pass.
 *
 * For each sequence n and value head h (key head j = h / (hv/hk)), over its
 * tokens in order, with S the dv x dk state of (n, h):
 *   alpha = exp(g[t][h])
 *   S <- alpha*S + beta[t][h] * (vc[t][h] - alpha*S kn[t][j]) kn[t][j]^T
 *   o[t][h] = S qn[t][j] / sqrt(dk)
 * The kernels evaluate this exactly (up to fp32 rounding) in 32-token chunks
 * counted from each sequence's first token.  Splitting a sequence across calls
 * at a multiple of 32 tokens is therefore bit-identical to one call; any other
 * split agrees within fp32 rounding.
 * Numerical domain: the products run on fp16 matrix cores with each fp32
 * operand split into a high and a low fp16 half (about 22 significant bits),
 * the low halves of the data-scaled operands carried x 2^10.  Accuracy holds
 * while 16*|S|, |beta (v - alpha-weighted S k)| and the chunk's write vectors
 * stay below 65504 (in practice |S| up to a few thousand, |v| up to ~6e4);
 * past that a low half overflows and the results turn non-finite, which the
 * output shows.  On the small side a split operand keeps its ~22 bits down
 * to |x| near 2^-13, below which its error is an absolute floor near 2^-34;
 * states whose RMS is above ~1e-6 hold 2e-4 of their RMS elementwise.
 * In:  cu_seqlens, qn, kn, vc, g, beta; state (read: S at the start).
 * Out: o; state (overwritten in place with S after the last token).
 * workspace: device scratch of >= gdn_scan_workspace_bytes(shape) bytes,
 * 256-byte aligned, owned by the caller; its contents are undefined after the
 * call and it must not be shared by calls in flight at the same time.
 */
int gdn_scan(const gdn_shape *shape, const int32_t *cu_seqlens,
             const float *qn, const float *kn, const float *vc,
             const float *g, const float *beta, float *state, float *o,
             void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of scratch gdn_scan needs for `shape` (0 if the shape is invalid):
 * (total_T/32 + n_seq + 1) slots, each holding hk key-head parts of 32 KB and
 * hv value-head parts of 6656 bytes. */
size_t gdn_scan_workspace_bytes(const gdn_shape *shape);

/*
 * gdn_post -- "Round 30 Track C Audit", section 1 (gdn_post): one sum of
 * squares per row, gamma, and the fp16/fp32 output switch; "opus_r25_gdn --
 * round 25 track A", "shipped": the sigmoid gate.
 *
 * For each (token, value head) row of dv values:
 *   y_i = o_i / sqrt(mean_i(o_i^2) + eps_rms) * gamma_i * z_i * sigmoid(z_i)
 * computed in fp32 and rounded to out_dtype (round to nearest even).
 * In: o, z, gamma.  Out: y.
 */
int gdn_post(const gdn_shape *shape, const float *o, const void *z,
             const void *gamma, void *y, void *stream);

/* Bytes of workspace gdn_prefill_layer needs for `shape` (0 if the shape is
 * invalid), by the path the shape takes, each part 256-byte aligned: o and
 * the scan scratch always; with fp32 io and hv/hk <= 8 also vc; with
 * hv/hk > 8 (the three stages in turn) also qn, kn, vc, g and beta. */
size_t gdn_prefill_workspace_bytes(const gdn_shape *shape);

/*
 * gdn_prefill_layer -- the three stages above in order on one stream, the
 * whole path of one layer.  Arguments are those of gdn_pre, gdn_scan and
 * gdn_post; the fp32 intermediates and the scan scratch live in `workspace`
 * (>= gdn_prefill_workspace_bytes(shape) bytes, device memory, 256-byte
 * aligned, contents undefined afterwards, not shared by calls in flight at the
 * same time).  hist and state are read and overwritten in place.
 *
 * With fp16 io, one sequence, hv/hk <= 8 and at least 32 CUs left free by
 * the chunk kernel's blocks (one per sequence, value head and 32 value
 * channels), post runs inside that kernel's launch on those CUs, each (chunk,
 * value head) once the chunk's o values of that head are stored (the result
 * is bit for bit that of the separate post).  Each of those waits is bounded (about 30-100 ms;
 * the environment variable GDN_POST_WAIT_POLLS, read at each call, can lower
 * the bound, GDN_LAYER_POST_FUSED=0 selects the separate post launch).  A wait
 * that runs out leaves y undefined for that unit (state and hist are not
 * affected) and sets bit 0 of the 32-bit word at byte offset
 * gdn_prefill_workspace_bytes(shape) - 256 of the workspace, which is 0
 * after a call in which no wait ran out; read it once the call has completed.
 * Only a device that cannot run the chunk blocks to completion (every chunk
 * block is dispatched before any post block) lets a wait run out.
 */
int gdn_prefill_layer(const gdn_shape *shape, const int32_t *cu_seqlens,
                      const void *qkv, const void *conv_w, const void *a,
                      const void *b, const void *A_log, const void *dt_bias,
                      const void *z, const void *gamma, void *hist,
                      float *state, void *y, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * gdn_step -- one decode token for each of n_seq sequences through the whole
 * layer.  "Round 30 Track C Audit", section 1 (gdn_scan_r findings): the
 * single-token update of the per-value-head state, the step every scan
 * variant is checked against; section 2: running T steps must agree with
 * one T-token pass.
 *
 * shape->total_T must equal shape->n_seq and shape->max_T must be 1: token
 * row n of qkv, a, b, z and y belongs to sequence n (no cu_seqlens).  Per
 * sequence n the arithmetic is that of gdn_pre, gdn_scan and gdn_post for
 * one token, with the same layouts:
 *   X = [hist[n]; qkv[n]] (4 x C), x~[c] = sum_m conv_w[c][m] X[m][c],
 *   s = SiLU(x~), qn/kn the L2-normalised key-head blocks, v the value block;
 *   alpha = exp(g), g and beta as in gdn_pre;
 *   S <- alpha*S + beta (v - alpha*S kn) kn^T,  o = S qn / sqrt(dk)  (fp32)
 *   y = o / sqrt(mean(o^2) + eps_rms) * gamma * z * sigmoid(z)  -> out_dtype
 *   hist_out[n] <- X[1..3]
 * In:  qkv [n_seq][C], conv_w, a, b [n_seq][hv], A_log, dt_bias, z
 *      [n_seq][hv][dv], gamma; hist and state (read).
 * Out: y [n_seq][hv][dv]; state (overwritten in place); the new history in
 *      hist_out, a buffer of hist's layout and dtype that must not overlap
 *      hist (16-byte aligned), which stays unchanged; or, with hist_out NULL
 *      or equal to hist, in hist itself.
 * No workspace.  One kernel is enqueued with a separate hist_out; in place,
 * two (the step, then the history shift, since every block of a key-head
 * group reads the group's old history).  A decode loop that alternates two
 * history buffers gets the single launch.
 */
int gdn_step(const gdn_shape *shape, const void *qkv, const void *conv_w,
             const void *a, const void *b, const void *A_log,
             const void *dt_bias, const void *z, const void *gamma, void *hist,
             void *hist_out, float *state, void *y, void *stream);

/*
 * gdn_prefill_layer_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): gdn_prefill_layer with the same arguments and results, except
 * that the workspace is a static device array of GDN_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on every device it runs on until the process
 * ends.  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine); the caller still provides every input and output.
 *
 * Shapes whose gdn_prefill_workspace_bytes exceeds GDN_NOALLOC_SCRATCH_BYTES
 * are rejected with GDN_E_TOO_LARGE before anything is enqueued (at
 * production width, 16 key and 48 value heads, about 2600 tokens fit).  The
 * array's device address is looked up on the first call on each device
 * (GDN_E_LAUNCH if the runtime refuses).  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (on different streams,
 * or from different threads) race and give undefined results; calls in
 * order on one stream are safe.  Nothing in the array needs to start at
 * zero: every byte a call reads was written earlier in the same call.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gdn_prefill_layer_noalloc(const gdn_shape *shape, const int32_t *cu_seqlens,
                              const void *qkv, const void *conv_w, const void *a,
                              const void *b, const void *A_log, const void *dt_bias,
                              const void *z, const void *gamma, void *hist,
                              float *state, void *y, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
