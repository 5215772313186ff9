/*
 * kvc.h -- C ABI of libkvc: prefill KV-cache compression for audio-language
 * models on AMD Instinct MI355X (gfx950).
 *
 * The method is AudioKV's (AudioKV article on seekfood.cn, sections 2-3;
 * abstract page "AudioKV: KV Cache Eviction in Efficient Large Audio Language
 * Models"), run per unit u = (sequence, layer, KV head):
 *
 *   1. scores   s[j] = mean over the unit's G*W observation-window queries of
 *               softmax_j(q . k_j / sqrt(d)) over the L audio keys (or the
 *               max over query heads of the head means, kvc_score)
 *               (article section 1.2; softmax(qK^T/sqrt(d)) as in the VoxZip
 *               digest's decayed-eviction equation)
 *   2. smooth   Spectral Score Smoothing (article section 2.2):
 *               F = rfft(s), E(k) = sum_{i<=k} |F_i|^2,
 *               k* = min{k : E(k) >= rho E(L/2)}, low-pass keeps bins 0..k*,
 *               s_hat = (1 - alpha) s + alpha irfft(F masked)
 *   3. budget   b_u = w + r + share of B_score proportional to S_u within
 *               the unit's budget pool (the sequence, or its layer)
 *               (article section 3.1; defaults from the section 5.1 config)
 *   4. select   the b_u - w largest s_hat among positions [0, L-w), equal
 *               values resolved toward the lower position, plus the window
 *               [L-w, L); listed in ascending position order
 *   5. gather   K_out[t] = K[idx[t]], V_out[t] = V[idx[t]]
 *
 * Conventions shared by every entry point:
 *   - Device pointers are HIP device memory on the current device; host
 *     pointers are named as such.  The library never allocates, frees or
 *     synchronises; all work is enqueued on `stream` (a hipStream_t passed
 *     as void*, NULL = the null stream) and the call returns once enqueued.
 *   - Units are ordered (sequence, layer, KV head), u = (i*n_layers + l)*
 *     n_kv_heads + h.  Score rows are varlen: unit u's row starts at
 *     element n_layers*n_kv_heads*seq_start[i] + (l*n_kv_heads + h)*L_i.
 *   - Validation is synchronous and launches nothing on failure.  A launch
 *     failure returns KVC_ERR_HIP (code in kvc_last_hip_error()).  Faults in
 *     kernels surface at the caller's next synchronisation.
 *   - Inputs are read-only, outputs fully overwritten, workspace contents
 *     are undefined on return.  Calls on different streams with disjoint
 *     outputs and workspaces may run concurrently.  Stateless, thread-safe.
 *   - Non-finite inputs are undefined behaviour, unless the environment
 *     sets KVC_CHECK_INPUTS=1: then kvc_compress and kvc_compress_layers
 *     first check every query, key and value element of the call's units
 *     (finite) and every head score (finite, >= 0), wait on `stream` for
 *     the result and return KVC_ERR_INVALID_ARG without compressing on a
 *     violation (a checking mode: it reads all of K and V once more and
 *     synchronises).
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = 1, /* null pointer, bad range, bad stride/alignment */
  KVC_ERR_UNSUPPORTED = 2, /* a valid problem outside what the kernels take */
  KVC_ERR_BUDGET = 3,      /* L <= w, or w + r > kbar for some sequence   */
  KVC_ERR_WORKSPACE = 4,   /* workspace_bytes below kvc_plan's figure     */
  KVC_ERR_HIP = 5          /* a HIP launch failed                         */
} kvc_status;

typedef enum { KVC_BF16 = 0, KVC_F32 = 1 } kvc_dtype;

/* Method parameters (AudioKV article, section 5.1 defaults in brackets). */
typedef struct {
  double alpha;      /* SSS blend weight, 0 <= alpha <= 1              [0.5] */
  double rho;        /* SSS energy cutoff ratio, 0 < rho <= 1          [0.7] */
  int32_t window;    /* w, most recent positions always kept, >= 0      [32] */
  double base_ratio; /* r = floor(base_ratio * kbar), 0 <= . <= 1      [0.5] */
  int32_t budget_pool; /* which heads share one budget pool (a kvc_pool)  [0] */
  int32_t score_pool;  /* pooling of step 1 over query heads (kvc_score) [0] */
} kvc_params;

/* Pooling of step 1 over the KV head's G query heads.  AudioKV's article
 * (section 1.2) does not say how the group's attention rows are combined:
 *   KVC_SCORE_MEAN  s = mean over all G*W window queries (per head mean,
 *                   then mean over heads)
 *   KVC_SCORE_MAX   s = max over the G heads of each head's mean over its
 *                   W window queries (a strongly attending head is not
 *                   averaged away, as in C3's max over a group's query
 *                   heads); needs n_window_q a multiple of 32. */
typedef enum { KVC_SCORE_MEAN = 0, KVC_SCORE_MAX = 1 } kvc_score;

/* Budget pool of step 3.  AudioKV's section 3.1 indexes the audio score by
 * layer and head without saying whether the score-proportional share is
 * split across the whole model or within each layer:
 *   KVC_POOL_SEQUENCE  one pool per sequence: all n_layers*n_kv_heads heads
 *   KVC_POOL_LAYER     one pool per (sequence, layer): its n_kv_heads heads
 * Either way every pool of n heads keeps n*min(kbar, L) rows in total. */
typedef enum { KVC_POOL_SEQUENCE = 0, KVC_POOL_LAYER = 1 } kvc_pool;

/* Problem shape.  Supported: 1 <= n_seq <= 64; head_dim in {64, 128};
 * gqa_group * n_window_q a multiple of 32 and at most 256; every sequence
 * length L with 64 <= L <= 65536 and L > window.  Lengths that are not
 * powers of two take the transform of step 2 through Bluestein's algorithm
 * (the chirp-z form of the DFT of length L, or of the L/2 packed values for
 * even L, as a convolution done with power-of-two FFTs: in one workgroup
 * up to 16384 points, beyond that split into transforms of 32768 points
 * across workgroups); n_layers * n_kv_heads <= 4096; k_stride[2] < 2^24. */
typedef struct {
  int32_t n_seq, n_layers, n_kv_heads, gqa_group, head_dim, n_window_q;
  kvc_dtype dtype;            /* element type of q, k, v, k_out, v_out     */
  const int64_t *seq_start;   /* host [n_seq+1], increasing: sequence i is
                                 tokens seq_start[i] .. seq_start[i+1]-1 of
                                 the K/V token axis                          */
  const double *retention;    /* host [n_seq], kept fraction in (0, 1]:
                                 kbar_i = floor(retention_i * L_i)          */
  int64_t k_stride[3];        /* elements between consecutive layers, KV
                                 heads, tokens of k; head_dim contiguous     */
  int64_t v_stride[3];        /* same for v.  Token rows 16-byte aligned.    */
} kvc_problem;

/* Sizing, on the host, no device work.  total_rows = sum over sequences of
 * n_layers*n_kv_heads*min(kbar_i, L_i) (the budgets sum to exactly this);
 * workspace_bytes is what kvc_compress and kvc_scores need.  Either output
 * pointer may be NULL. */
kvc_status kvc_plan(const kvc_problem *prob, const kvc_params *params,
                    int64_t *total_rows, size_t *workspace_bytes);

/* The whole path (steps 1-5) in one call.
 *   q_window    device [n_seq][n_layers][n_kv_heads*gqa_group][n_window_q]
 *               [head_dim]; q head j belongs to KV head j / gqa_group
 *   k, v        device, strided as in kvc_problem
 *   head_scores device float [n_layers][n_kv_heads], finite and >= 0 (the
 *               audio-head score S_{l,h}, the same for every sequence)
 *   k_out,v_out device [total_rows][head_dim], dtype of k/v
 *   idx_out     device int32 [total_rows]: kept positions (0-based within
 *               the sequence), ascending within each unit's segment
 *   seg_offsets device int64 [units+1]: unit u's rows are
 *               seg_offsets[u] .. seg_offsets[u+1]-1
 *   budgets     device int32 [units]
 *   workspace   device, >= kvc_plan's workspace_bytes, 256-byte aligned */
kvc_status kvc_compress(const kvc_problem *prob, const kvc_params *params,
                        const void *q_window, const void *k, const void *v,
                        const float *head_scores, void *k_out, void *v_out,
                        int32_t *idx_out, int64_t *seg_offsets,
                        int32_t *budgets, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Streaming prefill: steps 1-5 for the units of layers [layer_begin,
 * layer_end) only, so a caller can compress each layer (or group of layers)
 * as soon as its K/V exist.  Budgets and offsets depend only on the head
 * scores, the lengths and the retention, so they are computed for every unit
 * on every call (identically); the rows of the range's units land at their
 * final places in the whole-problem outputs, which the other layers' calls
 * fill in turn.  Arguments as for kvc_compress, except:
 *   q_window  device [n_seq][layer_end-layer_begin][n_kv_heads*gqa_group]
 *             [n_window_q][head_dim]: the range's window queries only
 *   k, v      device, element (l, h, t, c) of layer l in the range at
 *             (l - layer_begin)*stride[0] + h*stride[1] + t*stride[2] + c:
 *             pointers to the range's first layer, prob's strides
 *   k_out, v_out, idx_out, seg_offsets, budgets, workspace: sized for the
 *             whole problem (kvc_plan); rows of other layers are untouched.
 * 0 <= layer_begin < layer_end <= n_layers, else KVC_ERR_INVALID_ARG. */
kvc_status kvc_compress_layers(const kvc_problem *prob, const kvc_params *params,
                               int32_t layer_begin, int32_t layer_end,
                               const void *q_window, const void *k, const void *v,
                               const float *head_scores, void *k_out, void *v_out,
                               int32_t *idx_out, int64_t *seg_offsets,
                               int32_t *budgets, void *workspace,
                               size_t workspace_bytes, void *stream);

/* kvc_compress for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and arguments without a workspace.  The library
 * keeps the workspace in a static device array of KVC_NOALLOC_MAX_WORKSPACE
 * bytes, one copy per GPU, held from the first call on a device (the
 * current device) until the process ends; the call itself allocates and
 * frees nothing.  A problem whose kvc_plan workspace_bytes exceeds the
 * limit returns KVC_ERR_WORKSPACE before touching the device (48 layers x
 * 4 KV heads at L = 32768 need about 36 MiB).  All calls on one device
 * share its array: calls that overlap in time on one device (different
 * streams, or threads) race and must be serialised by the caller. */
#define KVC_NOALLOC_MAX_WORKSPACE (64u << 20)
kvc_status kvc_compress_noalloc(const kvc_problem *prob, const kvc_params *params,
                                const void *q_window, const void *k, const void *v,
                                const float *head_scores, void *k_out, void *v_out,
                                int32_t *idx_out, int64_t *seg_offsets,
                                int32_t *budgets, void *stream);

/* Stage entry points, same conventions; they run the kernels kvc_compress
 * runs, one step at a time.
 *
 * kvc_scores: step 1 -> s, device float varlen rows (see above).
 * kvc_smooth: step 2 on given rows s -> s_hat (same layout) and kstar
 *             (device int32 [units]).  The workspace (256-byte aligned,
 *             kvc_plan's workspace_bytes suffice) is used only when some
 *             length is not a power of two; it may be NULL otherwise.
 * kvc_budget: step 3 -> budgets [units], seg_offsets [units+1].
 * kvc_select: step 4 on given rows s_hat with given budgets/offsets ->
 *             idx_out.  s_hat must be finite; seg_offsets must be the
 *             exclusive prefix sum of budgets (seg_offsets[0] = 0) with
 *             min(window, L) <= budgets[u] <= L.
 * kvc_gather: step 5 for given idx/offsets -> k_out, v_out.  Every
 *             position must lie in [0, L) of its unit's sequence and every
 *             offset in [0, total_rows].  Out-of-range positions are read
 *             as position 0 (the kernel never reads outside the row), so
 *             the call returns KVC_OK with wrong rows; bad offsets are
 *             undefined behaviour.
 * With KVC_CHECK_INPUTS=1 in the environment, kvc_select and kvc_gather
 * first check these conditions on the device (positions, offsets, budgets,
 * finite s_hat), wait on `stream` for the result and return
 * KVC_ERR_INVALID_ARG, launching nothing else, on a violation. */
kvc_status kvc_scores(const kvc_problem *prob, const kvc_params *params,
                      const void *q_window, const void *k, float *s,
                      void *workspace, size_t workspace_bytes, void *stream);
/* The two passes of step 1, as kvc_scores runs them:
 * kvc_score_stats: per window query, the log-sum-exp of its logits over the
 *                  L keys, left in `workspace` (log2 units) for
 * kvc_score_pool:  the pooled softmax rows s, given that workspace.
 * kvc_score_stats followed by kvc_score_pool on the same workspace equals
 * kvc_scores. */
kvc_status kvc_score_stats(const kvc_problem *prob, const kvc_params *params,
                           const void *q_window, const void *k, void *workspace,
                           size_t workspace_bytes, void *stream);
kvc_status kvc_score_pool(const kvc_problem *prob, const kvc_params *params,
                          const void *q_window, const void *k, float *s,
                          void *workspace, size_t workspace_bytes, void *stream);
kvc_status kvc_smooth(const kvc_problem *prob, const kvc_params *params,
                      const float *s, float *s_hat, int32_t *kstar,
                      void *workspace, size_t workspace_bytes, void *stream);
kvc_status kvc_budget(const kvc_problem *prob, const kvc_params *params,
                      const float *head_scores, int32_t *budgets,
                      int64_t *seg_offsets, void *stream);
kvc_status kvc_select(const kvc_problem *prob, const kvc_params *params,
                      const float *s_hat, const int32_t *budgets,
                      const int64_t *seg_offsets, int32_t *idx_out,
                      void *stream);
kvc_status kvc_gather(const kvc_problem *prob, const kvc_params *params,
                      const void *k, const void *v, const int32_t *idx,
                      const int64_t *seg_offsets, void *k_out, void *v_out,
                      void *stream);

/* Static text for a status; never NULL. */
const char *kvc_status_str(kvc_status status);
/* hipError_t of the calling thread's last KVC_ERR_HIP, 0 if none. */
int kvc_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
