/*
 * kvc_voxzip.h -- C ABI of libkvc's decode-time cache eviction on AMD
 * Instinct MI355X (gfx950): VoxZip's temporally decayed accumulated
 * attention (VoxZip digest page "VoxZip: Semantic-Anchored Temporal KV
 * Cache Compression for Long-Context Audio Inference", method overview,
 * second stage "Temporally Decayed KV Cache Eviction"; gamma = 0.95, T = 4
 * sinks and a recent window of 20 % of the budget from its details list).
 *
 * One decode step, per cache u = (sequence, layer, KV head) holding n rows
 * (the last one is the new token's key/value, already appended):
 *
 *   1. accumulate  p_g = softmax_j(q_g . k_j / sqrt(d)) over the n rows for
 *                  each of the G query heads of the KV head's group;
 *                  A[j] = gamma * A_prev[j] + mean_g p_g[j]   (j < n-1)
 *                  A[n-1] = mean_g p_g[n-1]
 *   2. evict       if n > B (the cache budget): keep the first T rows, the
 *                  last M = floor(recent_frac * B) rows and the N = B - T - M
 *                  rows of largest A among [T, n - M) (equal values: lower
 *                  position first; -0.0 equals +0.0); otherwise keep all n
 *   3. gather      K_out[t] = K[kept[t]], V_out[t] = V[kept[t]],
 *                  A_out[t] = A[kept[t]], kept listed in ascending order
 *                  (the page's concatenation K[:T], K[I_hist], K[-M:])
 *
 * The page leaves open how A is trimmed after eviction; here it is gathered
 * with the same kept positions as K and V.  The page keeps A per layer; with
 * grouped-query attention each KV head's cache is evicted on its own here,
 * its query heads' rows averaged.
 *
 * Conventions are those of kvc.h: device pointers on the current device,
 * no allocation, no synchronisation, all work enqueued on `stream`;
 * validation is synchronous and launches nothing on failure; inputs are
 * read-only; outputs and workspace must not alias inputs.
 *
 * Layouts (elements):
 *   q          device [units][G][head_dim], dtype, contiguous: the new
 *              token's query for each query head of the group
 *   k, v       device: row t of cache u at u*stride[0] + t*stride[1];
 *              head_dim contiguous, rows 16-byte aligned; k_out and v_out
 *              use the same strides (a second set of cache buffers)
 *   a_prev     device float [units][capacity]: entries 0..n-2 used
 *   a_out      device float [units][capacity]: entries 0..new_len-1 written
 *   idx_out    device int32 [units][capacity]: kept positions, entries
 *              0..new_len-1 written
 * with units = n_seq * n_layers * n_kv_heads in (sequence, layer, head)
 * order and new_len = min(n, B) per sequence.
 */
#ifndef KVC_VOXZIP_H
#define KVC_VOXZIP_H

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  double gamma;       /* decay of the accumulated attention, finite, >= 0 [0.95] */
  int32_t n_sink;     /* T, leading rows always kept, >= 0                  [4] */
  double recent_frac; /* M = floor(recent_frac * B), 0 <= . <= 1          [0.2] */
} kvc_vz_params;

/* Supported: 1 <= n_seq <= 64; head_dim in {64, 128}; 1 <= gqa_group <= 32;
 * 1 <= capacity <= 65536; n_layers * n_kv_heads <= 4096. */
typedef struct {
  int32_t n_seq, n_layers, n_kv_heads, gqa_group, head_dim;
  kvc_dtype dtype;            /* element type of q, k, v, k_out, v_out          */
  int64_t capacity;           /* rows per cache in every cache-shaped buffer    */
  const int64_t *len;         /* host [n_seq]: rows n in each cache of sequence
                                 i, new token included, 1 <= n <= capacity      */
  const int64_t *budget;      /* host [n_seq]: B, with T + M <= B               */
  int64_t k_stride[2];        /* elements between caches, between rows of k     */
  int64_t v_stride[2];        /* same for v                                     */
} kvc_vz_problem;

/* Host only.  new_len (host [n_seq], may be NULL) receives min(n, B);
 * workspace_bytes (may be NULL) what kvc_vz_step and kvc_vz_accumulate
 * need. */
kvc_status kvc_vz_plan(const kvc_vz_problem *prob, const kvc_vz_params *params,
                       int64_t *new_len, size_t *workspace_bytes);

/* Steps 1-3 in one call.  workspace: device, 256-byte aligned, at least
 * kvc_vz_plan's workspace_bytes. */
kvc_status kvc_vz_step(const kvc_vz_problem *prob, const kvc_vz_params *params,
                       const void *q, const void *k, const void *v,
                       const float *a_prev, void *k_out, void *v_out,
                       float *a_out, int32_t *idx_out, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Stage entry points, running the kernels kvc_vz_step runs:
 * kvc_vz_accumulate: step 1 -> a (device float [units][capacity], entries
 *                    0..n-1), A before eviction.
 * kvc_vz_evict:      step 2 on given A -> idx_out.  A must be finite.
 * kvc_vz_gather:     step 3 for given A and kept positions -> k_out, v_out,
 *                    a_out.  Positions outside [0, n) read row 0. */
kvc_status kvc_vz_accumulate(const kvc_vz_problem *prob, const kvc_vz_params *params,
                             const void *q, const void *k, const float *a_prev,
                             float *a, void *workspace, size_t workspace_bytes,
                             void *stream);
kvc_status kvc_vz_evict(const kvc_vz_problem *prob, const kvc_vz_params *params,
                        const float *a, int32_t *idx_out, void *stream);
kvc_status kvc_vz_gather(const kvc_vz_problem *prob, const kvc_vz_params *params,
                         const void *k, const void *v, const float *a,
                         const int32_t *idx, void *k_out, void *v_out,
                         float *a_out, void *stream);

/* The decode step with the cache kept in place, for token-by-token decoding
 * where at most one row leaves a cache per step (n <= B + 1 for every
 * sequence, else KVC_ERR_UNSUPPORTED).  Instead of compacting the kept rows
 * into new buffers, every cache keeps its rows in slots 0..n-1 of k (and
 * of the caller's v, which the step never reads) and records in pos[s] the
 * place of slot s's row in the page's concatenated order (older rows lower;
 * a compact cache has pos[s] = s).  Per cache:
 *   1. accumulate  as kvc_vz_step, over the n slots: a[s] = gamma a[s] +
 *                  mean_g p_g[s] (the new token's slot holds a = 0)
 *   2. evict       if n > B: among the slots whose place is neither among
 *                  the T lowest nor the M highest, the one of smallest a
 *                  (equal values: the highest place) leaves -- the
 *                  complement of the N kept middle rows of kvc_vz_step
 *   3. free_slot[u] = the slot for the next token's row: the one that left,
 *                  else n while the cache grows (n < capacity), else -1;
 *                  its a is set to 0 and its pos to the next place.
 * Reading the slots in pos order gives kvc_vz_step's k_out, v_out, a_out.
 * The caller writes the next token's key and value into slot free_slot[u]
 * and calls again with n = min(n, B) + 1.  Per step only K is read (for
 * the logits), a and pos updated; no row moves.
 *   a          device float [units][capacity], in/out
 *   pos        device int32 [units][capacity], in/out
 *   free_slot  device int32 [units], out
 *   workspace  device, 256-byte aligned, >= kvc_vz_plan's workspace_bytes */
kvc_status kvc_vz_step_inplace(const kvc_vz_problem *prob, const kvc_vz_params *params,
                               const void *q, const void *k, float *a, int32_t *pos,
                               int32_t *free_slot, void *workspace, size_t workspace_bytes,
                               void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KVC_VOXZIP_H */
