/*
 * kvc_c3.h -- C ABI of libkvc's query-guided retrieval of audio KV on AMD
 * Instinct MI355X (gfx950): C3 (C3 digest page, "C3: Speech-Guided KV
 * Retrieval for Long-Context SpeechLLM Inference"; sections on the overall
 * flow, shared competition, content clustering and adaptive resolution, and
 * the reproduction notes: 8 k-means iterations, seed 0, initial granularity
 * 16, lambda = 0.5, R = 2, retrieval bypassed when the audio fits B).
 *
 * Per cache u = (sequence, layer, KV head) of n audio keys:
 *
 *   build (prefill)  recursive bisecting 2-means over the keys: a node with
 *                    more than 4 keys splits by 8 Lloyd iterations started
 *                    from two member keys picked by SplitMix64 of
 *                    (seed, u, depth, start, size); depth <= 24.  The
 *                    initial frontier is every node at depth
 *                    round(log2(n / 16)) plus the leaves above it.
 *   step (decode)    sigma_i = max over the G query heads of the group of
 *                    cos(q_g, c_i) for every frontier node i; nodes ranked by
 *                    sigma descending (ties: earlier start), whole nodes
 *                    taken until B keys (the crossing node gives the first
 *                    members of its range); kept positions listed ascending;
 *                    K, V rows gathered.  Then e = lambda e + (1 - lambda)
 *                    sigma, and min(#splits, #merges) exchanges: the R
 *                    frontier nodes with children of highest e split into
 *                    their children (which inherit e), the R sibling pairs of
 *                    lowest max(e_left, e_right), neither a split candidate,
 *                    merge into their parent (which takes that max).
 *                    A cache with n <= B keeps all n rows and its state.
 *
 * Every split decision is defined so that it is reproducible bit for bit:
 * keys snapped to the grid 2^-24 (only |k| < 2^-17 moves), exact fp64
 * member sums, each mean = sum / count correctly rounded in fp64;
 * assignment by s(k) > b with w = mu1 - mu0 rounded to fp32 then to 16
 * significant bits (|w| < 2^-100 -> 0), s(k) = sum_c k_c w_c in fp32 in
 * column order (exact products, so fused multiply-add changes nothing),
 * b = fp32 sum in column order of the rounded products
 * w_c * fp32((mu0_c + mu1_c) / 2); a key with
 * s(k) = b joins cluster 0 (the left child).  Members keep their relative
 * order.  Stored centroids are the exact means rounded to fp32 then bf16.
 * Nodes are numbered breadth first (children in parent order, left first).
 *
 * Conventions are those of kvc.h (device pointers, all work on `stream`,
 * validation synchronous, nothing launched on failure, inputs read-only),
 * with one exception: kvc_c3_build waits on `stream` once per tree level to
 * learn whether another level exists, and once at the end, so it returns
 * with its work finished.  Keys must be bf16, finite, |k| < 4096; a key
 * outside that range makes kvc_c3_build return KVC_ERR_INVALID_ARG after its
 * work (the index is then unspecified).
 *
 * Layouts (elements unless stated):
 *   k, v        device bf16: row t of cache u at u*stride[0] + t*stride[1],
 *               head_dim contiguous, 16-byte aligned rows
 *   k_out,v_out device bf16: row t of cache u at u*out_stride[0] +
 *               t*out_stride[1]; rows 0..min(n,B)-1 written
 *   q           device bf16 [units][G][head_dim]: the step's queries
 *   idx_out     device int32 [units][kept_cap]: kept positions, ascending,
 *               entries 0..min(n,B)-1 written
 *   sigma       device float [units][capacity]: entries 0..A_u-1
 *   index       device, index_bytes (kvc_c3_plan), 256-byte aligned; byte
 *               offsets of its arrays in kvc_c3_layout, NC = node_cap:
 *                 int32 start/size/left/parent/depth [units][NC]
 *                   (left = -1 for a leaf, right child = left + 1,
 *                    parent = -1 for the root)
 *                 int32 perm [units][capacity]: the members of node x are
 *                   perm[start[x] .. start[x] + size[x])
 *                 int32 n_nodes [units]
 *                 bf16 centroid [units][NC][head_dim]
 *   state       device, state_bytes, 256-byte aligned:
 *                 int32 count [units]: A_u, frontier entries
 *                 int32 frontier [units][capacity]: node ids, by start
 *                 double ema [units][capacity]: e per entry
 * with units = n_seq * n_layers * n_kv_heads in (sequence, layer, head)
 * order.  The library writes the index and states; callers read them.
 */
#ifndef KVC_C3_H
#define KVC_C3_H

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  double lambda;     /* EMA smoothing, 0 <= lambda <= 1            [0.5] */
  int32_t r_swaps;   /* R, exchanges per step, 0 <= R <= 8           [2] */
  uint64_t seed;     /* initial-centroid seed                        [0] */
} kvc_c3_params;

/* Supported: 1 <= n_seq <= 64; head_dim in {64, 128}; 1 <= gqa_group <= 32;
 * 1 <= capacity <= 131072; n_layers * n_kv_heads <= 4096. */
typedef struct {
  int32_t n_seq, n_layers, n_kv_heads, gqa_group, head_dim;
  int64_t capacity;           /* rows per cache in k and v                 */
  const int64_t *len;         /* host [n_seq]: n, 0 <= n <= capacity        */
  const int64_t *budget;      /* host [n_seq]: B >= 1                       */
  int64_t k_stride[2];        /* elements between caches, between rows      */
  int64_t v_stride[2];
  int64_t out_stride[2];      /* k_out and v_out                            */
} kvc_c3_problem;

typedef struct {
  int64_t node_cap;           /* NC = 2 * capacity                          */
  int64_t kept_cap;           /* max over sequences of min(n, B)            */
  size_t index_bytes, state_bytes;
  size_t build_workspace_bytes, step_workspace_bytes;
  size_t start, size, left, parent, depth, perm, n_nodes, centroid; /* index */
  size_t count, frontier, ema;                                       /* state */
} kvc_c3_layout;

/* Host only: sizes and offsets for a problem. */
kvc_status kvc_c3_plan(const kvc_c3_problem *prob, const kvc_c3_params *params,
                       kvc_c3_layout *layout);

/* Prefill: builds every cache's tree into `index` and writes the initial
 * frontier (e = 0) into `state`.  Waits on `stream` (see above). */
kvc_status kvc_c3_build(const kvc_c3_problem *prob, const kvc_c3_params *params,
                        const void *k, void *index, void *state, void *workspace,
                        size_t workspace_bytes, void *stream);

/* One decode step: scores, selection, gather and frontier update.  state_in
 * is read, state_out written (distinct buffers; the caller swaps them). */
kvc_status kvc_c3_step(const kvc_c3_problem *prob, const kvc_c3_params *params,
                       const void *index, const void *state_in, void *state_out,
                       const void *q, const void *k, const void *v, void *k_out,
                       void *v_out, int32_t *idx_out, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Stage entry points, running the kernels kvc_c3_step runs:
 * kvc_c3_score:  sigma of every frontier entry (caches with n <= B are
 *                skipped and their sigma left untouched).
 * kvc_c3_select: kept positions for given sigma -> idx_out.
 * kvc_c3_update: EMA and split/merge for given sigma -> state_out.
 * kvc_c3_gather: K, V rows of given kept positions -> k_out, v_out. */
kvc_status kvc_c3_score(const kvc_c3_problem *prob, const kvc_c3_params *params,
                        const void *index, const void *state, const void *q,
                        float *sigma, void *stream);
kvc_status kvc_c3_select(const kvc_c3_problem *prob, const kvc_c3_params *params,
                         const void *index, const void *state, const float *sigma,
                         int32_t *idx_out, void *stream);
kvc_status kvc_c3_update(const kvc_c3_problem *prob, const kvc_c3_params *params,
                         const void *index, const void *state_in, const float *sigma,
                         void *state_out, void *stream);
kvc_status kvc_c3_gather(const kvc_c3_problem *prob, const kvc_c3_params *params,
                         const void *k, const void *v, const int32_t *idx,
                         void *k_out, void *v_out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KVC_C3_H */
