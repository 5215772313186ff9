/*
 * kvc_wnw.h -- C ABI of libkvc's decode-time chunk recall on AMD Instinct
 * MI355X (gfx950): WnW (WnW digest page, "WnW: Waxing-and-Waning KV Cache for
 * Long-Form Speech LLMs"; the summary and method sections on anchor, tidal
 * and fixed KV heads, and the reproduction notes: 4 s chunks with a 2 s
 * stride, the top 3 chunks per step, release after 3 consecutive unselected
 * steps, 5 anchor heads, a host copy of every tidal head's KV).
 *
 * Roles come from an offline calibration (outside this library) as a table
 * of one role per KV head, shared by all sequences:
 *   anchor  the head's whole audio KV stays on the GPU; its attention over
 *           the audio drives the recall;
 *   tidal   the head's whole audio KV lives in host memory; the GPU holds the
 *           recalled blocks in a slot buffer;
 *   fixed   a static subset chosen at prefill, segment by segment
 *           (kvc_wnw_fixed_select).
 *
 * Per sequence of n audio tokens, with stride S and chunk length W = m S
 * (tokens; 4 s and 2 s at the model's audio token rate):
 *   block b   positions [b S, min((b + 1) S, n)), B = ceil(n / S) blocks
 *   chunk c   blocks c .. min(c + m, B) - 1, C = max(1, B - m + 1) chunks
 * One decode step (kvc_wnw_step):
 *   1. p_a[j] = mean over the G query heads of anchor a of
 *      softmax_j(q_g . k_j / sqrt(d)) over the n audio keys;
 *   2. sigma_c = sum over anchors of the mass of p_a on chunk c (computed as
 *      per-block masses, then summed over the chunk's blocks in order);
 *   3. the K chunks of largest sigma (ties: lower index) are selected;
 *   4. residency: a selected chunk gets idle count 0; a resident chunk not
 *      selected counts one more idle step and is released when the count
 *      reaches H; a block is resident while a resident chunk covers it;
 *      blocks that stay resident keep their slot, released blocks free
 *      theirs, newly resident blocks (ascending) take the free slots
 *      (ascending);
 *   5. recall: every tidal head's rows of each newly resident block are
 *      copied from its host copy into its slot (rows s*S .. s*S + rows - 1
 *      of the slot buffer).
 * The residency is per sequence, shared by all of its tidal heads.
 *
 * Conventions are those of kvc.h (device pointers unless stated, all work on
 * `stream`, validation synchronous, nothing launched on failure, inputs
 * read-only, state_in and state_out distinct).
 *
 * Layouts (elements unless stated; units u = (sequence, layer, KV head) in
 * that order, U = n_seq * n_layers * n_kv_heads):
 *   k        device bf16: row t of unit u at u*k_stride[0] + t*k_stride[1],
 *            head_dim contiguous; only anchor units are read
 *   q        device bf16 [n_seq][n_anchor][G][head_dim]: the step's queries
 *            of the anchor heads, anchors in (layer, head) order
 *   host_k,  host memory from hipHostMalloc (page-locked, device-accessible):
 *   host_v   row t of unit u at u*host_stride[0] + t*host_stride[1]; only
 *            tidal units are read (pageable memory is rejected)
 *   slot_k,  device bf16: slot row r of unit u at u*slot_stride[0] +
 *   slot_v   r*slot_stride[1], r < slot_cap * S; only tidal units written
 *   sigma    device float [n_seq][chunk_cap]: entries 0..C_i-1
 *   state    device, state_bytes, 256-byte aligned; byte offsets in
 *            kvc_wnw_layout:
 *              int32 idle [n_seq][chunk_cap]   -1 = not resident, else the
 *                                               consecutive unselected steps
 *              int32 slot_of_block [n_seq][block_cap]  slot or -1
 *              int32 block_of_slot [n_seq][slot_cap]   block or -1
 *              int32 selected [n_seq][top_chunks]  this step's chunks by
 *                                               score (entries past C_i: -1)
 *              int32 n_recalled [n_seq]
 *              int32 recalled_block, recalled_slot [n_seq][slot_cap]
 *                                               this step's recalls, by block
 */
#ifndef KVC_WNW_H
#define KVC_WNW_H

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { KVC_WNW_FIXED = 0, KVC_WNW_ANCHOR = 1, KVC_WNW_TIDAL = 2 };

typedef struct {
  int32_t chunk_len;      /* W, tokens per chunk (4 s), a multiple of S  [50] */
  int32_t chunk_stride;   /* S, tokens between chunk starts (2 s)         [25] */
  int32_t top_chunks;     /* K, chunks selected per step, 1 <= K <= 8      [3] */
  int32_t release_after;  /* H, unselected steps to release, 1 <= H <= 8   [3] */
} kvc_wnw_params;

/* Supported: 1 <= n_seq <= 64; head_dim in {64, 128}; 1 <= gqa_group <= 32;
 * 1 <= n <= capacity <= 131072; n_layers * n_kv_heads <= 4096; 1 to 64
 * anchor heads; W / S <= 8; C_i <= 65536. */
typedef struct {
  int32_t n_seq, n_layers, n_kv_heads, gqa_group, head_dim;
  int64_t capacity;          /* audio rows per unit in k and the host copies */
  const int64_t *len;        /* host [n_seq]: n                             */
  const uint8_t *role;       /* host [n_layers * n_kv_heads]: KVC_WNW_*     */
  int64_t k_stride[2];       /* anchors' keys: between units, between rows   */
  int64_t host_stride[2];    /* host_k and host_v                            */
  int64_t slot_stride[2];    /* slot_k and slot_v                            */
} kvc_wnw_problem;

typedef struct {
  int32_t n_anchor, n_tidal;
  int32_t block_cap, chunk_cap;  /* max over sequences of B_i and C_i        */
  int32_t slot_cap;              /* K * H * W / S: blocks per tidal slot buffer */
  size_t state_bytes, workspace_bytes;
  size_t idle, slot_of_block, block_of_slot, selected, n_recalled, recalled_block,
      recalled_slot;             /* byte offsets in state                     */
} kvc_wnw_layout;

/* Host only: sizes and offsets. */
kvc_status kvc_wnw_plan(const kvc_wnw_problem *prob, const kvc_wnw_params *params,
                        kvc_wnw_layout *layout);

/* The state before the first step: nothing resident, every slot free. */
kvc_status kvc_wnw_init(const kvc_wnw_problem *prob, const kvc_wnw_params *params, void *state,
                        void *stream);

/* One decode step: chunk scores from the anchors, selection, residency and
 * slots (state_in -> state_out), and the recall copies of the tidal heads.
 * sigma may be NULL. */
kvc_status kvc_wnw_step(const kvc_wnw_problem *prob, const kvc_wnw_params *params,
                        const void *q, const void *k, const void *state_in, void *state_out,
                        const void *host_k, const void *host_v, void *slot_k, void *slot_v,
                        float *sigma, void *workspace, size_t workspace_bytes, void *stream);

/* Stage entry points, running the kernels kvc_wnw_step runs:
 * kvc_wnw_chunk_scores: steps 1-2 -> sigma.
 * kvc_wnw_update:       steps 3-4 for given sigma -> state_out.
 * kvc_wnw_recall:       step 5 for the recalls listed in state. */
kvc_status kvc_wnw_chunk_scores(const kvc_wnw_problem *prob, const kvc_wnw_params *params,
                                const void *q, const void *k, float *sigma, void *workspace,
                                size_t workspace_bytes, void *stream);
kvc_status kvc_wnw_update(const kvc_wnw_problem *prob, const kvc_wnw_params *params,
                          const float *sigma, const void *state_in, void *state_out,
                          void *stream);
kvc_status kvc_wnw_recall(const kvc_wnw_problem *prob, const kvc_wnw_params *params,
                          const void *state, const void *host_k, const void *host_v,
                          void *slot_k, void *slot_v, void *stream);

/* Fixed heads at prefill: per-unit selection as kvc_select (same problem,
 * s_hat rows, budgets, offsets and output), except that the k = b - w kept
 * candidates are shared among segments [j seg, (j + 1) seg) of [0, L - w) in
 * proportion to their lengths (largest remainder, ties to the lower
 * segment), each segment keeping its quota of largest s_hat (ties: lower
 * position).  1 <= seg_len <= 64. */
kvc_status kvc_wnw_fixed_select(const kvc_problem *prob, const kvc_params *params,
                                int32_t seg_len, const float *s_hat, const int32_t *budgets,
                                const int64_t *seg_offsets, int32_t *idx_out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KVC_WNW_H */
