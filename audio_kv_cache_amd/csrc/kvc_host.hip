// kvc_host.hip -- the C ABI of include/kvc.h: validation, sizing, workspace
// carving and kernel launches.  No allocation, no synchronisation: every
// entry point enqueues on the caller's stream and returns.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "../../include/kvc.h"
#include "kvc_internal.h"
#include "kvc_wnw.h"

static thread_local int g_last_hip_error = 0;

static kvc_status hip_status(hipError_t e) {
  if (e == hipSuccess) return KVC_OK;
  g_last_hip_error = (int)e;
  return KVC_ERR_HIP;
}

extern "C" const char* kvc_status_str(kvc_status s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID_ARG: return "invalid argument";
    case KVC_ERR_UNSUPPORTED: return "unsupported problem shape";
    case KVC_ERR_BUDGET:
      return "infeasible budget (prefill: L <= window or window + base share > mean budget; "
             "decode: sinks + recent window > budget)";
    case KVC_ERR_WORKSPACE: return "workspace too small";
    case KVC_ERR_HIP: return "HIP launch failure";
  }
  return "unknown status";
}

extern "C" int kvc_last_hip_error(void) { return g_last_hip_error; }

void kvc_note_hip_error(int e) { g_last_hip_error = e; }

static bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

static size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

// kbar = floor(retention * L) in fp64, as the budget kernel computes it.
static int64_t kbar_of(double retention, int64_t L) {
  return (int64_t)floor(retention * (double)L);
}

// Validate and fill the kernel descriptor.
static kvc_status make_desc(const kvc_problem* p, const kvc_params* prm, KvcDesc* D) {
  if (!p || !prm || !D) return KVC_ERR_INVALID_ARG;
  if (!p->seq_start || !p->retention) return KVC_ERR_INVALID_ARG;
  if (p->n_seq < 1 || p->n_layers < 1 || p->n_kv_heads < 1 || p->gqa_group < 1 ||
      p->head_dim < 1 || p->n_window_q < 1)
    return KVC_ERR_INVALID_ARG;
  if (p->dtype != KVC_BF16 && p->dtype != KVC_F32) return KVC_ERR_INVALID_ARG;
  if (!(prm->alpha >= 0.0 && prm->alpha <= 1.0)) return KVC_ERR_INVALID_ARG;
  if (!(prm->rho > 0.0 && prm->rho <= 1.0)) return KVC_ERR_INVALID_ARG;
  if (!(prm->base_ratio >= 0.0 && prm->base_ratio <= 1.0)) return KVC_ERR_INVALID_ARG;
  if (prm->window < 0) return KVC_ERR_INVALID_ARG;
  if (prm->budget_pool != KVC_POOL_SEQUENCE && prm->budget_pool != KVC_POOL_LAYER)
    return KVC_ERR_INVALID_ARG;
  if (prm->score_pool != KVC_SCORE_MEAN && prm->score_pool != KVC_SCORE_MAX)
    return KVC_ERR_INVALID_ARG;
  const int esz = p->dtype == KVC_BF16 ? 2 : 4;
  for (int a = 0; a < 3; ++a)
    if (p->k_stride[a] < 0 || p->v_stride[a] < 0) return KVC_ERR_INVALID_ARG;
  if (p->k_stride[2] < p->head_dim || p->v_stride[2] < p->head_dim) return KVC_ERR_INVALID_ARG;
  for (int a = 0; a < 3; ++a)
    if ((p->k_stride[a] * esz) % 16 || (p->v_stride[a] * esz) % 16) return KVC_ERR_INVALID_ARG;
  for (int i = 0; i < p->n_seq && i < KVC_MAX_SEQ; ++i) {
    if (!(p->retention[i] > 0.0 && p->retention[i] <= 1.0)) return KVC_ERR_INVALID_ARG;
    if (p->seq_start[i + 1] < p->seq_start[i] || p->seq_start[i] < 0) return KVC_ERR_INVALID_ARG;
  }

  if (p->n_seq > KVC_MAX_SEQ) return KVC_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return KVC_ERR_UNSUPPORTED;
  // the score kernels address a 64-row key chunk with 32-bit byte offsets
  if (p->k_stride[2] >= (int64_t(1) << 24)) return KVC_ERR_UNSUPPORTED;
  const int64_t gw = (int64_t)p->gqa_group * p->n_window_q;
  if (gw % 32 != 0 || gw > KVC_MAX_GW) return KVC_ERR_UNSUPPORTED;
  if (prm->score_pool == KVC_SCORE_MAX && p->n_window_q % 32 != 0) return KVC_ERR_UNSUPPORTED;
  const int64_t upseq = (int64_t)p->n_layers * p->n_kv_heads;
  if (upseq > KVC_MAX_UNITS_PER_SEQ) return KVC_ERR_UNSUPPORTED;
  if (upseq * p->n_seq > (int64_t)1 << 30) return KVC_ERR_UNSUPPORTED;

  memset(D, 0, sizeof(*D));
  D->n_seq = p->n_seq;
  D->n_layers = p->n_layers;
  D->n_heads = p->n_kv_heads;
  D->gqa = p->gqa_group;
  D->d = p->head_dim;
  D->nwin = p->n_window_q;
  D->gw = (int)gw;
  D->upseq = (int)upseq;
  D->pool_size = prm->budget_pool == KVC_POOL_LAYER ? p->n_kv_heads : (int)upseq;
  D->score_max = prm->score_pool == KVC_SCORE_MAX;
  D->layer0 = 0;
  D->q_layers = p->n_layers;
  D->window = prm->window;
  D->dtype = p->dtype == KVC_BF16 ? 0 : 1;
  D->alpha = (float)prm->alpha;
  D->rho = (float)prm->rho;
  D->base_ratio = prm->base_ratio;
  for (int a = 0; a < 3; ++a) {
    D->ks[a] = p->k_stride[a];
    D->vs[a] = p->v_stride[a];
  }
  int64_t rows = 0, srows = 0;
  int64_t tiles = 0;
  for (int i = 0; i < p->n_seq; ++i) {
    const int64_t L = p->seq_start[i + 1] - p->seq_start[i];
    // (lengths that are not powers of two take Bluestein's algorithm)
    if (L < KVC_MIN_L || L > KVC_MAX_L) return KVC_ERR_UNSUPPORTED;
    if (L <= prm->window) return KVC_ERR_BUDGET;
    const int64_t kbar = kbar_of(p->retention[i], L);
    if (kbar < L) {
      const int64_t r = (int64_t)floor(prm->base_ratio * (double)kbar);
      if ((int64_t)prm->window + r > kbar) return KVC_ERR_BUDGET;
    }
    D->tok0[i] = p->seq_start[i];
    D->L[i] = (int32_t)L;
    D->log2L[i] = is_pow2(L) ? 63 - __builtin_clzll((unsigned long long)L) : -1;
    D->retention[i] = p->retention[i];
    D->row_base[i] = rows;
    D->srow_base[i] = srows;
    D->tile_base[i] = (int32_t)tiles;
    rows += upseq * std::min(kbar, L);
    srows += upseq * L;
    tiles += upseq * kvc_tiles_per_unit((int)L);
  }
  if (tiles > INT32_MAX / 2) return KVC_ERR_UNSUPPORTED;
  D->tok0[p->n_seq] = p->seq_start[p->n_seq];
  D->row_base[p->n_seq] = rows;
  D->srow_base[p->n_seq] = srows;
  D->tile_base[p->n_seq] = (int32_t)tiles;
  D->n_units = (int)(upseq * p->n_seq);
  D->total_tiles = (int)tiles;
  return KVC_OK;
}

static size_t score_rows_bytes(const KvcDesc& D) {
  return sizeof(float) * (size_t)D.srow_base[D.n_seq];
}

// Scratch of the smoothing launches for lengths that are not powers of two
// (one launch per sequence at a time, so the largest one).
// Sequences grouped by length (in order of first appearance), units
// [lo, hi) of each: one smoothing/selection launch per group.
template <class F>
static hipError_t for_each_length_group(const KvcDesc& D, int lo, int hi, F f) {
  bool done[KVC_MAX_SEQ] = {};
  for (int i = 0; i < D.n_seq; ++i) {
    if (done[i]) continue;
    KvcSeqGroup g;
    g.n = 0;
    g.lo = lo;
    g.hi = hi;
    for (int j = i; j < D.n_seq; ++j)
      if (!done[j] && D.L[j] == D.L[i]) {
        g.seq[g.n++] = (uint8_t)j;
        done[j] = true;
      }
    const hipError_t e = f(g);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static size_t sss_scratch_bytes(const KvcDesc& D) {
  size_t m = 0;
  (void)for_each_length_group(D, 0, D.upseq, [&](const KvcSeqGroup& g) {
    m = std::max(m, kvc_sss_scratch_bytes(D.L[g.seq[0]], g.n * D.upseq));
    return hipSuccess;
  });
  return (m + 255) & ~size_t(255);
}

extern "C" kvc_status kvc_plan(const kvc_problem* prob, const kvc_params* params,
                               int64_t* total_rows, size_t* workspace_bytes) {
  KvcDesc D;
  const kvc_status st = make_desc(prob, params, &D);
  if (st != KVC_OK) return st;
  if (total_rows) *total_rows = D.row_base[D.n_seq];
  if (workspace_bytes)
    *workspace_bytes = kvc_scores_workspace(D) + up256(score_rows_bytes(D)) + sss_scratch_bytes(D);
  return KVC_OK;
}

// Workspace layout: [lse2 | partials] (kvc_scores_workspace), the score
// rows, then the smoothing scratch for lengths that are not powers of two.
struct Carve {
  float* lse2;
  float2* partials;
  float* srows;
  void* sss;
};

static Carve carve(const KvcDesc& D, void* ws) {
  char* p = (char*)ws;
  Carve c;
  c.lse2 = (float*)p;
  p += up256(sizeof(float) * (size_t)D.n_units * D.gw);
  c.partials = (float2*)p;
  p += up256(sizeof(float2) * (size_t)D.total_tiles * D.gw);
  c.srows = (float*)p;
  p += up256(score_rows_bytes(D));
  c.sss = sss_scratch_bytes(D) ? (void*)p : nullptr;
  return c;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// KVC_CHECK_INPUTS=1 in the environment: kvc_compress and kvc_compress_layers
// first check that every input element they read is finite (and the head
// scores >= 0), wait for the result, and return KVC_ERR_INVALID_ARG without
// compressing otherwise.  Read on every call.
static bool check_inputs() {
  const char* e = getenv("KVC_CHECK_INPUTS");
  return e && e[0] == '1';
}

// Run an optional check that leaves a flag in device memory the call is
// about to overwrite anyway (an output of the entry point), wait for it and
// report KVC_ERR_INVALID_ARG if it was set.
template <class F>
static kvc_status run_check(int32_t* flag, hipStream_t s, F launch) {
  hipError_t e = kvc_launch_check_clear(flag, s);
  if (e == hipSuccess) e = launch();
  int32_t bad = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&bad, flag, sizeof(bad), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e);
  return bad ? KVC_ERR_INVALID_ARG : KVC_OK;
}

static kvc_status compress_range(const kvc_problem* prob, const kvc_params* params, int lb,
                                 int le, const void* q_window, const void* k, const void* v,
                                 const float* head_scores, void* k_out, void* v_out,
                                 int32_t* idx_out, int64_t* seg_offsets, int32_t* budgets,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  KvcDesc D;
  kvc_status st = make_desc(prob, params, &D);
  if (st != KVC_OK) return st;
  if (lb < 0 || le > D.n_layers || lb >= le) return KVC_ERR_INVALID_ARG;
  D.layer0 = lb;
  D.q_layers = le - lb;
  if (!q_window || !k || !v || !head_scores || !k_out || !v_out || !idx_out || !seg_offsets ||
      !budgets || !workspace)
    return KVC_ERR_INVALID_ARG;
  if (!aligned16(q_window) || !aligned16(k) || !aligned16(v) || !aligned16(k_out) ||
      !aligned16(v_out) || ((uintptr_t)workspace & 255u))
    return KVC_ERR_INVALID_ARG;
  const size_t need = kvc_scores_workspace(D) + up256(score_rows_bytes(D)) + sss_scratch_bytes(D);
  if (workspace_bytes < need) return KVC_ERR_WORKSPACE;
  const Carve c = carve(D, workspace);
  hipStream_t s = (hipStream_t)stream;
  if (check_inputs()) {
    // Optional checks: the flag lives in the score rows, which the scores
    // overwrite afterwards; this path waits for the check's result.
    int32_t* flag = (int32_t*)c.srows;
    hipError_t e = kvc_launch_check_clear(flag, s);
    for (int seq = 0; seq < D.n_seq && e == hipSuccess; ++seq) {
      const int u0 = (seq * D.n_layers + lb) * D.n_heads, u1 = (seq * D.n_layers + le) * D.n_heads;
      e = kvc_launch_check(D, u0, u1, q_window, k, v, head_scores, flag, s);
    }
    int32_t bad = 0;
    if (e == hipSuccess) e = hipMemcpyAsync(&bad, flag, sizeof(bad), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_status(e);
    if (bad) return KVC_ERR_INVALID_ARG;
  }
  // Budgets and offsets of every unit (they depend only on S, L and the
  // retention), then one launch per step and sequence over the units of
  // layers [lb, le) (more, smaller launches cost more in launch and queue
  // latency than they save).
  // Over every unit, the statistics pass of the scores takes the budget
  // step along where it can (the budget pools' workgroups beside its tiles).
  const bool whole = lb == 0 && le == D.n_layers;
  const bool hosted = whole && kvc_scores_host_budget(D);
  hipError_t e = hipSuccess;
  if (!hosted && (e = kvc_launch_budget(D, head_scores, budgets, seg_offsets, s)) != hipSuccess)
    return hip_status(e);
  if (whole) {
    // one launch per pass over every sequence's tiles
    const KvcBudgetArgs ba{head_scores, budgets, seg_offsets};
    if ((e = kvc_launch_scores(D, 0, D.n_units, q_window, k, c.srows, c.partials, c.lse2, s, 3,
                               hosted ? &ba : nullptr)) != hipSuccess)
      return hip_status(e);
  } else {
    for (int seq = 0; seq < D.n_seq; ++seq) {
      const int u0 = (seq * D.n_layers + lb) * D.n_heads, u1 = (seq * D.n_layers + le) * D.n_heads;
      if ((e = kvc_launch_scores(D, u0, u1, q_window, k, c.srows, c.partials, c.lse2, s)) !=
          hipSuccess)
        return hip_status(e);
    }
  }
  e = for_each_length_group(D, lb * D.n_heads, le * D.n_heads, [&](const KvcSeqGroup& g) {
    return kvc_launch_sss_select(D, g, 1 | 2, c.srows, nullptr, nullptr, budgets, seg_offsets,
                                 idx_out, c.sss, s);
  });
  if (e != hipSuccess) return hip_status(e);
  if (whole) {
    e = kvc_launch_gather(D, 0, D.n_units, k, v, idx_out, seg_offsets, k_out, v_out,
                          D.row_base[D.n_seq], s);
  } else {
    for (int seq = 0; seq < D.n_seq && e == hipSuccess; ++seq) {
      const int u0 = (seq * D.n_layers + lb) * D.n_heads;
      const int u1 = (seq * D.n_layers + le) * D.n_heads;
      // grid sizing only: the layers' share of the sequence's rows
      const int64_t est = (D.row_base[seq + 1] - D.row_base[seq]) * (le - lb) / D.n_layers;
      e = kvc_launch_gather(D, u0, u1, k, v, idx_out, seg_offsets, k_out, v_out, est, s);
    }
  }
  return hip_status(e);
}

extern "C" kvc_status kvc_compress(const kvc_problem* prob, const kvc_params* params,
                                   const void* q_window, const void* k, const void* v,
                                   const float* head_scores, void* k_out, void* v_out,
                                   int32_t* idx_out, int64_t* seg_offsets, int32_t* budgets,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  const int nl = prob ? prob->n_layers : 0;
  return compress_range(prob, params, 0, nl, q_window, k, v, head_scores, k_out, v_out, idx_out,
                        seg_offsets, budgets, workspace, workspace_bytes, stream);
}

extern "C" kvc_status kvc_compress_layers(const kvc_problem* prob, const kvc_params* params,
                                          int32_t layer_begin, int32_t layer_end,
                                          const void* q_window, const void* k, const void* v,
                                          const float* head_scores, void* k_out, void* v_out,
                                          int32_t* idx_out, int64_t* seg_offsets,
                                          int32_t* budgets, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return compress_range(prob, params, layer_begin, layer_end, q_window, k, v, head_scores, k_out,
                        v_out, idx_out, seg_offsets, budgets, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// kvc_compress_noalloc: kvc_compress with its workspace in a file-scope
// device array instead of a caller's buffer.  Each GPU the library runs on
// holds its own copy of the array (KVC_NOALLOC_MAX_WORKSPACE bytes) from the
// first call on that device until the process ends; every call on a device
// shares that device's copy, so calls that overlap on one device race.  The
// workspace needs no clearing: every step writes what it later reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KVC_NOALLOC_MAX_WORKSPACE];

#define KVC_MAX_DEVICES 64
static std::atomic<void*> g_scratch_ptr[KVC_MAX_DEVICES];

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current).  In host code the array's name is
// only a stand-in for the symbol: kernels get this address instead.
static hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= KVC_MAX_DEVICES) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

extern "C" kvc_status kvc_compress_noalloc(const kvc_problem* prob, const kvc_params* params,
                                           const void* q_window, const void* k, const void* v,
                                           const float* head_scores, void* k_out, void* v_out,
                                           int32_t* idx_out, int64_t* seg_offsets,
                                           int32_t* budgets, void* stream) {
  // Everything that can be rejected on the host is rejected before the
  // device is touched.
  KvcDesc D;
  const kvc_status st = make_desc(prob, params, &D);
  if (st != KVC_OK) return st;
  const size_t need = kvc_scores_workspace(D) + up256(score_rows_bytes(D)) + sss_scratch_bytes(D);
  if (need > (size_t)KVC_NOALLOC_MAX_WORKSPACE) return KVC_ERR_WORKSPACE;
  if (!q_window || !k || !v || !head_scores || !k_out || !v_out || !idx_out || !seg_offsets ||
      !budgets)
    return KVC_ERR_INVALID_ARG;
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return hip_status(e);
  return compress_range(prob, params, 0, prob->n_layers, q_window, k, v, head_scores, k_out,
                        v_out, idx_out, seg_offsets, budgets, ws,
                        (size_t)KVC_NOALLOC_MAX_WORKSPACE, stream);
}

static kvc_status scores_common(const kvc_problem* prob, const kvc_params* params,
                                const void* q_window, const void* k, float* s_out,
                                void* workspace, size_t workspace_bytes, void* stream, int which) {
  KvcDesc D;
  kvc_status st = make_desc(prob, params, &D);
  if (st != KVC_OK) return st;
  if (!q_window || !k || !workspace || ((which & 2) && !s_out)) return KVC_ERR_INVALID_ARG;
  if (!aligned16(q_window) || !aligned16(k) || ((uintptr_t)workspace & 255u) ||
      ((uintptr_t)s_out & 7u))
    return KVC_ERR_INVALID_ARG;
  if (workspace_bytes < kvc_scores_workspace(D)) return KVC_ERR_WORKSPACE;
  const Carve c = carve(D, workspace);
  return hip_status(kvc_launch_scores(D, 0, D.n_units, q_window, k, s_out, c.partials, c.lse2,
                                      (hipStream_t)stream, which));
}

extern "C" kvc_status kvc_scores(const kvc_problem* prob, const kvc_params* params,
                                 const void* q_window, const void* k, float* s_out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return scores_common(prob, params, q_window, k, s_out, workspace, workspace_bytes, stream, 3);
}

extern "C" kvc_status kvc_score_stats(const kvc_problem* prob, const kvc_params* params,
                                      const void* q_window, const void* k, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return scores_common(prob, params, q_window, k, nullptr, workspace, workspace_bytes, stream, 1);
}

extern "C" kvc_status kvc_score_pool(const kvc_problem* prob, const kvc_params* params,
                                     const void* q_window, const void* k, float* s_out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return scores_common(prob, params, q_window, k, s_out, workspace, workspace_bytes, stream, 2);
}

extern "C" kvc_status kvc_smooth(const kvc_problem* prob, const kvc_params* params,
                                 const float* s_in, float* s_hat, int32_t* kstar,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  KvcDesc D;
  kvc_status st = make_desc(prob, params, &D);
  if (st != KVC_OK) return st;
  if (!s_in || !s_hat || !kstar) return KVC_ERR_INVALID_ARG;
  if (((uintptr_t)s_in & 7u) || ((uintptr_t)s_hat & 7u)) return KVC_ERR_INVALID_ARG;
  const size_t need = sss_scratch_bytes(D);
  if (need && (!workspace || ((uintptr_t)workspace & 255u))) return KVC_ERR_INVALID_ARG;
  if (workspace_bytes < need) return KVC_ERR_WORKSPACE;
  return hip_status(for_each_length_group(D, 0, D.upseq, [&](const KvcSeqGroup& g) {
    return kvc_launch_sss_select(D, g, 1 | 4, s_in, s_hat, kstar, nullptr, nullptr, nullptr,
                                 need ? workspace : nullptr, (hipStream_t)stream);
  }));
}

extern "C" kvc_status kvc_budget(const kvc_problem* prob, const kvc_params* params,
                                 const float* head_scores, int32_t* budgets,
                                 int64_t* seg_offsets, void* stream) {
  KvcDesc D;
  kvc_status st = make_desc(prob, params, &D);
  if (st != KVC_OK) return st;
  if (!head_scores || !budgets || !seg_offsets) return KVC_ERR_INVALID_ARG;
  return hip_status(kvc_launch_budget(D, head_scores, budgets, seg_offsets, (hipStream_t)stream));
}

extern "C" kvc_status kvc_select(const kvc_problem* prob, const kvc_params* params,
                                 const float* s_hat, const int32_t* budgets,
                                 const int64_t* seg_offsets, int32_t* idx_out, void* stream) {
  KvcDesc D;
  kvc_status st = make_desc(prob, params, &D);
  if (st != KVC_OK) return st;
  if (!s_hat || !budgets || !seg_offsets || !idx_out) return KVC_ERR_INVALID_ARG;
  if ((uintptr_t)s_hat & 7u) return KVC_ERR_INVALID_ARG;
  if (check_inputs() && D.row_base[D.n_seq] > 0) {
    // the flag lives in idx_out, which the selection overwrites
    st = run_check(idx_out, (hipStream_t)stream, [&] {
      return kvc_launch_check_select(D, s_hat, budgets, seg_offsets, idx_out, (hipStream_t)stream);
    });
    if (st != KVC_OK) return st;
  }
  return hip_status(for_each_length_group(D, 0, D.upseq, [&](const KvcSeqGroup& g) {
    return kvc_launch_sss_select(D, g, 2, s_hat, nullptr, nullptr, budgets, seg_offsets, idx_out,
                                 nullptr, (hipStream_t)stream);
  }));
}

extern "C" kvc_status kvc_wnw_fixed_select(const kvc_problem* prob, const kvc_params* params,
                                           int32_t seg_len, const float* s_hat,
                                           const int32_t* budgets, const int64_t* seg_offsets,
                                           int32_t* idx_out, void* stream) {
  KvcDesc D;
  kvc_status st = make_desc(prob, params, &D);
  if (st != KVC_OK) return st;
  if (!s_hat || !budgets || !seg_offsets || !idx_out) return KVC_ERR_INVALID_ARG;
  if (seg_len < 1 || seg_len > 64) return KVC_ERR_INVALID_ARG;
  if ((uintptr_t)s_hat & 3u) return KVC_ERR_INVALID_ARG;
  return hip_status(kvc_launch_wnw_fixed_select(D, seg_len, s_hat, budgets, seg_offsets, idx_out,
                                                (hipStream_t)stream));
}

extern "C" kvc_status kvc_gather(const kvc_problem* prob, const kvc_params* params,
                                 const void* k, const void* v, const int32_t* idx,
                                 const int64_t* seg_offsets, void* k_out, void* v_out,
                                 void* stream) {
  KvcDesc D;
  kvc_status st = make_desc(prob, params, &D);
  if (st != KVC_OK) return st;
  if (!k || !v || !idx || !seg_offsets || !k_out || !v_out) return KVC_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_out) || !aligned16(v_out))
    return KVC_ERR_INVALID_ARG;
  if (check_inputs() && D.row_base[D.n_seq] > 0) {
    // the flag lives in k_out, which the gather overwrites
    st = run_check((int32_t*)k_out, (hipStream_t)stream, [&] {
      return kvc_launch_check_gather(D, idx, seg_offsets, (int32_t*)k_out, (hipStream_t)stream);
    });
    if (st != KVC_OK) return st;
  }
  return hip_status(kvc_launch_gather(D, 0, D.n_units, k, v, idx, seg_offsets, k_out, v_out,
                                      D.row_base[D.n_seq], (hipStream_t)stream));
}
