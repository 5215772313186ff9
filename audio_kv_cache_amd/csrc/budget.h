// budget.h -- head-aware token budget (step 3) of one budget pool: a
// sequence's n_layers x n_kv_heads heads, or the n_kv_heads heads of one of
// its layers.  A device function for one workgroup, used by the budget
// kernel and by the statistics pass of the scores, which runs the pools'
// workgroups beside its tiles.
//
// AudioKV article, section 3.1 (layered cache allocation): every head keeps
// a local window w plus a uniform base share r, and the remaining budget
// B_score is split in proportion to the head's audio score S_{l,h}; the
// section 5.1 config gives min_window 32 and base_ratio 0.5.  Here:
//   kbar = floor(retention * L), r = floor(base_ratio * kbar), fixed = w + r
//   R = n*kbar - n*fixed split as R*S_u/sum(S) (uniform if sum(S) == 0)
// A share may not exceed cap = L - fixed (a head cannot keep more than L
// tokens): shares at or above the cap are fixed there and the remaining pool
// is split again among the other heads.  Integer budgets by largest
// remainder, equal remainders to the lower head index.  kbar >= L keeps all.
//
// The arithmetic is IEEE fp64 in a fixed order (sums ascending in u) with no
// fused multiply-add, so the budgets are bit-identical to any other
// implementation of the same definition.
#pragma once
#include "kvc_internal.h"

// The pool's shared memory, in a buffer the caller gives (16-byte aligned):
// the score kernel that hosts budget workgroups shares one buffer between
// its two roles.
struct KvcBudgetSmem {
  double q[KVC_MAX_UNITS_PER_SEQ];
  float sS[KVC_MAX_UNITS_PER_SEQ];
  int32_t extra[KVC_MAX_UNITS_PER_SEQ];
  int64_t s_wsum[1024 / 64];
  int64_t s_R;
  uint8_t active[KVC_MAX_UNITS_PER_SEQ];
};

// One budget pool, workgroup `pool_wg` of the n_seq x pools grid, on
// BUDGET_THREADS threads (whole waves, at most 1024).
template <int BUDGET_THREADS>
__device__ __forceinline__ void kvc_budget_pool(const KvcDesc& D, const float* __restrict__ S,
                                                int32_t* __restrict__ budgets,
                                                int64_t* __restrict__ offsets, int pool_wg,
                                                KvcBudgetSmem& sm) {
#pragma clang fp contract(off)
  static_assert(BUDGET_THREADS % 64 == 0 && BUDGET_THREADS <= 1024, "whole waves, at most 1024");
  double* q = sm.q;
  float* sS = sm.sS;
  int32_t* extra = sm.extra;
  uint8_t* active = sm.active;
  int64_t& s_R = sm.s_R;
  int64_t* s_wsum = sm.s_wsum;

  // Pool `pool` of sequence `seq`: heads pool*n .. pool*n + n - 1 of the
  // sequence (flattened (layer, head) order, as S is laid out).  Every pool
  // keeps n*min(kbar, L) rows in total, so its first row is known up front.
  const int npools = D.upseq / D.pool_size;
  const int seq = pool_wg / npools;
  const int pool = pool_wg - seq * npools;
  const int n = D.pool_size;
  const int L = D.L[seq];
  const int tid = threadIdx.x;
  const int64_t u0 = (int64_t)seq * D.upseq + (int64_t)pool * n;
  S += (int64_t)pool * n;
  const bool last = seq == D.n_seq - 1 && pool == npools - 1;

  const int64_t kbar = (int64_t)floor(D.retention[seq] * (double)L);
  const int64_t row0 = D.row_base[seq] + (int64_t)pool * n * (kbar < L ? kbar : (int64_t)L);
  if (kbar >= L) {
    for (int u = tid; u < n; u += BUDGET_THREADS) {
      budgets[u0 + u] = L;
      offsets[u0 + u] = row0 + (int64_t)u * L;
    }
    if (last && tid == 0) offsets[u0 + n] = row0 + (int64_t)n * L;
    return;
  }
  const int64_t r = (int64_t)floor(D.base_ratio * (double)kbar);
  const int64_t fixed = (int64_t)D.window + r;
  const int64_t cap = (int64_t)L - fixed;

  for (int u = tid; u < n; u += BUDGET_THREADS) {
    active[u] = 1;
    extra[u] = 0;
    sS[u] = S[u];
  }
  __syncthreads();

  // Water-filling rounds, in wave 0 alone (lanes over the heads), so a
  // round costs no workgroup barrier.  Each round's sum of the active
  // scores is the sequential fp64 sum in ascending head order.  When every
  // partial sum of the scores is exact in fp64 -- all are multiples of the
  // finest grid 2^emin among them, and n * max(S) < 2^(emin + 53) -- that
  // sequential sum equals the exact sum, which the lanes then form in any
  // order (every subset sum is exact too); otherwise lane 0 adds the
  // scores one by one in head order.
  if (tid < 64) {
    const int lane = tid;
    float smax = 0.0f;
    int emin = INT32_MAX;
    for (int u = lane; u < n; u += 64) {
      const float v = sS[u];
      smax = fmaxf(smax, v);
      if (v > 0.0f) {
        const int be = (int)((__float_as_uint(v) >> 23) & 0xFFu);
        emin = min(emin, be == 0 ? -149 : be - 150);   // ulp exponent of v
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      smax = fmaxf(smax, __shfl_xor(smax, o));
      emin = min(emin, __shfl_xor(emin, o));
    }
    const bool exact = emin == INT32_MAX || (double)n * (double)smax < ldexp(1.0, emin + 53);
    int64_t R = (int64_t)n * kbar - (int64_t)n * fixed;
    for (;;) {
      double sumA = 0.0;
      int nA = 0;
      if (exact) {
        for (int u = lane; u < n; u += 64)
          if (active[u]) {
            sumA += (double)sS[u];
            ++nA;
          }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          sumA += __shfl_xor(sumA, o);
          nA += __shfl_xor(nA, o);
        }
      } else {
        if (lane == 0) {
          // 16 loads in flight, then the adds in head order (a clamped
          // index and a select instead of a branch per element)
          for (int u0 = 0; u0 < n; u0 += 16) {
            double x[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int u = min(u0 + j, n - 1);
              const float sv = sS[u];
              const bool a = (u0 + j < n) & (active[u] != 0);
              x[j] = a ? (double)sv : 0.0;
              nA += a;
            }
#pragma unroll
            for (int j = 0; j < 16; ++j) sumA += x[j];
          }
        }
        sumA = __shfl(sumA, 0);
        nA = __shfl(nA, 0);
      }
      const double Rd = (double)R;
      int capped = 0;
      for (int u = lane; u < n; u += 64) {
        if (!active[u]) continue;
        const double qu = sumA > 0.0 ? (Rd * (double)sS[u]) / sumA : Rd / (double)nA;
        q[u] = qu;
        capped += qu >= (double)cap;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) capped += __shfl_xor(capped, o);
      if (capped == 0 || nA == 0) break;
      for (int u = lane; u < n; u += 64)
        if (active[u] && q[u] >= (double)cap) {
          active[u] = 0;
          extra[u] = (int32_t)cap;
        }
      R -= cap * (int64_t)capped;
    }
    if (lane == 0) s_R = R;
  }
  __syncthreads();

  // Largest remainder over the heads still active.
  int64_t my_floor = 0;
  for (int u = tid; u < n; u += BUDGET_THREADS)
    if (active[u]) {
      const double fu = floor(q[u]);
      extra[u] = (int32_t)fu;
      my_floor += (int64_t)fu;
    }
  for (int o = 32; o > 0; o >>= 1) my_floor += __shfl_xor(my_floor, o);
  if ((tid & 63) == 0) s_wsum[tid >> 6] = my_floor;
  __syncthreads();
  int64_t floors = 0;
  for (int w = 0; w < BUDGET_THREADS / 64; ++w) floors += s_wsum[w];
  const int64_t deficit = s_R - floors;  // 0 <= deficit <= active count

  // Fractional parts once (inactive heads get -1, below every real one).
  for (int u = tid; u < n; u += BUDGET_THREADS) q[u] = active[u] ? q[u] - floor(q[u]) : -1.0;
  __syncthreads();
  for (int u = tid; u < n; u += BUDGET_THREADS) {
    if (!active[u]) continue;
    const double ru = q[u];
    int rank = 0;
#pragma unroll 8
    for (int v = 0; v < n; ++v) {
      const double rv = q[v];
      rank += (rv > ru) | ((rv == ru) & (v < u));
    }
    extra[u] += (rank < deficit ? 1 : 0);
  }
  __syncthreads();

  // Budgets and the exclusive prefix of row offsets, in u order.
  const int per = (n + BUDGET_THREADS - 1) / BUDGET_THREADS;
  const int lo = tid * per, hi = min(n, lo + per);
  int64_t part = 0;
  for (int u = lo; u < hi; ++u) part += fixed + extra[u];
  // inclusive scan of per-thread parts: wave scan then across waves
  int64_t incl = part;
  const int lane = tid & 63;
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  __syncthreads();
  if (lane == 63) s_wsum[tid >> 6] = incl;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < (tid >> 6); ++w) before += s_wsum[w];
  int64_t run = row0 + before + incl - part;
  for (int u = lo; u < hi; ++u) {
    const int64_t bu = fixed + extra[u];
    budgets[u0 + u] = (int32_t)bu;
    offsets[u0 + u] = run;
    run += bu;
  }
  if (last && hi == n && lo < hi) offsets[u0 + n] = run;
}
