// budget.hip -- head-aware token budget (step 3), one workgroup per budget
// pool: a sequence's n_layers x n_kv_heads heads, or the n_kv_heads heads of
// one of its layers.
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
#include "kvc_internal.h"

#pragma clang fp contract(off)

#define BUDGET_THREADS 1024

__global__ __launch_bounds__(BUDGET_THREADS) void kvc_budget_kernel(
    KvcDesc D, const float* __restrict__ S, int32_t* __restrict__ budgets,
    int64_t* __restrict__ offsets) {
  __shared__ double q[KVC_MAX_UNITS_PER_SEQ];
  __shared__ float sS[KVC_MAX_UNITS_PER_SEQ];
  __shared__ int32_t extra[KVC_MAX_UNITS_PER_SEQ];
  __shared__ uint8_t active[KVC_MAX_UNITS_PER_SEQ];
  __shared__ double s_sum;
  __shared__ int64_t s_R;
  __shared__ int s_nA, s_capped;
  __shared__ int64_t s_wsum[BUDGET_THREADS / 64];

  // Pool `pool` of sequence `seq`: heads pool*n .. pool*n + n - 1 of the
  // sequence (flattened (layer, head) order, as S is laid out).  Every pool
  // keeps n*min(kbar, L) rows in total, so its first row is known up front.
  const int npools = D.upseq / D.pool_size;
  const int seq = blockIdx.x / npools;
  const int pool = blockIdx.x - seq * npools;
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
  if (tid == 0) s_R = (int64_t)n * kbar - (int64_t)n * fixed;
  __syncthreads();

  // Water-filling rounds.
  for (;;) {
    if (tid == 0) {
      // Sequential in u (the order fixes the rounding); branch-free so the
      // LDS loads pipeline: adding +0.0 for an inactive head changes nothing.
      double acc = 0.0;
      int nA = 0;
      for (int u0 = 0; u0 < n; u0 += 16) {
        // 16 independent LDS loads first, then the adds in u order.
        // (loads at a clamped index, then a select: no branch per element,
        // so the 32 LDS loads are all in flight before the first add)
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
        for (int j = 0; j < 16; ++j) acc += x[j];
      }
      s_sum = acc;
      s_nA = nA;
      s_capped = 0;
    }
    __syncthreads();
    const double sumA = s_sum;
    const int nA = s_nA;
    const double Rd = (double)s_R;
    int my_capped = 0;
    for (int u = tid; u < n; u += BUDGET_THREADS) {
      if (!active[u]) continue;
      const double qu = sumA > 0.0 ? (Rd * (double)sS[u]) / sumA : Rd / (double)nA;
      q[u] = qu;
      if (qu >= (double)cap) ++my_capped;
    }
    if (my_capped) atomicAdd(&s_capped, my_capped);
    __syncthreads();
    const int capped = s_capped;
    if (capped == 0 || nA == 0) break;
    for (int u = tid; u < n; u += BUDGET_THREADS)
      if (active[u] && q[u] >= (double)cap) {
        active[u] = 0;
        extra[u] = (int32_t)cap;
      }
    __syncthreads();
    if (tid == 0) s_R -= cap * (int64_t)capped;
    __syncthreads();
  }

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

hipError_t kvc_launch_budget(const KvcDesc& D, const float* S, int32_t* budgets,
                             int64_t* offsets, hipStream_t st) {
  hipLaunchKernelGGL(kvc_budget_kernel, dim3(D.n_seq * (D.upseq / D.pool_size)),
                     dim3(BUDGET_THREADS), 0, st, D, S, budgets, offsets);
  return hipGetLastError();
}
