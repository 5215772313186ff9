// check.hip -- optional input checks of the prefill entry points (enabled by
// the environment variable KVC_CHECK_INPUTS=1): every window query, key and
// value element of the units in a call must be finite, every head score
// finite and >= 0 (kvc_compress*); every kept position inside its row and the
// segments consistent (kvc_gather); budgets, segments and smoothed scores
// usable by the selection (kvc_select).  A violation sets a flag.
#include "kvc_internal.h"

template <class E>
__device__ __forceinline__ bool kvc_piece_bad(uint4 x) {
  if constexpr (sizeof(E) == 2) {
    // bf16: exponent bits all ones -> Inf or NaN
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bad |= ((w[i] & 0x7F80u) == 0x7F80u) | (((w[i] >> 16) & 0x7F80u) == 0x7F80u);
    return bad;
  } else {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) bad |= (w[i] & 0x7F800000u) == 0x7F800000u;
    return bad;
  }
}

// grid: (row blocks of 256, units of the range); block 256.
template <class E>
__global__ __launch_bounds__(256) void kvc_check_kernel(KvcDesc D, int u0, const E* __restrict__ q,
                                                        const E* __restrict__ k,
                                                        const E* __restrict__ v,
                                                        const float* __restrict__ S,
                                                        int32_t* __restrict__ flag) {
  const int u = u0 + (int)blockIdx.y;
  const int seq = u / D.upseq, within = u - seq * D.upseq;
  const int l = within / D.n_heads, h = within - l * D.n_heads;
  const int L = D.L[seq];
  const int pieces = D.d * (int)sizeof(E) / 16;  // per row
  bool bad = false;
  const int r0 = blockIdx.x * 256;
  if (r0 < L) {
    const E* kb = k + kvc_kv_offset(D.ks, D, seq, l, h);
    const E* vb = v + kvc_kv_offset(D.vs, D, seq, l, h);
    const int rows = min(256, L - r0);
    for (int i = threadIdx.x; i < rows * pieces; i += 256) {
      const int r = r0 + i / pieces, p = i % pieces;
      bad |= kvc_piece_bad<E>(reinterpret_cast<const uint4*>(kb + (int64_t)r * D.ks[2])[p]);
      bad |= kvc_piece_bad<E>(reinterpret_cast<const uint4*>(vb + (int64_t)r * D.vs[2])[p]);
    }
  }
  if (blockIdx.x == 0) {
    const uint4* qb = reinterpret_cast<const uint4*>(q + kvc_q_offset(D, seq, l, h));
    const int n = D.gqa * D.nwin * pieces;
    for (int i = threadIdx.x; i < n; i += 256) bad |= kvc_piece_bad<E>(qb[i]);
    if (threadIdx.x == 0) {
      const float s = S[l * D.n_heads + h];
      bad |= !(s >= 0.0f) || s == INFINITY;
    }
  }
  if (bad) atomicOr(flag, 1);
}

// Segments of the stage entry points: offsets[0] = 0, every offset within
// [0, the problem's total rows] (the size of the output buffers), and unit
// u's segment holds between 0 and L rows (gather), or exactly budgets[u]
// rows with min(window, L) <= budgets[u] <= L (select).  A unit whose
// segment passes can be read and written in bounds.
__device__ inline bool kvc_segment_bad(const KvcDesc& D, int u, const int64_t* off,
                                       const int32_t* budgets) {
  const int seq = u / D.upseq;
  const int64_t L = D.L[seq], n = off[u + 1] - off[u], total = D.row_base[D.n_seq];
  bool bad = n < 0 || n > L || (u == 0 && off[0] != 0) || off[u] < 0 || off[u + 1] > total;
  if (budgets) {
    const int64_t b = budgets[u], w = D.window < L ? D.window : L;
    bad |= b != n || b < w || b > L;
  }
  return bad;
}

// grid: one workgroup per unit; the unit's kept positions must lie in [0, L).
__global__ __launch_bounds__(256) void kvc_check_gather_kernel(KvcDesc D,
                                                               const int32_t* __restrict__ idx,
                                                               const int64_t* __restrict__ off,
                                                               int32_t* __restrict__ flag) {
  const int u = blockIdx.x;
  __shared__ int sBad;
  if (threadIdx.x == 0) sBad = kvc_segment_bad(D, u, off, nullptr) ? 1 : 0;
  __syncthreads();
  if (sBad) {
    if (threadIdx.x == 0) atomicOr(flag, 1);
    return;
  }
  const int L = D.L[u / D.upseq];
  bool bad = false;
  for (int64_t t = off[u] + threadIdx.x; t < off[u + 1]; t += 256) bad |= (uint32_t)idx[t] >= (uint32_t)L;
  if (bad) atomicOr(flag, 1);
}

// grid: one workgroup per unit; budgets and segments as above, and the
// unit's smoothed score row finite.
__global__ __launch_bounds__(256) void kvc_check_select_kernel(KvcDesc D,
                                                               const float* __restrict__ s_hat,
                                                               const int32_t* __restrict__ budgets,
                                                               const int64_t* __restrict__ off,
                                                               int32_t* __restrict__ flag) {
  const int u = blockIdx.x, seq = u / D.upseq;
  if (threadIdx.x == 0 && kvc_segment_bad(D, u, off, budgets)) atomicOr(flag, 1);
  const int L = D.L[seq];
  const float* row = s_hat + D.srow_base[seq] + (int64_t)(u - seq * D.upseq) * L;
  bool bad = false;
  for (int j = threadIdx.x; j < L; j += 256) bad |= !(fabsf(row[j]) < INFINITY);
  if (bad) atomicOr(flag, 1);
}

hipError_t kvc_launch_check_gather(const KvcDesc& D, const int32_t* idx, const int64_t* off,
                                   int32_t* flag, hipStream_t st) {
  hipLaunchKernelGGL(kvc_check_gather_kernel, dim3((unsigned)D.n_units), dim3(256), 0, st, D,
                     idx, off, flag);
  return hipGetLastError();
}

hipError_t kvc_launch_check_select(const KvcDesc& D, const float* s_hat, const int32_t* budgets,
                                   const int64_t* off, int32_t* flag, hipStream_t st) {
  hipLaunchKernelGGL(kvc_check_select_kernel, dim3((unsigned)D.n_units), dim3(256), 0, st, D,
                     s_hat, budgets, off, flag);
  return hipGetLastError();
}

__global__ void kvc_check_clear_kernel(int32_t* flag) { flag[threadIdx.x] = 0; }  // one thread

hipError_t kvc_launch_check(const KvcDesc& D, int u0, int u1, const void* q, const void* k,
                            const void* v, const float* S, int32_t* flag, hipStream_t st) {
  if (u1 <= u0) return hipSuccess;
  int lmax = 1;
  for (int i = 0; i < D.n_seq; ++i) lmax = max(lmax, (int)D.L[i]);
  const dim3 grid((unsigned)((lmax + 255) / 256), (unsigned)(u1 - u0));
  if (D.dtype == 0)
    hipLaunchKernelGGL(kvc_check_kernel<uint16_t>, grid, dim3(256), 0, st, D, u0,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, S, flag);
  else
    hipLaunchKernelGGL(kvc_check_kernel<float>, grid, dim3(256), 0, st, D, u0, (const float*)q,
                       (const float*)k, (const float*)v, S, flag);
  return hipGetLastError();
}

hipError_t kvc_launch_check_clear(int32_t* flag, hipStream_t st) {
  hipLaunchKernelGGL(kvc_check_clear_kernel, dim3(1), dim3(1), 0, st, flag);
  return hipGetLastError();
}
