// gather.hip -- compaction of the kept K/V rows (step 5).
//
// K_out[t] = K[idx[t]], V_out[t] = V[idx[t]] for every compacted row t; the
// rows of unit u are seg_offsets[u] .. seg_offsets[u+1]-1 (the VoxZip
// digest writes the same compaction as K_{t+1} = Concat(K[:T], K[I_hist],
// K[-M:])).  Pure data movement: each lane moves 16-byte pieces, a 256-thread
// workgroup moves a contiguous run of output rows, loads are issued for K and
// V together so several 16-byte requests per lane are in flight, and both
// sides bypass the caches' retention (non-temporal loads: each kept row is
// read once; non-temporal stores: the output is not read again here).
#include "kvc_internal.h"

#define GATHER_THREADS 256
#define GATHER_LDS_UNITS 1024

template <int ROWB>
__global__ __launch_bounds__(GATHER_THREADS) void kvc_gather_kernel(
    KvcDesc D, int u0, int u1, const char* __restrict__ k, const char* __restrict__ v,
    const int32_t* __restrict__ idx, const int64_t* __restrict__ offsets,
    char* __restrict__ k_out, char* __restrict__ v_out) {
  constexpr int CH = ROWB / 16;                    // 16-byte chunks per row
  constexpr int ROWS_PER_PASS = GATHER_THREADS / CH;
  constexpr int PASSES = 4;
  constexpr int ROWS_PER_BLOCK = ROWS_PER_PASS * PASSES;
  // Rows of units [u0, u1) are offsets[u0] .. offsets[u1]-1; the grid
  // strides over them.
  // With at most GATHER_LDS_UNITS units the offsets are staged in LDS once
  // (one round of loads), so finding a row's unit costs no global latency.
  __shared__ int64_t soff[GATHER_LDS_UNITS + 1];
  const int nu = u1 - u0;
  const bool staged = nu <= GATHER_LDS_UNITS;
  if (staged) {
    for (int i = threadIdx.x; i <= nu; i += GATHER_THREADS) soff[i] = offsets[u0 + i];
    __syncthreads();
  }
  auto off = [&](int uu) { return staged ? soff[uu - u0] : offsets[uu]; };
  const int64_t rbeg = off(u0), rend = off(u1);
  const int esz = D.dtype == 0 ? 2 : 4;
  const int chunk = threadIdx.x % CH;
  for (int64_t r0 = rbeg + (int64_t)blockIdx.x * ROWS_PER_BLOCK; r0 < rend;
       r0 += (int64_t)gridDim.x * ROWS_PER_BLOCK) {
    // Unit owning this thread's first row: largest u with offsets[u] <= row.
    const int64_t t0 = r0 + threadIdx.x / CH;
    int lo = u0, hi = u1 - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off(mid) <= t0) lo = mid; else hi = mid - 1;
    }
    int u = lo;
    uint4 kv[PASSES], vv[PASSES];
    int64_t rows[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int64_t t = r0 + p * ROWS_PER_PASS + threadIdx.x / CH;
      rows[p] = t;
      if (t >= rend) continue;
      while (u + 1 < u1 && off(u + 1) <= t) ++u;
      const int seq = u / D.upseq;
      const int within = u - seq * D.upseq;
      const int l = within / D.n_heads, h = within - l * D.n_heads;
      int pos = idx[t];
      if ((unsigned)pos >= (unsigned)D.L[seq]) pos = 0;  // never read outside the row
      const char* ks = k + (kvc_kv_offset(D.ks, D, seq, l, h) + (int64_t)pos * D.ks[2]) * esz;
      const char* vs = v + (kvc_kv_offset(D.vs, D, seq, l, h) + (int64_t)pos * D.vs[2]) * esz;
      kv[p] = kvc_nt_load16(ks + chunk * 16);
      vv[p] = kvc_nt_load16(vs + chunk * 16);
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int64_t t = rows[p];
      if (t >= rend) continue;
      uint4* ko = reinterpret_cast<uint4*>(k_out + t * ROWB + chunk * 16);
      uint4* vo = reinterpret_cast<uint4*>(v_out + t * ROWB + chunk * 16);
      __builtin_nontemporal_store(kv[p].x, &ko->x);
      __builtin_nontemporal_store(kv[p].y, &ko->y);
      __builtin_nontemporal_store(kv[p].z, &ko->z);
      __builtin_nontemporal_store(kv[p].w, &ko->w);
      __builtin_nontemporal_store(vv[p].x, &vo->x);
      __builtin_nontemporal_store(vv[p].y, &vo->y);
      __builtin_nontemporal_store(vv[p].z, &vo->z);
      __builtin_nontemporal_store(vv[p].w, &vo->w);
    }
  }
}

// Units [u0, u1); est_rows sizes the grid (the kernel strides over any excess).
hipError_t kvc_launch_gather(const KvcDesc& D, int u0, int u1, const void* k, const void* v,
                             const int32_t* idx, const int64_t* offsets, void* k_out, void* v_out,
                             int64_t est_rows, hipStream_t st) {
  if (u1 <= u0) return hipSuccess;
  const int rowb = D.d * (D.dtype == 0 ? 2 : 4);
  auto go = [&](auto kern, int rows_per_block) {
    int64_t blocks = (est_rows + rows_per_block - 1) / rows_per_block;
    if (blocks < 1) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(GATHER_THREADS), 0, st, D, u0, u1,
                       (const char*)k, (const char*)v, idx, offsets, (char*)k_out, (char*)v_out);
  };
  switch (rowb) {
    case 128: go(kvc_gather_kernel<128>, GATHER_THREADS / 8 * 4); break;
    case 256: go(kvc_gather_kernel<256>, GATHER_THREADS / 16 * 4); break;
    case 512: go(kvc_gather_kernel<512>, GATHER_THREADS / 32 * 4); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
