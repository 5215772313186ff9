// kvc_internal.h -- definitions shared by libkvc's host code and its gfx950
// kernels (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define KVC_MAX_SEQ 64
#define KVC_MAX_UNITS_PER_SEQ 4096
#define KVC_MIN_L 64
#define KVC_MAX_L 65536
#define KVC_MAX_GW 256

// Keys covered by one score workgroup (a "tile"); shorter rows use one tile.
#define KVC_TILE_KEYS 2048
// Threads of the smoothing/selection workgroup (one workgroup per unit).
#define KVC_SSS_THREADS 1024

// Everything a kernel needs to know about the problem, passed by value as a
// kernel argument (about 2.7 KiB, under the 4 KiB argument limit).
struct KvcDesc {
  int32_t n_seq, n_layers, n_heads, gqa, d, nwin, gw, upseq;  // upseq = n_layers*n_heads
  int32_t window, dtype;                                      // dtype: 0 bf16, 1 f32
  int32_t pool_size;                    // heads per budget pool (upseq or n_heads)
  int32_t layer0, q_layers;             // q/k/v hold layers layer0 .. layer0+q_layers-1
  int32_t score_max;                    // 1: max over query heads of head means
  float alpha, rho;
  double base_ratio;
  int64_t ks[3], vs[3];                 // element strides: layer, head, token
  int64_t tok0[KVC_MAX_SEQ + 1];        // sequence i = tokens tok0[i] .. tok0[i+1]-1
  int64_t row_base[KVC_MAX_SEQ + 1];    // first compacted row of sequence i
  int64_t srow_base[KVC_MAX_SEQ + 1];   // first score-row element of sequence i
  double retention[KVC_MAX_SEQ];
  int32_t L[KVC_MAX_SEQ];
  int32_t log2L[KVC_MAX_SEQ];
  int32_t tile_base[KVC_MAX_SEQ + 1];   // first score tile of sequence i
  int32_t n_units;
  int32_t total_tiles;
};

// Element offsets of unit (seq, l, h)'s window queries in q_window and of
// its first K (or V) row: the q/k/v pointers hold layers layer0 onward.
__host__ __device__ inline int64_t kvc_q_offset(const KvcDesc& D, int seq, int l, int h) {
  return (((int64_t)seq * D.q_layers + (l - D.layer0)) * D.n_heads * D.gqa + (int64_t)h * D.gqa) *
         D.nwin * D.d;
}
__host__ __device__ inline int64_t kvc_kv_offset(const int64_t (&st)[3], const KvcDesc& D, int seq,
                                                 int l, int h) {
  return (int64_t)(l - D.layer0) * st[0] + (int64_t)h * st[1] + D.tok0[seq] * st[2];
}

// Score tiles of one unit's L keys: tiles of KVC_TILE_KEYS keys over the
// first L64 = L - L % 64 keys (the last one may be shorter, a multiple of 64),
// then KVC_TAIL_SPLITS tail tiles sharing the last L % 64 keys when there are
// any (at most KVC_TAIL_KEYS each).
#define KVC_TAIL_SPLITS 4
#define KVC_TAIL_KEYS 16
__host__ __device__ inline int kvc_main_tiles(int L) {
  return ((L & ~63) + KVC_TILE_KEYS - 1) / KVC_TILE_KEYS;
}
__host__ __device__ inline int kvc_tiles_per_unit(int L) {
  return kvc_main_tiles(L) + ((L & 63) ? KVC_TAIL_SPLITS : 0);
}

// Kernel launchers (defined next to each kernel).
hipError_t kvc_launch_budget(const KvcDesc& D, const float* S, int32_t* budgets,
                             int64_t* offsets, hipStream_t st);
// Range launches: units [u0, u1) (natural (seq, layer, head) order); the
// score launches take any range, the smoothing/selection launches a range
// within one sequence.
// which: 1 = statistics pass (+ LSE fold), 2 = pooling pass, 3 = both.
// Lane x of each 16-lane row rotated by R within the row (DPP row_ror: a
// VALU operand modifier, no round trip through LDS).
template <int R>
__device__ __forceinline__ float kvc_ror16(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + R, 0xF, 0xF, false));
}
// Max and sum over each 16-lane row of the wave, in every lane of the row
// (the sum's order of additions differs between the row's lanes).
__device__ __forceinline__ float kvc_row16_max(float x) {
  x = fmaxf(x, kvc_ror16<1>(x));
  x = fmaxf(x, kvc_ror16<2>(x));
  x = fmaxf(x, kvc_ror16<4>(x));
  return fmaxf(x, kvc_ror16<8>(x));
}
__device__ __forceinline__ float kvc_row16_sum(float x) {
  x += kvc_ror16<1>(x);
  x += kvc_ror16<2>(x);
  x += kvc_ror16<4>(x);
  return x + kvc_ror16<8>(x);
}

// A 16-byte load that does not keep its line in the caches (each row a
// gather reads is read once).
typedef unsigned int kvc_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 kvc_nt_load16(const void* p) {
  const kvc_u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const kvc_u32x4*>(p));
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// The budget step's arguments, for a statistics pass that runs the budget
// pools' workgroups beside its tiles (kvc_scores_host_budget).
struct KvcBudgetArgs {
  const float* S;
  int32_t* budgets;
  int64_t* offsets;
};
hipError_t kvc_launch_scores(const KvcDesc& D, int u0, int u1, const void* q, const void* k,
                             float* s, float2* partials, float* lse2, hipStream_t st,
                             int which = 3, const KvcBudgetArgs* budget = nullptr);
// Whether kvc_launch_scores over every unit can take the budget step along
// (its statistics kernel then holds the budget's LDS without losing
// occupancy); otherwise the caller launches kvc_launch_budget.
bool kvc_scores_host_budget(const KvcDesc& D);
// Smoothing/selection launch over several sequences of one length: units
// seq[k] * upseq + lo .. seq[k] * upseq + hi - 1 for k < n (workgroup
// b -> k = b / (hi - lo), unit lo + b % (hi - lo) of sequence seq[k]).
struct KvcSeqGroup {
  int32_t n, lo, hi;
  uint8_t seq[KVC_MAX_SEQ];
};
__host__ __device__ inline int kvc_group_unit(const KvcSeqGroup& g, int upseq, int b) {
  const int per = g.hi - g.lo;
  const int k = b / per;
  return (int)g.seq[k] * upseq + g.lo + (b - k * per);
}
// mode bit 0: smooth (else read s_hat from s_in); bit 1: select;
// bit 2: export s_hat and kstar.
// scratch: kvc_sss_scratch_bytes(L, u1 - u0) bytes, needed only when L is not
// a power of two (lengths handled through Bluestein's algorithm).
hipError_t kvc_launch_sss_select(const KvcDesc& D, const KvcSeqGroup& g, int mode,
                                 const float* s_in, float* s_hat_out, int32_t* kstar_out,
                                 const int32_t* budgets, const int64_t* offsets, int32_t* idx_out,
                                 void* scratch, hipStream_t st);
size_t kvc_sss_scratch_bytes(int L, int units);
hipError_t kvc_launch_gather(const KvcDesc& D, int u0, int u1, const void* k, const void* v,
                             const int32_t* idx, const int64_t* offsets, void* k_out, void* v_out,
                             int64_t est_rows, hipStream_t st);

// Segment-wise selection of fixed heads (wnw.hip): every unit, as kvc_select.
hipError_t kvc_launch_wnw_fixed_select(const KvcDesc& D, int seg, const float* s_hat,
                                       const int32_t* budgets, const int64_t* offsets,
                                       int32_t* idx_out, hipStream_t st);

// Optional input checks (check.hip): units [u0, u1) of one call; a bad
// element sets *flag (cleared first by kvc_launch_check_clear).
hipError_t kvc_launch_check(const KvcDesc& D, int u0, int u1, const void* q, const void* k,
                            const void* v, const float* S, int32_t* flag, hipStream_t st);
hipError_t kvc_launch_check_clear(int32_t* flag, hipStream_t st);
// Optional checks of the stage entry points' caller-made inputs.
hipError_t kvc_launch_check_gather(const KvcDesc& D, const int32_t* idx, const int64_t* off,
                                   int32_t* flag, hipStream_t st);
hipError_t kvc_launch_check_select(const KvcDesc& D, const float* s_hat, const int32_t* budgets,
                                   const int64_t* off, int32_t* flag, hipStream_t st);

// Record a HIP error for kvc_last_hip_error() (calling thread).
void kvc_note_hip_error(int e);

// Workspace needed by the score kernels.
size_t kvc_scores_workspace(const KvcDesc& D);
