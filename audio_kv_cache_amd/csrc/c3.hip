// c3.hip -- C3 query-guided retrieval of audio KV (kvc_c3.h).
//
// C3 digest page ("C3: Speech-Guided KV Retrieval for Long-Context
// SpeechLLM Inference"): at prefill every (layer, KV head) cache gets a
// binary tree of key clusters from recursive bisecting 2-means (8 Lloyd
// iterations per split, seed 0); a decode step scores the active frontier of
// the tree by the best cosine over the group's query heads, fills the budget
// with the members of the best nodes, and moves resolution with an EMA of
// the scores and paired split/merge exchanges.
//
// Build, level synchronous over every cache at once (one tree depth per
// round; the host waits once per depth for two counts):
//   local   nodes of 5..96 keys, each owned by the 128-position chunk that
//           holds its first member: the workgroup stages the members' keys
//           in LDS once and runs all 8 Lloyd iterations there -- a thread
//           per key for the fp32 hyperplane test, a wave per node for the
//           exact fp64 member sums (64 lanes over the columns, keys in
//           order) -- then partitions the node's perm range in place.
//   span    nodes over 96 keys: per iteration one launch over 128-key
//           blocks of every such node (hyperplane test, exact block sums
//           added with fp64 atomics, exact in any order) and one launch per
//           node for the new means; then a stable partition per node.
//   ids     one workgroup per cache: breadth-first ids of the new children
//           (a scan over the depth's nodes), their records and centroids,
//           and the next depth's local heads and span list.
// Every sum that feeds a split is exact (keys on the 2^-24 grid, |k| < 4096,
// n <= 2^17: partial sums stay multiples of 2^-24 below 2^29), so the
// reduction order on the GPU cannot change a decision; the fp32 hyperplane
// test uses a fixed column order and exact products.
//
// Step: score (workgroups over the frontier entries, thread per entry),
// select + update (one 1024-lane workgroup per cache: weighted radix select
// of the best nodes, a position bitmap in LDS listed ascending, then the EMA
// and R masked max/min reductions for the exchanges), gather.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "../../include/kvc_c3.h"
#include "kvc_internal.h"

// Separate roundings wherever the code writes a product and a sum; the one
// fused multiply-add used (the hyperplane test) is written out and exact.
#pragma clang fp contract(off)

#define C3_MAX_SEQ 64
#define C3_MAX_CAP 131072
#define C3_MAX_G 32
#define C3_LEAF 4
#define C3_ITERS 8
#define C3_MAXD 24
#define C3_CH 128                          // positions per local chunk
#define C3_MLOC 96                         // largest node split in one workgroup
#define C3_ROWS (C3_CH + C3_MLOC - 1)      // keys a local workgroup can hold
#define C3_HEADS (C3_CH / (C3_LEAF + 1) + 1)
#define C3_T 256
#define C3_BIG 1024
#define C3_SW 8                            // score workgroups per cache

struct C3Desc {
  int32_t n_seq, upseq, gqa, d, n_units, R;
  int32_t cap, ncap, nchunk, kept_cap;
  double lam;
  uint64_t seed;
  int64_t ks[2], vs[2], os[2];
  int32_t len[C3_MAX_SEQ], budget[C3_MAX_SEQ];
};

struct C3Index {
  int32_t *start, *size, *left, *parent, *depth, *perm, *nn;
  uint16_t* cent;
};

struct C3State {
  int32_t* count;
  int32_t* fr;
  double* e;
};

struct C3Work {
  uint16_t* cres;    // [U][cap][d]: child centroids, at each child's start
  int32_t* res_n0;   // [U][cap]: split result at each node's start (n0, or -1)
  uint8_t* flags;    // [U][cap]: cluster of each position (span nodes)
  int32_t* head;     // [U][cap]: local node starting here at this depth, or -1
  int32_t* ptmp;     // [U][cap]
  int32_t* lvl;      // [U][C3_MAXD + 2]: first id of each depth
  double* rsum;      // [U][d]
  int32_t* tiny;     // [U]: 1 if a nonzero key value of the cache lies below 2^-17
  int2* snode;       // [2][smax]: (cache, node) of each span slot
  float* sw;         // [smax][d]
  float* sb;         // [smax]
  double* s0;        // [smax][d]
  double* s1;        // [smax][d]
  int32_t* sn1;      // [smax]
  int32_t* salive;   // [smax]: 1 iterating, 2 converged (split found), 0 abandoned
  int32_t* sflip;    // [smax]: rows that changed cluster in the current iteration
  int32_t* cnt;      // [C3_MAXD + 1][4]: candidates, span nodes, largest span
                     // node, chunks holding local nodes
  int32_t* cflag;    // [U * nchunk]: chunk already listed for the next depth
  int32_t* clist;    // [2][U * nchunk]: chunks holding local nodes, per depth parity
  int32_t* err;      // [1]
  int32_t smax;
};

// ---------------------------------------------------------------------------
// Arithmetic of the split decisions
// ---------------------------------------------------------------------------
__device__ inline float c3_bf(uint32_t h) { return __uint_as_float(h << 16); }

__device__ inline uint16_t c3_to_bf16(double x) {
  const uint32_t b = __float_as_uint((float)x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// Snap a bf16 key to the grid 2^-24 (only |k| < 2^-17 moves) and flag keys
// outside the supported range (|k| >= 4096, inf, nan).
__device__ inline uint32_t c3_snap(uint32_t h, int& bad) {
  const uint32_t e = (h >> 7) & 0xFFu;
  if (e >= 127u + 12u) {
    bad = 1;
    return h;
  }
  if (e >= 110u) return h;
  const float y = rintf(__uint_as_float(h << 16) * 0x1p24f) * 0x1p-24f;
  return __float_as_uint(y) >> 16;
}

__device__ inline uint4 c3_snap8(uint4 v, int& bad) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = c3_snap(w[i] & 0xFFFFu, bad) | (c3_snap(w[i] >> 16, bad) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

typedef unsigned short c3_u16x2 __attribute__((ext_vector_type(2)));

// c3_snap8 for keys already range-checked: the 8 values only change when
// one of them is a nonzero below 2^-17 (|bits| - 1 < 0x36FF), which a packed
// 16-bit test finds for all 8 at once.
__device__ inline uint4 c3_snap8_fast(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  c3_u16x2 lo = {0xFFFFu, 0xFFFFu};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c3_u16x2 a = __builtin_bit_cast(c3_u16x2, w[i] & 0x7FFF7FFFu);
    a = a - (c3_u16x2){1u, 1u};
    lo = __builtin_elementwise_min(lo, a);
  }
  if (lo.x >= 0x36FFu && lo.y >= 0x36FFu) return v;
  int ignored = 0;
  return c3_snap8(v, ignored);
}

// x / n, correctly rounded, from y = 1/n correctly rounded: q = x y is
// within an ulp of x/n, the remainder x - n q is exact in one fused
// multiply-add, and one correction q + r y rounded once gives the correctly
// rounded quotient (Markstein's theorem on division by Newton correction,
// for round-to-nearest without underflow or overflow; here x is a multiple
// of 2^-24 below 2^29 in magnitude and n a count below 2^18).  Three
// operations per column instead of a full division.
__device__ inline double c3_div(double x, double n, double y) {
  const double q = x * y;
  const double r = fma(-q, n, x);
  return fma(r, y, q);
}

__device__ inline float c3_round16(float x) {
  const uint32_t b = __float_as_uint(x);
  return __uint_as_float((b + 0x7Fu + ((b >> 8) & 1u)) & 0xFFFFFF00u);
}

// Hyperplane between two fp64 means for the CPL columns of this lane (lane l
// owns columns CPL*l ..); returns b on every lane.  b is the fp32 sum of the
// rounded products in column order: each lane reads every lane's products
// in turn and adds them one at a time (all 64 lanes active).
template <int CPL>
__device__ inline float c3_bisect(const double* mu0, const double* mu1, float* w) {
  float p[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    float wf = c3_round16((float)(mu1[i] - mu0[i]));
    if (fabsf(wf) < 0x1p-100f) wf = 0.0f;
    const float mf = (float)(0.5 * (mu0[i] + mu1[i]));
    w[i] = wf;
    p[i] = wf * mf;
  }
  float s = 0.0f;
  for (int l = 0; l < 64; ++l)
#pragma unroll
    for (int i = 0; i < CPL; ++i) s = s + __shfl(p[i], l);
  return s;
}

// The CPL column values of this lane in a key row staged in LDS.
template <int CPL>
__device__ inline void c3_row_vals(const unsigned char* row, int lane, double* v) {
  if constexpr (CPL == 2) {
    const uint32_t h = *reinterpret_cast<const uint32_t*>(row + lane * 4);
    v[0] = (double)c3_bf(h & 0xFFFFu);
    v[CPL - 1] = (double)c3_bf(h >> 16);
  } else {
    const uint32_t h = *reinterpret_cast<const uint16_t*>(row + lane * 2);
    v[0] = (double)c3_bf(h);
  }
}

// s(k) = sum_c k_c w_c in fp32, column order; every product is exact.
template <int D>
__device__ inline float c3_plane(const unsigned char* row, const float* w) {
  const uint4* kr = reinterpret_cast<const uint4*>(row);
  const float4* wr = reinterpret_cast<const float4*>(w);
  float s = 0.0f;
#pragma unroll
  for (int c8 = 0; c8 < D / 8; ++c8) {
    const uint4 kk = kr[c8];
    const float4 w0 = wr[2 * c8], w1 = wr[2 * c8 + 1];
    s = fmaf(c3_bf(kk.x & 0xFFFFu), w0.x, s);
    s = fmaf(c3_bf(kk.x >> 16), w0.y, s);
    s = fmaf(c3_bf(kk.y & 0xFFFFu), w0.z, s);
    s = fmaf(c3_bf(kk.y >> 16), w0.w, s);
    s = fmaf(c3_bf(kk.z & 0xFFFFu), w1.x, s);
    s = fmaf(c3_bf(kk.z >> 16), w1.y, s);
    s = fmaf(c3_bf(kk.w & 0xFFFFu), w1.z, s);
    s = fmaf(c3_bf(kk.w >> 16), w1.w, s);
  }
  return s;
}

// Stage key rows into LDS (padded rows of RB bytes), snapped to the grid:
// row r < rows with valid[r] >= 0 comes from key src[r] of cache u.  Every
// load of a thread is issued before its first LDS store.  (The key range
// was checked when the root sums were taken.)
template <int D, int MAXR>
__device__ inline void c3_stage(const C3Desc& P, int u, const uint16_t* __restrict__ k,
                                const int* src, const signed char* valid, int rows,
                                unsigned char* sK, bool tiny) {
  constexpr int RB = 2 * D + 16, PPR = D / 8, PER = (MAXR * PPR + C3_T - 1) / C3_T;
  uint4 buf[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int i = threadIdx.x + p * C3_T;
    const int r = i / PPR, pc = i - r * PPR;
    if (r < rows && (valid == nullptr || valid[r] >= 0))
      buf[p] = kvc_nt_load16(k + u * P.ks[0] + (int64_t)src[r] * P.ks[1] + pc * 8);
  }
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int i = threadIdx.x + p * C3_T;
    const int r = i / PPR, pc = i - r * PPR;
    if (r < rows && (valid == nullptr || valid[r] >= 0))
      *reinterpret_cast<uint4*>(sK + r * RB + pc * 16) = tiny ? c3_snap8_fast(buf[p]) : buf[p];
  }
}

__device__ inline uint64_t c3_mix(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Two distinct members (indices into the node's range) for the initial means.
__device__ inline void c3_init_pair(uint64_t seed, int u, int dep, int start, int size, int* a0,
                                    int* a1) {
  const uint64_t h0 = c3_mix(seed ^ ((uint64_t)u << 40) ^ ((uint64_t)dep << 32) ^ (uint64_t)start);
  const uint64_t h1 = c3_mix(h0);
  const uint64_t x0 = h0 % (uint64_t)size;
  *a0 = (int)x0;
  *a1 = (int)((x0 + 1 + h1 % (uint64_t)(size - 1)) % (uint64_t)size);
}

__device__ inline int c3_n(const C3Desc& P, int u) { return P.len[u / P.upseq]; }
__device__ inline int c3_b(const C3Desc& P, int u) { return P.budget[u / P.upseq]; }

// Exclusive prefix sum of v over the workgroup in thread order, and the
// total.  `scratch` holds one value per wave.  Two barriers.
template <int NT>
__device__ inline int c3_block_scan(int v, int* scratch, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int c = scratch[w];
    off += w < wave ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}

// List chunk g (cache u's chunk of position p) for the local kernel of the
// next depth, once.
__device__ inline void c3_list_chunk(const C3Desc& P, const C3Work& W, int u, int p, int dep1) {
  const int g = u * P.nchunk + p / C3_CH;
  if (atomicExch(&W.cflag[g], 1) == 0) {
    const int i = atomicAdd(&W.cnt[dep1 * 4 + 3], 1);
    W.clist[(dep1 & 1) * P.n_units * P.nchunk + i] = g;
  }
}

// ---------------------------------------------------------------------------
// Build: roots
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(C3_T) void c3_init_kernel(C3Desc P, C3Index X, C3Work W) {
  const int u = blockIdx.x, n = c3_n(P, u);
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  for (int p = threadIdx.x; p < n; p += C3_T) {
    X.perm[ub + p] = p;
    W.head[ub + p] = -1;
  }
  for (int c = threadIdx.x; c < P.nchunk; c += C3_T) W.cflag[(size_t)u * P.nchunk + c] = 0;
  for (int c = threadIdx.x; c < P.d; c += C3_T) W.rsum[(size_t)u * P.d + c] = 0.0;
  if (threadIdx.x == 0) {
    W.tiny[u] = 0;
    X.nn[u] = n > 0 ? 1 : 0;
    int32_t* lv = W.lvl + (size_t)u * (C3_MAXD + 2);
    lv[0] = 0;
    lv[1] = n > 0 ? 1 : 0;
    if (n > 0) {
      X.start[nb] = 0;
      X.size[nb] = n;
      X.left[nb] = -1;
      X.parent[nb] = -1;
      X.depth[nb] = 0;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && n > C3_LEAF) {
    if (n <= C3_MLOC) {
      W.head[ub] = 0;
      c3_list_chunk(P, W, u, 0, 0);
    } else {
      const int s = atomicAdd(&W.cnt[1], 1);
      W.snode[s] = make_int2(u, 0);
    }
  }
}

// Exact fp64 column sums of every cache's keys (the root's mean).  Thread t
// owns 16-byte piece t % (D/8) of rows t / (D/8) + k * RG of its chunk.
template <int D>
__global__ __launch_bounds__(C3_T) void c3_root_sum_kernel(C3Desc P, C3Work W,
                                                           const uint16_t* __restrict__ k) {
  constexpr int PPR = D / 8, RG = C3_T / PPR, PER = C3_CH / RG;
  const int u = blockIdx.x / P.nchunk, chn = blockIdx.x - u * P.nchunk;
  const int n = c3_n(P, u), base = chn * C3_CH;
  if (base >= n) return;
  const int rows = min(C3_CH, n - base);
  const int pc = threadIdx.x % PPR, rg = threadIdx.x / PPR;
  uint4 buf[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int r = rg + p * RG;
    if (r < rows)
      buf[p] = kvc_nt_load16(k + u * P.ks[0] + (int64_t)(base + r) * P.ks[1] + pc * 8);
  }
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  int bad = 0, tiny = 0;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    if (rg + p * RG >= rows) continue;
    const uint4 v = c3_snap8(buf[p], bad);
    tiny |= (v.x != buf[p].x) | (v.y != buf[p].y) | (v.z != buf[p].z) | (v.w != buf[p].w);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += (double)c3_bf(w[j] & 0xFFFFu);
      acc[2 * j + 1] += (double)c3_bf(w[j] >> 16);
    }
  }
  __shared__ double red[RG][D];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rg][pc * 8 + j] = acc[j];
  if (bad) atomicOr(W.err, 1);
  if (tiny) atomicOr(&W.tiny[u], 1);
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += C3_T) {
    double t = 0.0;
    for (int g = 0; g < RG; ++g) t += red[g][c];
    atomicAdd(&W.rsum[(size_t)u * D + c], t);
  }
}

__global__ __launch_bounds__(C3_T) void c3_root_fin_kernel(C3Desc P, C3Index X, C3Work W) {
  const int u = blockIdx.x, n = c3_n(P, u);
  if (n == 0) return;
  for (int c = threadIdx.x; c < P.d; c += C3_T)
    X.cent[(size_t)u * P.ncap * P.d + c] = c3_to_bf16(W.rsum[(size_t)u * P.d + c] / (double)n);
}

// ---------------------------------------------------------------------------
// Build: nodes of 5..96 keys, all 8 iterations in one workgroup
// ---------------------------------------------------------------------------
// Bits [r0, r0 + m) (m <= 96) of a 256-bit row mask held in 4 words: the
// first 64 in lo, the rest in hi.
__device__ inline void c3_take_bits(const uint64_t* wd, int r0, int m, uint64_t& lo,
                                    uint64_t& hi) {
  auto at = [&](int pos) -> uint64_t {
    const int w = pos >> 6, sh = pos & 63;
    const uint64_t a = w < 4 ? wd[w] : 0ull;
    const uint64_t b = w + 1 < 4 ? wd[w + 1] : 0ull;
    return sh ? (a >> sh) | (b << (64 - sh)) : a;
  };
  lo = at(r0);
  hi = at(r0 + 64);
  if (m < 64) {
    lo &= (1ull << m) - 1ull;
    hi = 0ull;
  } else {
    hi &= (1ull << (m - 64)) - 1ull;
  }
}

// a[0..7] += (or -=) the 8 columns at piece gl of every row r0 + bit of
// (lo, hi); four rows' loads in flight at a time.  The values are on the
// 2^-24 grid, so the sums are exact in any order.
template <int RB, bool SUB>
__device__ inline void c3_acc_rows(const unsigned char* sK, int r0, uint64_t lo, uint64_t hi,
                                   int gl, double (&a)[8]) {
  while (lo | hi) {
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (lo) {
        rr[q] = r0 + __builtin_ctzll(lo);
        lo &= lo - 1ull;
      } else if (hi) {
        rr[q] = r0 + 64 + __builtin_ctzll(hi);
        hi &= hi - 1ull;
      } else {
        rr[q] = -1;
      }
    }
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (rr[q] >= 0) v[q] = *reinterpret_cast<const uint4*>(sK + rr[q] * RB + gl * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (rr[q] < 0) continue;
      const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const double x0 = (double)c3_bf(w[i] & 0xFFFFu), x1 = (double)c3_bf(w[i] >> 16);
        if (SUB) {
          a[2 * i] -= x0;
          a[2 * i + 1] -= x1;
        } else {
          a[2 * i] += x0;
          a[2 * i + 1] += x1;
        }
      }
    }
  }
}

// Hyperplane between two fp64 means for the 8 columns of piece gl (columns
// 8 gl .. 8 gl + 7); the lanes of one node are LPN consecutive lanes of one
// wave, all active together.  The normal w goes to the node's LDS row (row
// [8 gl .. 8 gl + 7]) and b, the fp32 sum of the rounded products in column
// order, is returned on every lane of the node: the products pass through
// the same row (two stores per lane, then every lane reads the whole row,
// the reads of one node broadcast) and each lane adds them one at a time.
// Only the node's lanes touch the row here, and one wave's LDS operations
// are done in order, so no barrier is needed.
template <int LPN>
__device__ inline float c3_bisect8(const double (&mu0)[8], const double (&mu1)[8], float* row,
                                   int gl) {
  float w[8], p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float wf = c3_round16((float)(mu1[i] - mu0[i]));
    if (fabsf(wf) < 0x1p-100f) wf = 0.0f;
    const float mf = (float)(0.5 * (mu0[i] + mu1[i]));
    w[i] = wf;
    p[i] = wf * mf;
  }
  float4* r4 = reinterpret_cast<float4*>(row);
  r4[2 * gl] = make_float4(p[0], p[1], p[2], p[3]);
  r4[2 * gl + 1] = make_float4(p[4], p[5], p[6], p[7]);
  float s = 0.0f;
#pragma unroll
  for (int c4 = 0; c4 < 2 * LPN; ++c4) {
    const float4 v = r4[c4];
    s = s + v.x;
    s = s + v.y;
    s = s + v.z;
    s = s + v.w;
  }
  r4[2 * gl] = make_float4(w[0], w[1], w[2], w[3]);
  r4[2 * gl + 1] = make_float4(w[4], w[5], w[6], w[7]);
  return s;
}

template <int D>
__global__ __launch_bounds__(C3_T) void c3_local_kernel(C3Desc P, int dep, C3Index X, C3Work W,
                                                        const uint16_t* __restrict__ k) {
  constexpr int RB = 2 * D + 16;          // padded LDS row: conflict-free row-per-lane reads
  constexpr int LPN = D / 8;              // lanes per node in the member-sum phase
  constexpr int GPW = 64 / LPN;           // nodes per wave at a time
  constexpr int NW = C3_T / 64;
  constexpr int NPR = GPW * NW;           // nodes per round
  constexpr int ROUNDS = (C3_HEADS + NPR - 1) / NPR;
  __shared__ __align__(16) unsigned char sK[C3_ROWS * RB];
  __shared__ __align__(16) float sW[C3_HEADS][D + 4];
  __shared__ float sB[C3_HEADS];
  __shared__ int sStart[C3_HEADS], sSize[C3_HEADS], sNode[C3_HEADS], sA0[C3_HEADS],
      sA1[C3_HEADS], sDead[C3_HEADS], sN0[C3_HEADS];
  __shared__ int sPerm[C3_ROWS];
  __shared__ signed char sRowNode[C3_ROWS];
  __shared__ uint64_t sBits[NW], sOld[NW];   // cluster-1 flag of every row, new and previous
  __shared__ int sConv[C3_HEADS];             // 1 once the partition stopped changing
  __shared__ int sNh, sLeft[2];

  const int g = W.clist[(dep & 1) * P.n_units * P.nchunk + blockIdx.x];
  const int u = g / P.nchunk, chn = g - u * P.nchunk;
  const int n = c3_n(P, u), base = chn * C3_CH;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane / LPN, gl = lane % LPN;
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  if (tid == 0) W.cflag[g] = 0;

  // Heads in position order: a ballot per wave of the chunk's positions.
  static_assert(C3_CH == 128, "two waves cover a chunk");
  if (tid < NW) sBits[tid] = 0ull;
  int myhead = -1;
  if (tid < C3_CH) {
    myhead = (base + tid < n) ? W.head[ub + base + tid] : -1;
    const uint64_t hb = __ballot(myhead >= 0);
    if (lane == 0) sOld[wave] = hb;
  }
  __syncthreads();
  if (myhead >= 0) {
    const uint64_t below = lane ? (sOld[wave] & ((1ull << lane) - 1ull)) : 0ull;
    const int rank = (wave ? __popcll(sOld[0]) : 0) + __popcll(below);
    sNode[rank] = myhead;
    sStart[rank] = base + tid;
    sSize[rank] = X.size[nb + myhead];
  }
  if (tid == 0) sNh = __popcll(sOld[0]) + __popcll(sOld[1]);
  __syncthreads();
  const int nh = sNh;
  if (nh == 0) return;
  const int row0 = sStart[0];
  const int rows = sStart[nh - 1] + sSize[nh - 1] - row0;
  if (tid < nh) {
    int a0, a1;
    c3_init_pair(P.seed, u, dep, sStart[tid], sSize[tid], &a0, &a1);
    sA0[tid] = a0;
    sA1[tid] = a1;
    sDead[tid] = 0;
    sConv[tid] = 0;
  }
  for (int r = tid; r < rows; r += C3_T) {
    int j = -1;
    for (int h = 0; h < nh; ++h)
      if (r >= sStart[h] - row0 && r < sStart[h] - row0 + sSize[h]) j = h;
    sRowNode[r] = (signed char)j;
    sPerm[r] = j >= 0 ? X.perm[ub + row0 + r] : 0;
  }
  __syncthreads();
  c3_stage<D, C3_ROWS>(P, u, k, sPerm, sRowNode, rows, sK, W.tiny[u] != 0);
  __syncthreads();

  // A node is owned by gpn groups of LPN lanes (lane gl: columns
  // 8 gl .. 8 gl + 7; group part p: the node's rows r0 + p, r0 + p + gpn,
  // ...), which keep partial totals and cluster-1 sums in registers and
  // combine them with shuffles (exact).  Few nodes get more groups each.
  const int gpn = (nh * 4 <= NPR) ? 4 : ((nh * 2 <= NPR) ? 2 : 1);
  const int part = grp % gpn;
  const uint64_t pat =
      gpn == 1 ? ~0ull : ((gpn == 2 ? 0x5555555555555555ull : 0x1111111111111111ull) << part);
  auto combine = [&](const double (&a)[8], double (&out)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = a[i];
    if (gpn >= 2)
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] += __shfl_xor(out[i], LPN);
    if (gpn >= 4)
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] += __shfl_xor(out[i], 2 * LPN);
  };
  double tot[ROUNDS][8], s1[ROUNDS][8];
#pragma unroll
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int j = (rd * NPR + wave * GPW + grp) / gpn;
    const bool valid = j < nh;
    double pt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pt[i] = s1[rd][i] = 0.0;
    int r0 = 0, m = 0;
    if (valid) {
      r0 = sStart[j] - row0;
      m = sSize[j];
      const uint64_t lo = m >= 64 ? ~0ull : (1ull << m) - 1ull;
      const uint64_t hi = m > 64 ? (1ull << (m - 64)) - 1ull : 0ull;
      c3_acc_rows<RB, false>(sK, r0, lo & pat, hi & pat, gl, pt);
    }
    combine(pt, tot[rd]);
    if (valid && part == 0) {
      double m0[8], m1[8];
      const uint4 v0 = *reinterpret_cast<const uint4*>(sK + (r0 + sA0[j]) * RB + gl * 16);
      const uint4 v1 = *reinterpret_cast<const uint4*>(sK + (r0 + sA1[j]) * RB + gl * 16);
      const uint32_t h0[4] = {v0.x, v0.y, v0.z, v0.w}, h1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m0[2 * i] = (double)c3_bf(h0[i] & 0xFFFFu);
        m0[2 * i + 1] = (double)c3_bf(h0[i] >> 16);
        m1[2 * i] = (double)c3_bf(h1[i] & 0xFFFFu);
        m1[2 * i + 1] = (double)c3_bf(h1[i] >> 16);
      }
      const float b = c3_bisect8<LPN>(m0, m1, &sW[j][0], gl);
      if (gl == 0) sB[j] = b;
    }
  }
  __syncthreads();

  // Iterations stop early for a node whose partition repeats: its means,
  // and so every later partition, are then the same (exact arithmetic).
  for (int it = 0; it < C3_ITERS; ++it) {
    // Hyperplane test, a thread per row; one ballot word per wave.
    {
      const int r = tid;
      const int j = r < rows ? sRowNode[r] : -1;
      const uint64_t prev = sBits[wave];
      bool f;
      if (j >= 0 && sConv[j])
        f = (prev >> lane) & 1ull;
      else
        f = j >= 0 && !sDead[j] && c3_plane<D>(sK + r * RB, &sW[j][0]) > sB[j];
      const uint64_t word = __ballot(f);
      if (lane == 0) {
        sOld[wave] = prev;
        sBits[wave] = word;
      }
      if (tid == 0) sLeft[it & 1] = 0;
    }
    __syncthreads();
    // New means from the rows whose cluster changed (exact running sums).
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
      const int j = (rd * NPR + wave * GPW + grp) / gpn;
      const bool live = j < nh && !sDead[j] && !sConv[j];
      int m = 1, n1 = 0;
      bool same = false;
      if (live) {
        const int r0 = sStart[j] - row0;
        m = sSize[j];
        uint64_t nlo, nhi, olo, ohi;
        c3_take_bits(sBits, r0, m, nlo, nhi);
        c3_take_bits(sOld, r0, m, olo, ohi);
        c3_acc_rows<RB, false>(sK, r0, nlo & ~olo & pat, nhi & ~ohi & pat, gl, s1[rd]);
        c3_acc_rows<RB, true>(sK, r0, olo & ~nlo & pat, ohi & ~nhi & pat, gl, s1[rd]);
        n1 = __popcll(nlo) + __popcll(nhi);
        same = it > 0 && nlo == olo && nhi == ohi;
      }
      double sf[8];
      combine(s1[rd], sf);
      if (!live || part != 0) continue;
      if (n1 == 0 || n1 == m) {
        if (gl == 0) {
          sDead[j] = 1;
          W.res_n0[ub + sStart[j]] = -1;
        }
        continue;
      }
      // exact member sums divided by the counts, correctly rounded (one
      // division per count, then c3_div per column)
      const double n0d = (double)(m - n1), n1d = (double)n1;
      const double y0 = 1.0 / n0d, y1 = 1.0 / n1d;
      double mu0[8], mu1[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mu0[i] = c3_div(tot[rd][i] - sf[i], n0d, y0);
        mu1[i] = c3_div(sf[i], n1d, y1);
      }
      if (same && gl == 0) sConv[j] = 1;
      if (!same && gl == 0) sLeft[it & 1] = 1;
      if (it + 1 < C3_ITERS && !same) {
        const float b = c3_bisect8<LPN>(mu0, mu1, &sW[j][0], gl);
        if (gl == 0) sB[j] = b;
      } else {
        const int n0 = m - n1;
        uint32_t c0[4], c1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c0[i] = (uint32_t)c3_to_bf16(mu0[2 * i]) | ((uint32_t)c3_to_bf16(mu0[2 * i + 1]) << 16);
          c1[i] = (uint32_t)c3_to_bf16(mu1[2 * i]) | ((uint32_t)c3_to_bf16(mu1[2 * i + 1]) << 16);
        }
        *reinterpret_cast<uint4*>(W.cres + (ub + sStart[j]) * D + gl * 8) =
            make_uint4(c0[0], c0[1], c0[2], c0[3]);
        *reinterpret_cast<uint4*>(W.cres + (ub + sStart[j] + n0) * D + gl * 8) =
            make_uint4(c1[0], c1[1], c1[2], c1[3]);
        if (gl == 0) {
          sN0[j] = n0;
          W.res_n0[ub + sStart[j]] = n0;
        }
      }
    }
    __syncthreads();
    if (sLeft[it & 1] == 0) break;
  }

  // Stable partition of each split node's range, in place (this workgroup
  // alone reads and writes the positions of the nodes it owns).
  for (int r = tid; r < rows; r += C3_T) {
    const int j = sRowNode[r];
    if (j < 0 || sDead[j]) continue;
    const int r0 = sStart[j] - row0;
    uint64_t lo, hi;
    c3_take_bits(sBits, r0, r - r0 + 1, lo, hi);   // bits r0 .. r
    const int f = (int)((r - r0 < 64 ? lo >> (r - r0) : hi >> (r - r0 - 64)) & 1ull);
    const int ones = __popcll(lo) + __popcll(hi) - f;   // ones before r
    const int rank = f ? ones : (r - r0) - ones;
    const int np = sStart[j] + (f ? sN0[j] + rank : rank);
    X.perm[ub + np] = sPerm[r];
  }
}

// ---------------------------------------------------------------------------
// Build: nodes over 96 keys, one launch per iteration
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void c3_span_init_kernel(C3Desc P, int dep, int par, C3Index X,
                                                          C3Work W, const uint16_t* __restrict__ k) {
  constexpr int CPL = D / 64;
  const int s = blockIdx.x, lane = threadIdx.x;
  const int2 un = W.snode[par * W.smax + s];
  const int u = un.x, x = un.y;
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  const int st = X.start[nb + x], m = X.size[nb + x];
  int a0, a1;
  c3_init_pair(P.seed, u, dep, st, m, &a0, &a1);
  const uint16_t* r0 = k + u * P.ks[0] + (int64_t)X.perm[ub + st + a0] * P.ks[1];
  const uint16_t* r1 = k + u * P.ks[0] + (int64_t)X.perm[ub + st + a1] * P.ks[1];
  double m0[CPL], m1[CPL];
  float w[CPL];
  int bad = 0;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    m0[i] = (double)c3_bf(c3_snap(r0[lane * CPL + i], bad));
    m1[i] = (double)c3_bf(c3_snap(r1[lane * CPL + i], bad));
  }
  const float b = c3_bisect<CPL>(m0, m1, w);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    W.sw[(size_t)s * D + lane * CPL + i] = w[i];
    W.s0[(size_t)s * D + lane * CPL + i] = 0.0;
    W.s1[(size_t)s * D + lane * CPL + i] = 0.0;
  }
  if (lane == 0) {
    W.sb[s] = b;
    W.sn1[s] = 0;
    W.sflip[s] = 0;
    W.salive[s] = 1;
  }
}

// Column sums of rows base + bit of a uniform 32-bit mask, lanes over the
// columns (CPL each); four rows' loads in flight at a time.  Exact.
template <int RB, int CPL, bool SUB>
__device__ inline void c3_acc_cols(const unsigned char* sK, int base, uint32_t mask, int lane,
                                   double (&a)[CPL]) {
  while (mask) {
    int rr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rr[q] = mask ? base + __builtin_ctz(mask) : -1;
      mask &= mask ? mask - 1u : 0u;
    }
    double v[4][CPL];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (rr[q] >= 0) c3_row_vals<CPL>(sK + rr[q] * RB, lane, v[q]);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (rr[q] >= 0)
#pragma unroll
        for (int i = 0; i < CPL; ++i) a[i] = SUB ? a[i] - v[q][i] : a[i] + v[q][i];
  }
}

// C3_SPB consecutive 128-key blocks of one span node per workgroup: the
// next two blocks' keys are loaded into registers (two buffers) while the
// current one is tested (one block in flight streamed the keys at 4.4 TB/s,
// two at 5.1 at depth 0).  Iteration 0 adds every row to the node's total
// and the rows of cluster 1 to its cluster-1 sum; later iterations add and
// subtract only the rows that changed cluster (the previous cluster of each
// position is kept in the flags array).  One set of atomics per workgroup.
#define C3_SPB 4
template <int D>
__global__ __launch_bounds__(C3_T) void c3_span_iter_kernel(C3Desc P, int par, int it, C3Index X,
                                                            C3Work W, const uint16_t* __restrict__ k) {
  constexpr int RB = 2 * D + 16, CPL = D / 64, PPR = D / 8, NW = C3_T / 64;
  constexpr int PER = C3_CH * PPR / C3_T;       // 16-byte pieces per thread and block
  static_assert(2 * NW * D * 8 <= C3_CH * RB, "the block reduction fits in the key tile");
  __shared__ __align__(16) unsigned char sK[C3_CH * RB];
  __shared__ __align__(16) float sWv[D + 4];
  __shared__ uint64_t sNew[C3_CH / 64], sOld[C3_CH / 64];
  __shared__ int sPerm[C3_SPB * C3_CH];
  double(*red0)[D] = reinterpret_cast<double(*)[D]>(sK);          // after the last block
  double(*red1)[D] = reinterpret_cast<double(*)[D]>(sK + NW * D * 8);
  const int s = blockIdx.x;
  if (W.salive[s] != 1) return;
  const int2 un = W.snode[par * W.smax + s];
  const int u = un.x, x = un.y;
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  const int st = X.start[nb + x], m = X.size[nb + x];
  const int q0 = st + blockIdx.y * (C3_SPB * C3_CH);
  if (q0 >= st + m) return;
  const int total = min(C3_SPB * C3_CH, st + m - q0);
  const int nblk = (total + C3_CH - 1) / C3_CH;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool tiny = W.tiny[u] != 0;
  for (int i = tid; i < total; i += C3_T) sPerm[i] = X.perm[ub + q0 + i];
  for (int c = tid; c < D; c += C3_T) sWv[c] = W.sw[(size_t)s * D + c];
  const float b = W.sb[s];
  __syncthreads();
  uint4 buf[2][PER];
  int oldf[2] = {0, 0};
  auto load = [&](int slot, int blk) {
    const int rows = min(C3_CH, total - blk * C3_CH);
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int i = tid + p * C3_T, r = i / PPR, pc = i - r * PPR;
      if (r < rows)
        buf[slot][p] = kvc_nt_load16(
            k + u * P.ks[0] + (int64_t)sPerm[blk * C3_CH + r] * P.ks[1] + pc * 8);
    }
    oldf[slot] = (it > 0 && tid < rows) ? W.flags[ub + q0 + blk * C3_CH + tid] : 0;
  };
  load(0, 0);
  if (nblk > 1) load(1, 1);
  double a0[CPL], a1[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) a0[i] = a1[i] = 0.0;
  int dn1 = 0, flips = 0;
#pragma unroll
  for (int blk = 0; blk < C3_SPB; ++blk) {
    if (blk >= nblk) break;
    const int rows = min(C3_CH, total - blk * C3_CH);
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int i = tid + p * C3_T, r = i / PPR, pc = i - r * PPR;
      if (r < rows)
        *reinterpret_cast<uint4*>(sK + r * RB + pc * 16) =
            tiny ? c3_snap8_fast(buf[blk & 1][p]) : buf[blk & 1][p];
    }
    const bool o = oldf[blk & 1] != 0;
    __syncthreads();
    if (blk + 2 < nblk) load(blk & 1, blk + 2);
    if (tid < C3_CH) {
      const size_t pos = ub + q0 + blk * C3_CH + tid;
      const bool f = tid < rows && c3_plane<D>(sK + tid * RB, sWv) > b;
      if (tid < rows) W.flags[pos] = f ? 1 : 0;
      const uint64_t wn = __ballot(f), wo = __ballot(o);
      if (lane == 0) {
        sNew[wave] = wn;
        sOld[wave] = wo;
      }
    }
    __syncthreads();
    // Wave w handles rows 32w .. 32w + 31, lanes over the columns.
    const int rb = wave * 32;
    const int nr = max(0, min(32, rows - rb));
    const uint32_t live = nr >= 32 ? 0xFFFFFFFFu : (1u << nr) - 1u;
    const uint32_t nw = (uint32_t)(sNew[rb >> 6] >> (rb & 63)) & live;
    const uint32_t ow = (uint32_t)(sOld[rb >> 6] >> (rb & 63)) & live;
    if (it == 0) {
      c3_acc_cols<RB, CPL, false>(sK, rb, live, lane, a0);
      c3_acc_cols<RB, CPL, false>(sK, rb, nw, lane, a1);
    } else {
      c3_acc_cols<RB, CPL, false>(sK, rb, nw & ~ow, lane, a1);
      c3_acc_cols<RB, CPL, true>(sK, rb, ow & ~nw, lane, a1);
    }
    dn1 += __popc(nw) - __popc(ow);
    flips += __popc(nw ^ ow);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    red0[wave][lane * CPL + i] = a0[i];
    red1[wave][lane * CPL + i] = a1[i];
  }
  __shared__ int sDn[NW], sFl[NW];
  if (lane == 0) {
    sDn[wave] = dn1;
    sFl[wave] = flips;
  }
  __syncthreads();
  for (int c = tid; c < (it == 0 ? 2 * D : D); c += C3_T) {
    const int h = c < D ? 1 : 0, cc = c < D ? c : c - D;
    double t = 0.0;
    for (int w = 0; w < NW; ++w) t += h ? red1[w][cc] : red0[w][cc];
    atomicAdd(h ? &W.s1[(size_t)s * D + cc] : &W.s0[(size_t)s * D + cc], t);
  }
  if (tid == 0) {
    atomicAdd(&W.sn1[s], sDn[0] + sDn[1] + sDn[2] + sDn[3]);
    if (it > 0) atomicAdd(&W.sflip[s], sFl[0] + sFl[1] + sFl[2] + sFl[3]);
  }
}

// New means of a span node from its total (s0) and running cluster-1 sum
// (s1) and count; the last iteration records the split.
template <int D>
__global__ __launch_bounds__(64) void c3_span_fin_kernel(C3Desc P, int par, int it, int last,
                                                         C3Index X, C3Work W) {
  constexpr int CPL = D / 64;
  const int s = blockIdx.x, lane = threadIdx.x;
  if (W.salive[s] != 1) return;
  const int2 un = W.snode[par * W.smax + s];
  const int u = un.x, x = un.y;
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  const int st = X.start[nb + x], m = X.size[nb + x];
  const int n1 = W.sn1[s];
  if (n1 == 0 || n1 == m) {
    if (lane == 0) {
      W.salive[s] = 0;
      W.res_n0[ub + st] = -1;
    }
    return;
  }
  // exact member sums divided by the counts, correctly rounded
  const double n0d = (double)(m - n1), n1d = (double)n1;
  const double y0 = 1.0 / n0d, y1 = 1.0 / n1d;
  double mu0[CPL], mu1[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const size_t o = (size_t)s * D + lane * CPL + i;
    mu0[i] = c3_div(W.s0[o] - W.s1[o], n0d, y0);
    mu1[i] = c3_div(W.s1[o], n1d, y1);
  }
  // A partition that repeats the previous one is a fixed point: record the
  // split now and stop iterating this node.
  const bool conv = it > 0 && W.sflip[s] == 0;
  if (lane == 0) W.sflip[s] = 0;
  if (conv && lane == 0) W.salive[s] = 2;
  if (!last && !conv) {
    float w[CPL];
    const float b = c3_bisect<CPL>(mu0, mu1, w);
#pragma unroll
    for (int i = 0; i < CPL; ++i) W.sw[(size_t)s * D + lane * CPL + i] = w[i];
    if (lane == 0) W.sb[s] = b;
  } else {
    const int n0 = m - n1;
    uint16_t* c0 = W.cres + (ub + st) * D;
    uint16_t* c1 = W.cres + (ub + st + n0) * D;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      c0[lane * CPL + i] = c3_to_bf16(mu0[i]);
      c1[lane * CPL + i] = c3_to_bf16(mu1[i]);
    }
    if (lane == 0) W.res_n0[ub + st] = n0;
  }
}

// Stable partition of a split span node's perm range (through ptmp).
__global__ __launch_bounds__(C3_BIG) void c3_span_part_kernel(C3Desc P, int par, C3Index X,
                                                              C3Work W) {
  __shared__ int scan[C3_BIG / 64];
  const int s = blockIdx.x;
  if (W.salive[s] == 0) return;
  const int2 un = W.snode[par * W.smax + s];
  const int u = un.x, x = un.y;
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  const int st = X.start[nb + x], m = X.size[nb + x];
  const int n0 = W.res_n0[ub + st];
  int zeros = 0;
  for (int b0 = 0; b0 < m; b0 += C3_BIG) {
    const int i = b0 + threadIdx.x;
    const bool in = i < m;
    const int f = in ? W.flags[ub + st + i] : 0;
    int tot;
    const int zb = c3_block_scan<C3_BIG>(in && !f, scan, &tot) + zeros;
    if (in) W.ptmp[ub + st + (f ? n0 + (i - zb) : zb)] = X.perm[ub + st + i];
    zeros += tot;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < m; i += C3_BIG) X.perm[ub + st + i] = W.ptmp[ub + st + i];
}

// ---------------------------------------------------------------------------
// Build: children ids and records, next depth's work lists
// ---------------------------------------------------------------------------
// Copy of N 16-byte pieces with every load issued before the first store.
// Written as a plain copy, the compiler turns it into a memory copy whose
// expansion waits on each load before its store, N latencies in a row; the
// source is read once, so non-temporal loads suit it and keep the loads
// apart from the stores.
typedef unsigned int c3_u32x4 __attribute__((ext_vector_type(4)));
template <int N>
__device__ __forceinline__ void c3_copy_row(const uint4* src, uint4* dst) {
  const c3_u32x4* s = reinterpret_cast<const c3_u32x4*>(src);
  c3_u32x4* d = reinterpret_cast<c3_u32x4*>(dst);
  c3_u32x4 r[N];
#pragma unroll
  for (int i = 0; i < N; ++i) r[i] = __builtin_nontemporal_load(s + i);
#pragma unroll
  for (int i = 0; i < N; ++i) d[i] = r[i];
}

template <int D>
__global__ __launch_bounds__(C3_BIG) void c3_ids_kernel(C3Desc P, int dep, C3Index X, C3Work W) {
  __shared__ int scan[C3_BIG / 64];
  const int u = blockIdx.x;
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  int32_t* lv = W.lvl + (size_t)u * (C3_MAXD + 2);
  const int lo = lv[dep], hi = lv[dep + 1];
  int made = 0, cand = 0, big = 0;
  int32_t* cnt = W.cnt + (dep + 1) * 4;
  const int par = (dep + 1) & 1;
  for (int b0 = lo; b0 < hi; b0 += C3_BIG) {
    const int x = b0 + threadIdx.x;
    const bool in = x < hi;
    int st = 0, m = 0, n0 = -1;
    if (in) {
      st = X.start[nb + x];
      m = X.size[nb + x];
      if (m > C3_LEAF) n0 = W.res_n0[ub + st];
      W.head[ub + st] = -1;
    }
    const bool ok = n0 > 0;
    int tot;
    const int rank = c3_block_scan<C3_BIG>(ok, scan, &tot);
    if (ok) {
      const int l = hi + 2 * (made + rank);
      X.left[nb + x] = l;
      const int cs[2] = {st, st + n0}, cm[2] = {n0, m - n0};
#pragma unroll
      for (int side = 0; side < 2; ++side) {
        const size_t y = nb + l + side;
        X.start[y] = cs[side];
        X.size[y] = cm[side];
        X.left[y] = -1;
        X.parent[y] = x;
        X.depth[y] = dep + 1;
        c3_copy_row<D / 8>(reinterpret_cast<const uint4*>(W.cres + (ub + cs[side]) * D),
                           reinterpret_cast<uint4*>(X.cent + y * D));
        if (cm[side] > C3_LEAF) {
          ++cand;
          if (cm[side] <= C3_MLOC) {
            W.head[ub + cs[side]] = l + side;
            c3_list_chunk(P, W, u, cs[side], dep + 1);
          } else {
            big = max(big, cm[side]);
            const int slot = atomicAdd(&cnt[1], 1);
            W.snode[par * W.smax + slot] = make_int2(u, l + side);
          }
        }
      }
    }
    made += tot;
  }
  if (cand) atomicAdd(&cnt[0], cand);
  if (big) atomicMax(&cnt[2], big);
  __syncthreads();
  if (threadIdx.x == 0) {
    lv[dep + 2] = hi + 2 * made;
    X.nn[u] = hi + 2 * made;
  }
}

// Initial frontier: nodes at depth round(log2(n/16)) and leaves above it,
// listed by start; e = 0.
__global__ __launch_bounds__(C3_BIG) void c3_frontier_kernel(C3Desc P, C3Index X, C3State S,
                                                             C3Work W) {
  __shared__ int scan[C3_BIG / 64];
  const int u = blockIdx.x, n = c3_n(P, u);
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  int d0 = 0;
  while ((int64_t)n * n >= (int64_t(1) << (2 * d0 + 9))) ++d0;
  for (int p = threadIdx.x; p < n; p += C3_BIG) W.ptmp[ub + p] = -1;
  __syncthreads();
  const int nn = X.nn[u];
  for (int x = threadIdx.x; x < nn; x += C3_BIG) {
    const int dp = X.depth[nb + x];
    if (dp == d0 || (dp < d0 && X.left[nb + x] < 0)) W.ptmp[ub + X.start[nb + x]] = x;
  }
  __syncthreads();
  int a = 0;
  for (int b0 = 0; b0 < n; b0 += C3_BIG) {
    const int p = b0 + threadIdx.x;
    const int x = p < n ? W.ptmp[ub + p] : -1;
    int tot;
    const int r = c3_block_scan<C3_BIG>(x >= 0, scan, &tot) + a;
    if (x >= 0) {
      S.fr[ub + r] = x;
      S.e[ub + r] = 0.0;
    }
    a += tot;
  }
  if (threadIdx.x == 0) S.count[u] = a;
}

// ---------------------------------------------------------------------------
// Step: scores
// ---------------------------------------------------------------------------
// sigma = max over the group's query heads of cos(q_g, c) for every frontier
// centroid c, on v_mfma_f32_16x16x32_bf16: the G query heads are the A rows
// (16 per block, zero past G) and 16 frontier centroids the B columns; at
// k-step ks lane l holds dims ks*32 + (l/16)*8 .. +7 of both operands, so a
// centroid row is read as 64-byte runs, and all of a wave's loads (64
// entries) are in flight before its first MFMA.  Output lane l holds entry
// l % 16 for heads (l/16)*4 .. +3 of the block.  The centroid's squared norm
// is summed by the four lanes holding its dims, then across them.
typedef __bf16 c3_bf16x8 __attribute__((ext_vector_type(8)));
typedef float c3_f4 __attribute__((ext_vector_type(4)));

template <int D, int HPT>
__global__ __launch_bounds__(C3_T) void c3_score_kernel(C3Desc P, C3Index X, C3State S,
                                                        const uint16_t* __restrict__ q,
                                                        float* __restrict__ sigma) {
  constexpr int KS = D / 32, NQB = (HPT + 15) / 16, WPB = C3_T / 64;
  __shared__ float sQn[HPT];
  const int u = blockIdx.x / C3_SW, part = blockIdx.x - u * C3_SW;
  if (c3_n(P, u) <= c3_b(P, u)) return;
  const int G = P.gqa, A = S.count[u];
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const uint16_t* qs = q + (size_t)u * G * D;
  // Issue order: the wave's first 64 frontier indices, the query rows (the
  // A operand, and for threads below HPT the row of their head's norm), then
  // the first 64 centroid rows, so that only the index -> row dependence is
  // serial (entries past A reload the last one and are not written).
  uint4 kraw[4][KS];
  int xs[4];
  auto load_ids = [&](int b) {
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) xs[kg] = S.fr[ub + min(b + kg * 16 + col, A - 1)];
  };
  auto load_rows = [&]() {
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const uint16_t* row = X.cent + (nb + xs[kg]) * D + grp * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kraw[kg][ks] = *reinterpret_cast<const uint4*>(row + ks * 32);
    }
  };
  const int base0 = (part * WPB + wave) * 64;
  int base = base0;
  const bool any = base0 < A;
  if (any) load_ids(base0);
  uint4 qraw[NQB][KS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qraw[qb][ks] = *reinterpret_cast<const uint4*>(qs + (size_t)min(qb * 16 + col, G - 1) * D + ks * 32 + grp * 8);
  const bool nthread = (int)threadIdx.x < HPT;
  uint4 qr[D / 8];
  if (nthread) {
    const uint4* qrow = reinterpret_cast<const uint4*>(qs + (size_t)min((int)threadIdx.x, G - 1) * D);
#pragma unroll
    for (int p = 0; p < D / 8; ++p) qr[p] = qrow[p];
  }
  if (any) load_rows();
  // query norms: a thread per head, the squares summed in dimension order
  if (nthread) {
    float s = 0.0f;
#pragma unroll
    for (int p = 0; p < D / 8; ++p) {
      const uint32_t w[4] = {qr[p].x, qr[p].y, qr[p].z, qr[p].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = c3_bf(w[j] & 0xFFFFu), hi = c3_bf(w[j] >> 16);
        s = fmaf(lo, lo, s);
        s = fmaf(hi, hi, s);
      }
    }
    sQn[threadIdx.x] = (int)threadIdx.x < G ? sqrtf(s) : 0.0f;
  }
  // A operand; heads past G: the last head's bits masked to zero
  c3_bf16x8 qa[NQB][KS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const uint32_t keep = qb * 16 + col < G ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 raw = qraw[qb][ks];
      raw.x &= keep;
      raw.y &= keep;
      raw.z &= keep;
      raw.w &= keep;
      __builtin_memcpy(&qa[qb][ks], &raw, 16);
    }
  }
  __syncthreads();
  float qn[NQB][4];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = qb * 16 + grp * 4 + i;
      qn[qb][i] = h < G ? sQn[h] : 0.0f;
    }
  for (; base < A; base += C3_SW * C3_T) {
    if (base != base0) {
      load_ids(base);
      load_rows();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      c3_bf16x8 kb[KS];
      float cn = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        __builtin_memcpy(&kb[ks], &kraw[kg][ks], 16);
        const uint32_t w[4] = {kraw[kg][ks].x, kraw[kg][ks].y, kraw[kg][ks].z, kraw[kg][ks].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = c3_bf(w[j] & 0xFFFFu), hi = c3_bf(w[j] >> 16);
          cn = fmaf(lo, lo, cn);
          cn = fmaf(hi, hi, cn);
        }
      }
      cn += __shfl_xor(cn, 16);
      cn += __shfl_xor(cn, 32);
      cn = sqrtf(cn);
      float best = -INFINITY;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        if (qb * 16 >= G) break;   // (uniform: no heads in this block)
        c3_f4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[qb][ks], kb[ks], t, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (qb * 16 + grp * 4 + i < G) {
            const float den = qn[qb][i] * cn;
            best = fmaxf(best, den > 0.0f ? t[i] / den : 0.0f);
          }
      }
      best = fmaxf(best, __shfl_xor(best, 16));
      best = fmaxf(best, __shfl_xor(best, 32));
      const int i = base + kg * 16 + col;
      if (grp == 0 && i < A) sigma[ub + i] = best;
    }
  }
}

// ---------------------------------------------------------------------------
// Step: selection and frontier update (one workgroup per cache)
// ---------------------------------------------------------------------------
// Ascending key of a score for a descending order: larger sigma first
// (-0.0 taken as +0.0).
__device__ inline uint32_t c3_desc_key(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ~ord;
}

__device__ inline double c3_ema(const C3Desc& P, double e, float s) {
  const double a = P.lam * e;
  const double c = (1.0 - P.lam) * (double)s;
  return a + c;
}

__global__ __launch_bounds__(C3_BIG) void c3_select_update_kernel(
    C3Desc P, C3Index X, C3State Sin, const float* __restrict__ sigma, int32_t* __restrict__ idx,
    C3State Sout, int do_sel, int do_upd) {
  __shared__ uint32_t hist[C3_BIG / 64][256];
  __shared__ uint32_t bm[C3_MAX_CAP / 32];
  __shared__ int scan[C3_BIG / 64];
  __shared__ uint32_t s_digit, s_below;
  __shared__ double rv[C3_BIG / 64];
  __shared__ int ri[C3_BIG / 64];
  __shared__ int sSplit[8], sMerge[8];
  __shared__ int sNs, sNm;
  const int u = blockIdx.x, n = c3_n(P, u), B = c3_b(P, u);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const size_t ub = (size_t)u * P.cap, nb = (size_t)u * P.ncap;
  const int A = Sin.count[u];
  const int32_t* F = Sin.fr + ub;
  const double* E = Sin.e + ub;
  const float* sg = sigma + ub;
  const int32_t* NS = X.start + nb;
  const int32_t* NZ = X.size + nb;
  const int32_t* NL = X.left + nb;
  const int32_t* NP = X.parent + nb;
  if (n <= B) {
    if (do_sel)
      for (int t = tid; t < n; t += C3_BIG) idx[(size_t)u * P.kept_cap + t] = t;
    if (do_upd) {
      for (int i = tid; i < A; i += C3_BIG) {
        Sout.fr[ub + i] = F[i];
        Sout.e[ub + i] = E[i];
      }
      if (tid == 0) Sout.count[u] = A;
    }
    return;
  }

  if (do_sel) {
    // Key, node and weight of the thread's entries tid and tid + C3_BIG,
    // read once (entries past 2 C3_BIG are read again in every pass).
    uint32_t ck[2], cw[2];
    int cx[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + j * C3_BIG;
      cx[j] = i < A ? F[i] : 0;
      ck[j] = i < A ? c3_desc_key(sg[i]) : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) cw[j] = tid + j * C3_BIG < A ? (uint32_t)NZ[cx[j]] : 0u;
    // Weighted radix select: the smallest key T with weight(key <= T) >= B.
    uint32_t prefix = 0, pmask = 0, need = (uint32_t)B;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = lane; b < 256; b += 64) hist[wave][b] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (tid + j * C3_BIG < A && (ck[j] & pmask) == prefix)
          atomicAdd(&hist[wave][(ck[j] >> shift) & 255u], cw[j]);
      for (int i = tid + 2 * C3_BIG; i < A; i += C3_BIG) {
        const uint32_t key = c3_desc_key(sg[i]);
        if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], (uint32_t)NZ[F[i]]);
      }
      __syncthreads();
      if (wave == 0) {
        uint32_t c4[4], own = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t s = 0;
          for (int w = 0; w < C3_BIG / 64; ++w) s += hist[w][4 * lane + e];
          c4[e] = s;
          own += s;
        }
        uint32_t incl = own;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_up(incl, o);
          if (lane >= o) incl += y;
        }
        const uint32_t excl = incl - own;
        if (excl < need && need <= incl) {
          uint32_t run = excl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (run < need && need <= run + c4[e]) {
              s_digit = (uint32_t)(4 * lane + e);
              s_below = run;
            }
            run += c4[e];
          }
        }
      }
      __syncthreads();
      prefix |= s_digit << shift;
      pmask |= 255u << shift;
      need -= s_below;
      __syncthreads();
    }
    // Keys below T are taken whole; entries equal to T (ties) in entry order
    // until `need` keys.  Their members go into a position bitmap.
    const int nw = (n + 31) >> 5;
    for (int w = tid; w < nw; w += C3_BIG) bm[w] = 0;
    __syncthreads();
    int tie_before = 0;
    for (int b0 = 0; b0 < A; b0 += C3_BIG) {
      const int i = b0 + tid;
      const bool in = i < A;
      const int jc = b0 / C3_BIG;   // uniform
      const uint32_t key = !in ? 0xFFFFFFFFu : jc < 2 ? ck[jc & 1] : c3_desc_key(sg[i]);
      const int x = !in ? 0 : jc < 2 ? cx[jc & 1] : F[i];
      const int m = !in ? 0 : jc < 2 ? (int)cw[jc & 1] : NZ[x];
      const bool eq = in && key == prefix;
      int tot;
      const int before = c3_block_scan<C3_BIG>(eq ? m : 0, scan, &tot) + tie_before;
      int take = 0;
      if (in && key < prefix) take = m;
      if (eq) take = min(m, max(0, (int)need - before));
      if (take > 0) {
        const int st = NS[x];
        for (int j = 0; j < take; ++j) {
          const int pos = X.perm[ub + st + j];
          atomicOr(&bm[pos >> 5], 1u << (pos & 31));
        }
      }
      tie_before += tot;
    }
    __syncthreads();
    int kept = 0;
    for (int b0 = 0; b0 < nw; b0 += C3_BIG) {
      const int w = b0 + tid;
      const uint32_t bits = w < nw ? bm[w] : 0u;
      int tot;
      int r = c3_block_scan<C3_BIG>(__popc(bits), scan, &tot) + kept;
      uint32_t v = bits;
      while (v) {
        const int bit = __ffs(v) - 1;
        idx[(size_t)u * P.kept_cap + r++] = w * 32 + bit;
        v &= v - 1;
      }
      kept += tot;
    }
  }

  if (do_upd) {
    // R masked max reductions: split candidates (nodes with children),
    // highest e, earliest entry on ties.
    const int R = P.R;
    if (tid == 0) {
      sNs = 0;
      sNm = 0;
    }
    // Entries tid and tid + C3_BIG, read once for all rounds: EMA, whether
    // the node has children, and whether (i, i + 1) is a sibling pair and
    // its larger EMA (entries past 2 C3_BIG are read again in every round).
    double cema[2], cpr[2];
    bool ckid[2], cpair[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = tid + j * C3_BIG;
      ckid[j] = cpair[j] = false;
      cema[j] = cpr[j] = 0.0;
      if (i < A) {
        const int x = F[i];
        cema[j] = c3_ema(P, E[i], sg[i]);
        ckid[j] = NL[x] >= 0;
        if (i + 1 < A) {
          const int pp = NP[x];
          cpair[j] = pp >= 0 && NL[pp] == x && F[i + 1] == x + 1;
          if (cpair[j]) cpr[j] = fmax(cema[j], c3_ema(P, E[i + 1], sg[i + 1]));
        }
      }
    }
    __syncthreads();
    for (int round = 0; round < R; ++round) {
      double bv = -INFINITY;
      int bi = -1;
      const int ns = sNs;
      auto consider = [&](int i, bool kid, double e) {
        if (!kid) return;
        bool chosen = false;
        for (int t = 0; t < ns; ++t) chosen |= sSplit[t] == i;
        if (chosen) return;
        if (bi < 0 || e > bv || (e == bv && i < bi)) {
          bv = e;
          bi = i;
        }
      };
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (tid + j * C3_BIG < A) consider(tid + j * C3_BIG, ckid[j], cema[j]);
      for (int i = tid + 2 * C3_BIG; i < A; i += C3_BIG)
        consider(i, NL[F[i]] >= 0, c3_ema(P, E[i], sg[i]));
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const double ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
          bv = ov;
          bi = oi;
        }
      }
      if (lane == 0) {
        rv[wave] = bv;
        ri[wave] = bi;
      }
      __syncthreads();
      if (tid == 0) {
        double v = -INFINITY;
        int b = -1;
        for (int w = 0; w < C3_BIG / 64; ++w)
          if (ri[w] >= 0 && (b < 0 || rv[w] > v || (rv[w] == v && ri[w] < b))) {
            v = rv[w];
            b = ri[w];
          }
        if (b >= 0) sSplit[sNs++] = b;
      }
      __syncthreads();
    }
    // R masked min reductions over sibling pairs (i, i + 1), neither a split
    // candidate: lowest max(e_i, e_i+1), earliest pair on ties.
    const int ns = sNs;
    for (int round = 0; round < R; ++round) {
      double bv = INFINITY;
      int bi = -1;
      const int nm = sNm;
      auto consider = [&](int i, bool pair, double pr) {
        if (!pair) return;
        bool skip = false;
        for (int t = 0; t < ns; ++t) skip |= sSplit[t] == i || sSplit[t] == i + 1;
        for (int t = 0; t < nm; ++t) skip |= sMerge[t] == i;
        if (skip) return;
        if (bi < 0 || pr < bv || (pr == bv && i < bi)) {
          bv = pr;
          bi = i;
        }
      };
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (tid + j * C3_BIG + 1 < A) consider(tid + j * C3_BIG, cpair[j], cpr[j]);
      for (int i = tid + 2 * C3_BIG; i + 1 < A; i += C3_BIG) {
        const int x = F[i];
        const int p = NP[x];
        const bool pair = p >= 0 && NL[p] == x && F[i + 1] == x + 1;
        consider(i, pair, pair ? fmax(c3_ema(P, E[i], sg[i]), c3_ema(P, E[i + 1], sg[i + 1])) : 0.0);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const double ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (oi >= 0 && (bi < 0 || ov < bv || (ov == bv && oi < bi))) {
          bv = ov;
          bi = oi;
        }
      }
      if (lane == 0) {
        rv[wave] = bv;
        ri[wave] = bi;
      }
      __syncthreads();
      if (tid == 0) {
        double v = INFINITY;
        int b = -1;
        for (int w = 0; w < C3_BIG / 64; ++w)
          if (ri[w] >= 0 && (b < 0 || rv[w] < v || (rv[w] == v && ri[w] < b))) {
            v = rv[w];
            b = ri[w];
          }
        if (b >= 0) sMerge[sNm++] = b;
      }
      __syncthreads();
    }
    const int kx = min(sNs, sNm);
    // Rewrite the frontier: a split entry emits its two children, a merged
    // pair its parent, every other entry itself.
    int outp = 0;
    for (int b0 = 0; b0 < A; b0 += C3_BIG) {
      const int i = b0 + tid;
      int cnt = 0;
      bool sp = false, mg = false;
      if (i < A) {
        for (int t = 0; t < kx; ++t) {
          sp |= sSplit[t] == i;
          mg |= sMerge[t] == i;
        }
        bool second = false;
        for (int t = 0; t < kx; ++t) second |= sMerge[t] == i - 1;
        cnt = sp ? 2 : (second ? 0 : 1);
      }
      int tot;
      const int o = c3_block_scan<C3_BIG>(cnt, scan, &tot) + outp;
      if (cnt > 0) {
        const int x = F[i];
        const double e = c3_ema(P, E[i], sg[i]);
        if (sp) {
          const int l = NL[x];
          Sout.fr[ub + o] = l;
          Sout.fr[ub + o + 1] = l + 1;
          Sout.e[ub + o] = e;
          Sout.e[ub + o + 1] = e;
        } else if (mg) {
          Sout.fr[ub + o] = NP[x];
          Sout.e[ub + o] = fmax(e, c3_ema(P, E[i + 1], sg[i + 1]));
        } else {
          Sout.fr[ub + o] = x;
          Sout.e[ub + o] = e;
        }
      }
      outp += tot;
    }
    if (tid == 0) Sout.count[u] = outp;
  }
}

// ---------------------------------------------------------------------------
// Step: gather of the kept rows
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(C3_T) void c3_gather_kernel(C3Desc P, int bpc,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ idx,
                                                         uint16_t* __restrict__ ko,
                                                         uint16_t* __restrict__ vo) {
  constexpr int PPR = D / 8;
  constexpr int RPP = C3_T / PPR;
  constexpr int PASSES = 4;
  const int u = blockIdx.x / bpc;
  const int t0 = (blockIdx.x - u * bpc) * RPP * PASSES;
  const int n = c3_n(P, u);
  const int nl = min(n, c3_b(P, u));
  if (t0 >= nl) return;
  const int pc = threadIdx.x % PPR;
  uint4 kv[PASSES], vv[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + p * RPP + threadIdx.x / PPR;
    if (t >= nl) continue;
    int s = idx[(size_t)u * P.kept_cap + t];
    if ((unsigned)s >= (unsigned)n) s = 0;
    kv[p] = kvc_nt_load16(k + u * P.ks[0] + (int64_t)s * P.ks[1] + pc * 8);
    vv[p] = kvc_nt_load16(v + u * P.vs[0] + (int64_t)s * P.vs[1] + pc * 8);
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + p * RPP + threadIdx.x / PPR;
    if (t >= nl) continue;
    uint4* kd = reinterpret_cast<uint4*>(ko + u * P.os[0] + (int64_t)t * P.os[1] + pc * 8);
    uint4* vd = reinterpret_cast<uint4*>(vo + u * P.os[0] + (int64_t)t * P.os[1] + pc * 8);
    __builtin_nontemporal_store(kv[p].x, &kd->x);
    __builtin_nontemporal_store(kv[p].y, &kd->y);
    __builtin_nontemporal_store(kv[p].z, &kd->z);
    __builtin_nontemporal_store(kv[p].w, &kd->w);
    __builtin_nontemporal_store(vv[p].x, &vd->x);
    __builtin_nontemporal_store(vv[p].y, &vd->y);
    __builtin_nontemporal_store(vv[p].z, &vd->z);
    __builtin_nontemporal_store(vv[p].w, &vd->w);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static kvc_status c3_hip(hipError_t e) {
  if (e == hipSuccess) return KVC_OK;
  kvc_note_hip_error((int)e);
  return KVC_ERR_HIP;
}

static size_t c3_up(size_t x) { return (x + 255) & ~size_t(255); }

static kvc_status c3_desc(const kvc_c3_problem* p, const kvc_c3_params* prm, C3Desc* V) {
  if (!p || !prm || !V || !p->len || !p->budget) return KVC_ERR_INVALID_ARG;
  if (p->n_seq < 1 || p->n_layers < 1 || p->n_kv_heads < 1 || p->gqa_group < 1 ||
      p->head_dim < 1 || p->capacity < 1)
    return KVC_ERR_INVALID_ARG;
  if (!(prm->lambda >= 0.0 && prm->lambda <= 1.0) || prm->r_swaps < 0 || prm->r_swaps > 8)
    return KVC_ERR_INVALID_ARG;
  for (int a = 0; a < 2; ++a) {
    if (p->k_stride[a] < 0 || p->v_stride[a] < 0 || p->out_stride[a] < 0) return KVC_ERR_INVALID_ARG;
    if (p->k_stride[a] % 8 || p->v_stride[a] % 8 || p->out_stride[a] % 8) return KVC_ERR_INVALID_ARG;
  }
  if (p->k_stride[1] < p->head_dim || p->v_stride[1] < p->head_dim || p->out_stride[1] < p->head_dim)
    return KVC_ERR_INVALID_ARG;
  if (p->k_stride[0] < p->k_stride[1] * p->capacity || p->v_stride[0] < p->v_stride[1] * p->capacity)
    return KVC_ERR_INVALID_ARG;
  if (p->n_seq > C3_MAX_SEQ || p->capacity > C3_MAX_CAP) return KVC_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return KVC_ERR_UNSUPPORTED;
  if (p->gqa_group > C3_MAX_G) return KVC_ERR_UNSUPPORTED;
  const int64_t upseq = (int64_t)p->n_layers * p->n_kv_heads;
  if (upseq > KVC_MAX_UNITS_PER_SEQ) return KVC_ERR_UNSUPPORTED;
  memset(V, 0, sizeof(*V));
  int64_t kept = 1;
  for (int i = 0; i < p->n_seq; ++i) {
    const int64_t n = p->len[i], B = p->budget[i];
    if (n < 0 || n > p->capacity || B < 1) return KVC_ERR_INVALID_ARG;
    V->len[i] = (int32_t)n;
    V->budget[i] = (int32_t)std::min<int64_t>(B, INT32_MAX);
    kept = std::max(kept, std::min(n, B));
  }
  if (p->out_stride[0] < p->out_stride[1] * kept) return KVC_ERR_INVALID_ARG;
  V->n_seq = p->n_seq;
  V->upseq = (int32_t)upseq;
  V->gqa = p->gqa_group;
  V->d = p->head_dim;
  V->n_units = (int32_t)(upseq * p->n_seq);
  V->R = prm->r_swaps;
  V->cap = (int32_t)p->capacity;
  V->ncap = (int32_t)(2 * p->capacity);
  V->nchunk = (int32_t)((p->capacity + C3_CH - 1) / C3_CH);
  V->kept_cap = (int32_t)kept;
  V->lam = prm->lambda;
  V->seed = prm->seed;
  for (int a = 0; a < 2; ++a) {
    V->ks[a] = p->k_stride[a];
    V->vs[a] = p->v_stride[a];
    V->os[a] = p->out_stride[a];
  }
  return KVC_OK;
}

static int64_t c3_smax(const C3Desc& V) {
  return (int64_t)V.n_units * (V.cap / (C3_MLOC + 1) + 1);
}

static void c3_layout(const C3Desc& V, kvc_c3_layout* L) {
  memset(L, 0, sizeof(*L));
  const size_t U = (size_t)V.n_units, NC = (size_t)V.ncap, CAP = (size_t)V.cap, D = (size_t)V.d;
  L->node_cap = (int64_t)NC;
  L->kept_cap = V.kept_cap;
  size_t o = 0;
  L->start = o;    o += c3_up(4 * U * NC);
  L->size = o;     o += c3_up(4 * U * NC);
  L->left = o;     o += c3_up(4 * U * NC);
  L->parent = o;   o += c3_up(4 * U * NC);
  L->depth = o;    o += c3_up(4 * U * NC);
  L->perm = o;     o += c3_up(4 * U * CAP);
  L->n_nodes = o;  o += c3_up(4 * U);
  L->centroid = o; o += c3_up(2 * U * NC * D);
  L->index_bytes = o;
  o = 0;
  L->count = o;    o += c3_up(4 * U);
  L->frontier = o; o += c3_up(4 * U * CAP);
  L->ema = o;      o += c3_up(8 * U * CAP);
  L->state_bytes = o;
  const size_t S = (size_t)c3_smax(V);
  L->build_workspace_bytes = c3_up(2 * U * CAP * D) + c3_up(4 * U * CAP) + c3_up(U * CAP) +
                             c3_up(4 * U * CAP) + c3_up(4 * U * CAP) +
                             c3_up(4 * U * (C3_MAXD + 2)) + c3_up(8 * U * D) + c3_up(4 * U) +
                             c3_up(8 * 2 * S) +
                             c3_up(4 * S * D) + c3_up(4 * S) + 2 * c3_up(8 * S * D) + c3_up(4 * S) +
                             c3_up(4 * S) + c3_up(4 * S) + c3_up(16 * (C3_MAXD + 1)) + c3_up(4) +
                             c3_up(4 * U * V.nchunk) + c3_up(8 * U * V.nchunk);
  L->step_workspace_bytes = c3_up(4 * U * CAP);
}

static C3Index c3_index(const kvc_c3_layout& L, const void* base) {
  char* b = (char*)base;
  C3Index X;
  X.start = (int32_t*)(b + L.start);
  X.size = (int32_t*)(b + L.size);
  X.left = (int32_t*)(b + L.left);
  X.parent = (int32_t*)(b + L.parent);
  X.depth = (int32_t*)(b + L.depth);
  X.perm = (int32_t*)(b + L.perm);
  X.nn = (int32_t*)(b + L.n_nodes);
  X.cent = (uint16_t*)(b + L.centroid);
  return X;
}

static C3State c3_state(const kvc_c3_layout& L, const void* base) {
  char* b = (char*)base;
  C3State S;
  S.count = (int32_t*)(b + L.count);
  S.fr = (int32_t*)(b + L.frontier);
  S.e = (double*)(b + L.ema);
  return S;
}

static C3Work c3_work(const C3Desc& V, void* ws) {
  const size_t U = (size_t)V.n_units, CAP = (size_t)V.cap, D = (size_t)V.d;
  const size_t S = (size_t)c3_smax(V);
  char* p = (char*)ws;
  C3Work W;
  W.cres = (uint16_t*)p;   p += c3_up(2 * U * CAP * D);
  W.res_n0 = (int32_t*)p;  p += c3_up(4 * U * CAP);
  W.flags = (uint8_t*)p;   p += c3_up(U * CAP);
  W.head = (int32_t*)p;    p += c3_up(4 * U * CAP);
  W.ptmp = (int32_t*)p;    p += c3_up(4 * U * CAP);
  W.lvl = (int32_t*)p;     p += c3_up(4 * U * (C3_MAXD + 2));
  W.rsum = (double*)p;     p += c3_up(8 * U * D);
  W.tiny = (int32_t*)p;    p += c3_up(4 * U);
  W.snode = (int2*)p;      p += c3_up(8 * 2 * S);
  W.sw = (float*)p;        p += c3_up(4 * S * D);
  W.sb = (float*)p;        p += c3_up(4 * S);
  W.s0 = (double*)p;       p += c3_up(8 * S * D);
  W.s1 = (double*)p;       p += c3_up(8 * S * D);
  W.sn1 = (int32_t*)p;     p += c3_up(4 * S);
  W.salive = (int32_t*)p;  p += c3_up(4 * S);
  W.sflip = (int32_t*)p;   p += c3_up(4 * S);
  W.cnt = (int32_t*)p;     p += c3_up(16 * (C3_MAXD + 1));
  W.err = (int32_t*)p;     p += c3_up(4);
  W.cflag = (int32_t*)p;   p += c3_up(4 * U * V.nchunk);
  W.clist = (int32_t*)p;
  W.smax = (int32_t)S;
  return W;
}

static bool c3_a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool c3_a256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

extern "C" kvc_status kvc_c3_plan(const kvc_c3_problem* prob, const kvc_c3_params* params,
                                  kvc_c3_layout* layout) {
  C3Desc V;
  const kvc_status st = c3_desc(prob, params, &V);
  if (st != KVC_OK) return st;
  if (!layout) return KVC_ERR_INVALID_ARG;
  c3_layout(V, layout);
  return KVC_OK;
}

#define C3_LAUNCH(D_, kern, grid, block, ...)                                       \
  do {                                                                              \
    if ((D_) == 128)                                                                \
      hipLaunchKernelGGL((kern<128>), (grid), (block), 0, st, __VA_ARGS__);          \
    else                                                                            \
      hipLaunchKernelGGL((kern<64>), (grid), (block), 0, st, __VA_ARGS__);           \
  } while (0)

extern "C" kvc_status kvc_c3_build(const kvc_c3_problem* prob, const kvc_c3_params* params,
                                   const void* k, void* index, void* state, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  C3Desc V;
  kvc_status rs = c3_desc(prob, params, &V);
  if (rs != KVC_OK) return rs;
  if (!k || !index || !state || !workspace) return KVC_ERR_INVALID_ARG;
  if (!c3_a16(k) || !c3_a256(index) || !c3_a256(state) || !c3_a256(workspace))
    return KVC_ERR_INVALID_ARG;
  kvc_c3_layout L;
  c3_layout(V, &L);
  if (workspace_bytes < L.build_workspace_bytes) return KVC_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const C3Index X = c3_index(L, index);
  const C3State S = c3_state(L, state);
  const C3Work W = c3_work(V, workspace);
  const uint16_t* kk = (const uint16_t*)k;
  hipError_t e = hipMemsetAsync(W.cnt, 0, c3_up(16 * (C3_MAXD + 1)) + c3_up(4), st);
  if (e != hipSuccess) return c3_hip(e);
  const unsigned U = (unsigned)V.n_units;
  hipLaunchKernelGGL(c3_init_kernel, dim3(U), dim3(C3_T), 0, st, V, X, W);
  C3_LAUNCH(V.d, c3_root_sum_kernel, dim3(U * V.nchunk), dim3(C3_T), V, W, kk);
  hipLaunchKernelGGL(c3_root_fin_kernel, dim3(U), dim3(C3_T), 0, st, V, X, W);
  if ((e = hipGetLastError()) != hipSuccess) return c3_hip(e);
  // Depth 0 work, known on the host.
  int cand = 0, span = 0, big = 0, chunks = 0;
  for (int u = 0; u < V.n_units; ++u) {
    const int n = V.len[u / V.upseq];
    if (n > C3_LEAF) ++cand;
    if (n > C3_LEAF && n <= C3_MLOC) ++chunks;
    if (n > C3_MLOC) {
      ++span;
      big = std::max(big, n);
    }
  }
  for (int dep = 0; dep < C3_MAXD && cand > 0; ++dep) {
    const int par = dep & 1;
    if (chunks > 0)
      C3_LAUNCH(V.d, c3_local_kernel, dim3((unsigned)chunks), dim3(C3_T), V, dep, X, W, kk);
    if (span > 0) {
      const dim3 g1((unsigned)span),
          g2((unsigned)span, (unsigned)((big + C3_SPB * C3_CH - 1) / (C3_SPB * C3_CH)));
      C3_LAUNCH(V.d, c3_span_init_kernel, g1, dim3(64), V, dep, par, X, W, kk);
      for (int it = 0; it < C3_ITERS; ++it) {
        C3_LAUNCH(V.d, c3_span_iter_kernel, g2, dim3(C3_T), V, par, it, X, W, kk);
        C3_LAUNCH(V.d, c3_span_fin_kernel, g1, dim3(64), V, par, it, it + 1 == C3_ITERS ? 1 : 0, X,
                  W);
      }
      hipLaunchKernelGGL(c3_span_part_kernel, g1, dim3(C3_BIG), 0, st, V, par, X, W);
    }
    C3_LAUNCH(V.d, c3_ids_kernel, dim3(U), dim3(C3_BIG), V, dep, X, W);
    if ((e = hipGetLastError()) != hipSuccess) return c3_hip(e);
    int32_t h[4];
    e = hipMemcpyAsync(h, W.cnt + (dep + 1) * 4, sizeof(h), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return c3_hip(e);
    cand = h[0];
    span = h[1];
    big = h[2];
    chunks = h[3];
    if (span > W.smax) return KVC_ERR_UNSUPPORTED;  // cannot happen: span nodes are disjoint
  }
  hipLaunchKernelGGL(c3_frontier_kernel, dim3(U), dim3(C3_BIG), 0, st, V, X, S, W);
  if ((e = hipGetLastError()) != hipSuccess) return c3_hip(e);
  int32_t bad = 0;
  e = hipMemcpyAsync(&bad, W.err, sizeof(bad), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return c3_hip(e);
  return bad ? KVC_ERR_INVALID_ARG : KVC_OK;
}

static hipError_t c3_launch_score(const C3Desc& V, const C3Index& X, const C3State& S,
                                  const void* q, float* sigma, hipStream_t st) {
  const dim3 grid((unsigned)V.n_units * C3_SW), block(C3_T);
  const uint16_t* qq = (const uint16_t*)q;
  if (V.d == 128) {
    if (V.gqa <= 8)
      hipLaunchKernelGGL((c3_score_kernel<128, 8>), grid, block, 0, st, V, X, S, qq, sigma);
    else
      hipLaunchKernelGGL((c3_score_kernel<128, 32>), grid, block, 0, st, V, X, S, qq, sigma);
  } else {
    if (V.gqa <= 8)
      hipLaunchKernelGGL((c3_score_kernel<64, 8>), grid, block, 0, st, V, X, S, qq, sigma);
    else
      hipLaunchKernelGGL((c3_score_kernel<64, 32>), grid, block, 0, st, V, X, S, qq, sigma);
  }
  return hipGetLastError();
}

static hipError_t c3_launch_su(const C3Desc& V, const C3Index& X, const C3State& Sin,
                               const float* sigma, int32_t* idx, const C3State& Sout, int sel,
                               int upd, hipStream_t st) {
  hipLaunchKernelGGL(c3_select_update_kernel, dim3((unsigned)V.n_units), dim3(C3_BIG), 0, st, V,
                     X, Sin, sigma, idx, Sout, sel, upd);
  return hipGetLastError();
}

static hipError_t c3_launch_gather(const C3Desc& V, const void* k, const void* v,
                                   const int32_t* idx, void* ko, void* vo, hipStream_t st) {
  const int rpb = (C3_T / (V.d / 8)) * 4;
  const int bpc = (V.kept_cap + rpb - 1) / rpb;
  C3_LAUNCH(V.d, c3_gather_kernel, dim3((unsigned)((int64_t)V.n_units * bpc)), dim3(C3_T), V, bpc,
            (const uint16_t*)k, (const uint16_t*)v, idx, (uint16_t*)ko, (uint16_t*)vo);
  return hipGetLastError();
}

static kvc_status c3_common(const kvc_c3_problem* prob, const kvc_c3_params* params, C3Desc* V,
                            kvc_c3_layout* L) {
  const kvc_status rs = c3_desc(prob, params, V);
  if (rs != KVC_OK) return rs;
  c3_layout(*V, L);
  return KVC_OK;
}

extern "C" kvc_status kvc_c3_score(const kvc_c3_problem* prob, const kvc_c3_params* params,
                                   const void* index, const void* state, const void* q,
                                   float* sigma, void* stream) {
  C3Desc V;
  kvc_c3_layout L;
  kvc_status rs = c3_common(prob, params, &V, &L);
  if (rs != KVC_OK) return rs;
  if (!index || !state || !q || !sigma || !c3_a256(index) || !c3_a256(state) || !c3_a16(q))
    return KVC_ERR_INVALID_ARG;
  return c3_hip(c3_launch_score(V, c3_index(L, index), c3_state(L, state), q, sigma,
                                (hipStream_t)stream));
}

extern "C" kvc_status kvc_c3_select(const kvc_c3_problem* prob, const kvc_c3_params* params,
                                    const void* index, const void* state, const float* sigma,
                                    int32_t* idx_out, void* stream) {
  C3Desc V;
  kvc_c3_layout L;
  kvc_status rs = c3_common(prob, params, &V, &L);
  if (rs != KVC_OK) return rs;
  if (!index || !state || !sigma || !idx_out || !c3_a256(index) || !c3_a256(state))
    return KVC_ERR_INVALID_ARG;
  const C3State S = c3_state(L, state);
  return c3_hip(c3_launch_su(V, c3_index(L, index), S, sigma, idx_out, S, 1, 0,
                             (hipStream_t)stream));
}

extern "C" kvc_status kvc_c3_update(const kvc_c3_problem* prob, const kvc_c3_params* params,
                                    const void* index, const void* state_in, const float* sigma,
                                    void* state_out, void* stream) {
  C3Desc V;
  kvc_c3_layout L;
  kvc_status rs = c3_common(prob, params, &V, &L);
  if (rs != KVC_OK) return rs;
  if (!index || !state_in || !sigma || !state_out || state_in == state_out || !c3_a256(index) ||
      !c3_a256(state_in) || !c3_a256(state_out))
    return KVC_ERR_INVALID_ARG;
  return c3_hip(c3_launch_su(V, c3_index(L, index), c3_state(L, state_in), sigma, nullptr,
                             c3_state(L, state_out), 0, 1, (hipStream_t)stream));
}

extern "C" kvc_status kvc_c3_gather(const kvc_c3_problem* prob, const kvc_c3_params* params,
                                    const void* k, const void* v, const int32_t* idx, void* k_out,
                                    void* v_out, void* stream) {
  C3Desc V;
  kvc_c3_layout L;
  kvc_status rs = c3_common(prob, params, &V, &L);
  if (rs != KVC_OK) return rs;
  if (!k || !v || !idx || !k_out || !v_out || !c3_a16(k) || !c3_a16(v) || !c3_a16(k_out) ||
      !c3_a16(v_out))
    return KVC_ERR_INVALID_ARG;
  return c3_hip(c3_launch_gather(V, k, v, idx, k_out, v_out, (hipStream_t)stream));
}

extern "C" kvc_status kvc_c3_step(const kvc_c3_problem* prob, const kvc_c3_params* params,
                                  const void* index, const void* state_in, void* state_out,
                                  const void* q, const void* k, const void* v, void* k_out,
                                  void* v_out, int32_t* idx_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  C3Desc V;
  kvc_c3_layout L;
  kvc_status rs = c3_common(prob, params, &V, &L);
  if (rs != KVC_OK) return rs;
  if (!index || !state_in || !state_out || state_in == state_out || !q || !k || !v || !k_out ||
      !v_out || !idx_out || !workspace)
    return KVC_ERR_INVALID_ARG;
  if (!c3_a256(index) || !c3_a256(state_in) || !c3_a256(state_out) || !c3_a256(workspace) ||
      !c3_a16(q) || !c3_a16(k) || !c3_a16(v) || !c3_a16(k_out) || !c3_a16(v_out))
    return KVC_ERR_INVALID_ARG;
  if (workspace_bytes < L.step_workspace_bytes) return KVC_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const C3Index X = c3_index(L, index);
  const C3State Si = c3_state(L, state_in), So = c3_state(L, state_out);
  float* sigma = (float*)workspace;
  hipError_t e = c3_launch_score(V, X, Si, q, sigma, st);
  if (e == hipSuccess) e = c3_launch_su(V, X, Si, sigma, idx_out, So, 1, 1, st);
  if (e == hipSuccess) e = c3_launch_gather(V, k, v, idx_out, k_out, v_out, st);
  return c3_hip(e);
}
