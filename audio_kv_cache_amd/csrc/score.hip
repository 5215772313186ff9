// score.hip -- observation-window importance scores (step 1) on MFMA.
//
// AudioKV article, section 1.2: the raw importance score of each audio
// position is the attention it receives from the observation window; with
// the softmax(q K^T / sqrt(d)) form written in the VoxZip digest's
// decayed-eviction equation, per unit (sequence, layer, KV head):
//   s[j] = 1/(G W) * sum_{g,q} exp(l[gq,j] - LSE[gq]),  l = q . k_j / sqrt(d),
// the softmax taken over all L audio keys.
//
// Two passes over K, both GEMM-shaped (Q [G W, d] x K^T [d, keys]):
//   stats  per query (max, sum of exp) of each 2048-key tile, folded per
//          unit into LSE (log2 units) by a small kernel after it
//   pool   recompute the logits, p = exp2(l*c - LSE2), sum over the G*W
//          queries, write s.
// Inside a lane's half row the head dimension is read in a permuted order
// (lane group g owns d in [g*d/G, (g+1)*d/G)); the same permutation is
// applied to Q and K, so the contraction is unchanged and every lane reads
// contiguous memory.
//
// bf16 inputs (v_mfma_f32_32x32x16_bf16, fp32 accumulate): query-stationary
// kernels -- each wave holds two 32-query blocks (and, pooling, their LSE)
// in registers while the workgroup streams the tile's keys through
// double-buffered LDS chunks; the MFMAs of one block are interleaved with
// the exponentials of the previous one.  fp32 inputs: key-stationary
// kernels (Q in LDS, each wave streams its own K rows into operand
// registers), widened to fp64 and contracted with v_mfma_f64_16x16x4f64,
// which keeps the logits exact to ~1e-15 so the 1e-5 fp32 tolerance is met
// with margin.
#include <type_traits>

#include "budget.h"
#include "kvc_internal.h"

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float floatx16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef double doublex4 __attribute__((__vector_size__(4 * sizeof(double))));

#define SCORE_THREADS 256
#define SCORE_WAVES 4

static constexpr float kLog2e = 1.4426950408889634f;

struct TF64 {
  using elem_t = float;
  using frag_t = double;
  using acc_t = doublex4;
  static constexpr int M = 16, KS = 4, E = 1, NOUT = 4, G = 4;
  static constexpr int MINB = 1;
  __device__ static acc_t zero() { return acc_t{}; }
  __device__ static acc_t mma(frag_t a, frag_t b, acc_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  // (measured: element i of lane l is row 4 i + l / 16)
  __device__ static int out_row(int i, int lane) { return 4 * i + (lane >> 4); }
  __device__ static float val(const acc_t& a, int i) { return (float)a[i]; }
  template <int NK>
  __device__ static void load(frag_t (&f)[NK], const elem_t* p) {
#pragma unroll
    for (int kk = 0; kk < NK; kk += 4) {
      const float4 raw = reinterpret_cast<const float4*>(p)[kk / 4];
      f[kk + 0] = raw.x;
      f[kk + 1] = raw.y;
      f[kk + 2] = raw.z;
      f[kk + 3] = raw.w;
    }
  }
};

// Per-instance tiling: RB key row blocks per wave step in the stats pass,
// CB key column blocks per wave step in the pooling pass.
template <class T, int D> struct Tiling;
template <> struct Tiling<TF64, 64> { static constexpr int RB = 1, CB = 1; };
template <> struct Tiling<TF64, 128> { static constexpr int RB = 1, CB = 1; };

// The dispatcher hands workgroup b of a launch to XCD b % 8, and each XCD
// has its own L2.  Renumber so that XCD x runs one contiguous range of tiles:
// the tiles of a unit then share one L2, which serves the unit's window
// queries after the first read instead of every XCD fetching them again.
// A bijection on [0, n) for any n.
__device__ inline int xcd_local_tile(int b, int n) {
  constexpr int kXcds = 8;
  const int x = b % kXcds, per = n / kXcds, rem = n % kXcds;
  return x * per + (x < rem ? x : rem) + b / kXcds;
}

// The same ranges, each walked from its last tile to its first: a pass that
// follows one in xcd_local_tile order starts on the tiles whose keys the
// other read last (still in the XCD's L2 and the memory-side cache).
__device__ inline int xcd_local_tile_rev(int b, int n) {
  constexpr int kXcds = 8;
  const int x = b % kXcds, per = n / kXcds, rem = n % kXcds;
  const int cnt = per + (x < rem ? 1 : 0);
  return x * per + (x < rem ? x : rem) + (cnt - 1 - b / kXcds);
}

struct TileInfo {
  int seq, u, l, h, t, tpu, L, keys, key0;
  bool tail;   // a tile of the L % 64 keys past the last multiple of 64 (kvc_score_tail_kernel)
};

__device__ inline TileInfo tile_info(const KvcDesc& Dsc, int tile) {
  TileInfo ti;
  int seq = 0;
  while (seq + 1 < Dsc.n_seq && Dsc.tile_base[seq + 1] <= tile) ++seq;
  ti.seq = seq;
  ti.L = Dsc.L[seq];
  ti.tpu = kvc_tiles_per_unit(ti.L);
  const int rel = tile - Dsc.tile_base[seq];
  const int uin = rel / ti.tpu;
  ti.t = rel - uin * ti.tpu;
  ti.u = seq * Dsc.upseq + uin;
  ti.l = uin / Dsc.n_heads;
  ti.h = uin - ti.l * Dsc.n_heads;
  const int L64 = ti.L & ~63;
  ti.tail = ti.t >= kvc_main_tiles(ti.L);
  ti.key0 = ti.tail ? L64 : ti.t * KVC_TILE_KEYS;
  ti.keys = ti.tail ? ti.L - L64 : min(KVC_TILE_KEYS, L64 - ti.key0);
  return ti;
}

// Copy the unit's G*W window queries into LDS rows of stride QS elements.
template <class T, int D, int QS>
__device__ inline void stage_q(typename T::elem_t* sQ, const typename T::elem_t* qg, int gw) {
  using elem_t = typename T::elem_t;
  constexpr int CPR = D * (int)sizeof(elem_t) / 16;  // 16-byte chunks per row
  for (int c = threadIdx.x; c < gw * CPR; c += SCORE_THREADS) {
    const int row = c / CPR, col = c - row * CPR;
    const uint4 v = reinterpret_cast<const uint4*>(qg + (size_t)row * D)[col];
    *reinterpret_cast<uint4*>(sQ + row * QS + col * (16 / (int)sizeof(elem_t))) = v;
  }
}

__device__ inline void merge_stat(float& m, float& z, float m2, float z2, float c) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  const float a = (m == -INFINITY) ? 0.f : z * __builtin_amdgcn_exp2f((m - mm) * c);
  const float b = (m2 == -INFINITY) ? 0.f : z2 * __builtin_amdgcn_exp2f((m2 - mm) * c);
  m = mm;
  z = a + b;
}

// ---------------------------------------------------------------------------
// Pass 1: per-query softmax statistics of each tile, folded per unit.
// ---------------------------------------------------------------------------
// NBC: number of 32/16-query blocks (G W / M) when fixed at compile time,
// 0 to read it from the descriptor (a runtime bound costs the compiler the
// freedom to overlap one block's exponentials with the next block's MFMAs).
template <class T, int D, int NBC>
__global__ __launch_bounds__(SCORE_THREADS, T::MINB) void kvc_score_stats_kernel(
    KvcDesc Dsc, int tile0, const typename T::elem_t* __restrict__ q,
    const typename T::elem_t* __restrict__ k, float2* __restrict__ partials) {
  using elem_t = typename T::elem_t;
  using frag_t = typename T::frag_t;
  using acc_t = typename T::acc_t;
  constexpr int M = T::M, G = T::G, NK = D / T::KS, RB = Tiling<T, D>::RB;
  constexpr int QS = D + 16 / (int)sizeof(elem_t);
  constexpr int MAXCB = NBC > 0 ? NBC : KVC_MAX_GW / M;
  constexpr int KW = RB * M;

  __shared__ __attribute__((aligned(16))) elem_t sQ[MAXCB * M * QS];
  __shared__ float2 sStat[SCORE_WAVES][MAXCB * M];

  const int tile = tile0 + xcd_local_tile((int)blockIdx.x, (int)gridDim.x);
  const TileInfo ti = tile_info(Dsc, tile);
  if (ti.tail) return;  // kvc_score_tail_kernel
  const int gw = NBC > 0 ? NBC * M : Dsc.gw;
  const int ncb = NBC > 0 ? NBC : gw / M;
  const float c = kLog2e / sqrtf((float)D);
  const elem_t* qg =
      q + kvc_q_offset(Dsc, ti.seq, ti.l, ti.h);
  const elem_t* ku = k + kvc_kv_offset(Dsc.ks, Dsc, ti.seq, ti.l, ti.h);
  stage_q<T, D, QS>(sQ, qg, gw);
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lrow = lane % M, lgrp = lane / M;
  float m[MAXCB], z[MAXCB];
#pragma unroll
  for (int cb = 0; cb < MAXCB; ++cb) {
    m[cb] = -INFINITY;
    z[cb] = 0.f;
  }

  const int ngroups = ti.keys / KW;
  // Software pipeline over query blocks: the MFMAs of block cb+1 are issued
  // before the exponentials of block cb, and a scheduling barrier per stage
  // keeps the compiler from hoisting further blocks (which would exhaust
  // the registers).
  auto mma_blk = [&](acc_t (&acc)[RB], const frag_t (&a)[RB][NK], int cb, int qoff) {
    frag_t b[NK];
    int qo = cb * M * QS + qoff;
    asm volatile("" : "+v"(qo));  // load this block's Q here, not earlier
    T::template load<NK>(b, sQ + qo);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      acc[rb] = T::zero();
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) acc[rb] = T::mma(a[rb][kk], b[kk], acc[rb]);
    }
  };
  auto stat_blk = [&](const acc_t (&acc)[RB], float& mref, float& zref) {
    float mloc = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < T::NOUT; ++i) mloc = fmaxf(mloc, T::val(acc[rb], i));
    const float mnew = fmaxf(mref, mloc);
    const float nmc = -mnew * c;
    float zz = (mref == -INFINITY) ? 0.f : zref * __builtin_amdgcn_exp2f((mref - mnew) * c);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < T::NOUT; ++i) zz += __builtin_amdgcn_exp2f(fmaf(T::val(acc[rb], i), c, nmc));
    mref = mnew;
    zref = zz;
  };
  auto load_keys = [&](frag_t (&a)[RB][NK], int grp) {
    const int kb = ti.key0 + grp * KW;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      T::template load<NK>(a[rb], ku + (int64_t)(kb + rb * M + lrow) * Dsc.ks[2] + lgrp * (D / G));
  };
  auto group = [&](const frag_t (&a)[RB][NK]) {
    // Q fragments do not change between key groups; an opaque lane index
    // keeps the compiler from hoisting them all out of the loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int qoff = (ln % M) * QS + (ln / M) * (D / G);
    if constexpr (NBC > 0) {
      acc_t X[RB], Y[RB];
      mma_blk(X, a, 0, qoff);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int cb = 0; cb < NBC; ++cb) {
        if (cb + 1 < NBC) mma_blk((cb & 1) ? X : Y, a, cb + 1, qoff);
        stat_blk((cb & 1) ? Y : X, m[cb], z[cb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < MAXCB; ++cb) {
        if (cb < ncb) {
          acc_t X[RB];
          mma_blk(X, a, cb, qoff);
          stat_blk(X, m[cb], z[cb]);
        }
      }
    }
  };
  // Two register buffers: the next group's keys load while this one computes.
  frag_t a0[RB][NK], a1[RB][NK];
  if (wave < ngroups) load_keys(a0, wave);
  for (int grp = wave; grp < ngroups; grp += 2 * SCORE_WAVES) {
    const bool more = grp + SCORE_WAVES < ngroups;
    if (more) load_keys(a1, grp + SCORE_WAVES);
    group(a0);
    if (!more) break;
    if (grp + 2 * SCORE_WAVES < ngroups) load_keys(a0, grp + 2 * SCORE_WAVES);
    group(a1);
  }

  // Fold the lane groups holding the same query, then the waves.
#pragma unroll
  for (int cb = 0; cb < MAXCB; ++cb) {
    if (cb < ncb) {
#pragma unroll
      for (int o = M; o < 64; o <<= 1) {
        const float m2 = __shfl_xor(m[cb], o);
        const float z2 = __shfl_xor(z[cb], o);
        merge_stat(m[cb], z[cb], m2, z2, c);
      }
      if (lgrp == 0) sStat[wave][cb * M + lrow] = make_float2(m[cb], z[cb]);
    }
  }
  __syncthreads();
  if (threadIdx.x < gw) {
    float mm = -INFINITY, zz = 0.f;
#pragma unroll
    for (int w = 0; w < SCORE_WAVES; ++w) merge_stat(mm, zz, sStat[w][threadIdx.x].x, sStat[w][threadIdx.x].y, c);
    partials[(size_t)tile * gw + threadIdx.x] = make_float2(mm, zz);
  }
}

// Fold the per-tile statistics of each unit into LSE (log2 units): one
// workgroup per unit, one thread per window query.
__global__ __launch_bounds__(KVC_MAX_GW) void kvc_score_lse_kernel(KvcDesc Dsc, int unit0, float c,
                                                                   const float2* __restrict__ partials,
                                                                   float* __restrict__ lse2) {
  const int u = unit0 + (int)blockIdx.x;
  const int seq = u / Dsc.upseq;
  const int tpu = kvc_tiles_per_unit(Dsc.L[seq]);
  const int tile0 = Dsc.tile_base[seq] + (u - seq * Dsc.upseq) * tpu;
  const int gw = Dsc.gw;
  if ((int)threadIdx.x >= gw) return;
  // Tiles merged in order; eight tiles' loads in flight at a time.
  const float2* pp = partials + (size_t)tile0 * gw + threadIdx.x;
  float mm = -INFINITY, zz = 0.f;
  int t = 0;
  for (; t + 8 <= tpu; t += 8) {
    float2 p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = pp[(size_t)(t + i) * gw];
#pragma unroll
    for (int i = 0; i < 8; ++i) merge_stat(mm, zz, p[i].x, p[i].y, c);
  }
  for (; t < tpu; ++t) {
    const float2 p = pp[(size_t)t * gw];
    merge_stat(mm, zz, p.x, p.y, c);
  }
  lse2[(size_t)u * gw + threadIdx.x] = mm * c + __builtin_amdgcn_logf(zz);
}

// ---------------------------------------------------------------------------
// Pass 2: probabilities pooled over the window queries and the GQA group.
// ---------------------------------------------------------------------------
template <class T, int D, int NBC, int CBT = Tiling<T, D>::CB, bool PIPE = true>
__global__ __launch_bounds__(SCORE_THREADS, T::MINB) void kvc_score_pool_kernel(
    KvcDesc Dsc, int tile0, const typename T::elem_t* __restrict__ q,
    const typename T::elem_t* __restrict__ k, const float* __restrict__ lse2,
    float* __restrict__ s) {
  using elem_t = typename T::elem_t;
  using frag_t = typename T::frag_t;
  using acc_t = typename T::acc_t;
  constexpr int M = T::M, G = T::G, NK = D / T::KS, CB = CBT;
  constexpr int QS = D + 16 / (int)sizeof(elem_t);
  constexpr int MAXRB = NBC > 0 ? NBC : KVC_MAX_GW / M;
  constexpr int KW = CB * M;

  __shared__ __attribute__((aligned(16))) elem_t sQ[MAXRB * M * QS];
  __shared__ float sL[MAXRB * M];

  const int tile = tile0 + xcd_local_tile_rev((int)blockIdx.x, (int)gridDim.x);
  const TileInfo ti = tile_info(Dsc, tile);
  if (ti.tail) return;  // kvc_score_tail_kernel
  const int gw = NBC > 0 ? NBC * M : Dsc.gw;
  const int nrb = NBC > 0 ? NBC : gw / M;
  const float c = kLog2e / sqrtf((float)D);
  const float inv_gw = 1.0f / (float)gw;
  const elem_t* qg =
      q + kvc_q_offset(Dsc, ti.seq, ti.l, ti.h);
  const elem_t* ku = k + kvc_kv_offset(Dsc.ks, Dsc, ti.seq, ti.l, ti.h);
  stage_q<T, D, QS>(sQ, qg, gw);
  if (threadIdx.x < gw) sL[threadIdx.x] = lse2[(size_t)ti.u * gw + threadIdx.x];
  __syncthreads();

  float* srow = s + Dsc.srow_base[ti.seq] + (int64_t)(ti.u - ti.seq * Dsc.upseq) * ti.L;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lrow = lane % M, lgrp = lane / M;
  const int ngroups = ti.keys / KW;
  // Same two-stage pipeline as the statistics pass, over query row blocks.
  auto mma_blk = [&](acc_t (&acc)[CB], const frag_t (&b)[CB][NK], int rb, int qoff) {
    frag_t a[NK];
    int qo = rb * M * QS + qoff;
    asm volatile("" : "+v"(qo));  // load this block's Q here, not earlier
    T::template load<NK>(a, sQ + qo);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      acc[cb] = T::zero();
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) acc[cb] = T::mma(a[kk], b[cb][kk], acc[cb]);
    }
  };
  auto pool_blk = [&](const acc_t (&acc)[CB], float (&acc_s)[CB], int rb, int ln) {
    float nl[T::NOUT];
    int lb = rb * M;
    asm volatile("" : "+v"(lb));  // load this block's LSE here, not earlier
#pragma unroll
    for (int i = 0; i < T::NOUT; ++i) nl[i] = -sL[lb + T::out_row(i, ln)];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < T::NOUT; ++i) sum += __builtin_amdgcn_exp2f(fmaf(T::val(acc[cb], i), c, nl[i]));
      acc_s[cb] += sum;
    }
  };
  auto load_keys = [&](frag_t (&b)[CB][NK], int grp) {
    const int kb = ti.key0 + grp * KW;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
      T::template load<NK>(b[cb], ku + (int64_t)(kb + cb * M + lrow) * Dsc.ks[2] + lgrp * (D / G));
  };
  auto group = [&](const frag_t (&b)[CB][NK], int grp) {
    const int kb = ti.key0 + grp * KW;
    // The Q fragments and LSE values of a query block do not change from one
    // key group to the next; an opaque lane index keeps the compiler from
    // hoisting all of them out of the loop (they would not fit in registers).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int qoff = (ln % M) * QS + (ln / M) * (D / G);
    float acc_s[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc_s[cb] = 0.f;
    if constexpr (NBC > 0 && PIPE) {
      acc_t X[CB], Y[CB];
      mma_blk(X, b, 0, qoff);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < NBC; ++rb) {
        if (rb + 1 < NBC) mma_blk((rb & 1) ? X : Y, b, rb + 1, qoff);
        pool_blk((rb & 1) ? Y : X, acc_s, rb, ln);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Max pooling over query heads: each head's W rows are whole blocks
      // (W a multiple of 32); at a head's last block its sum is completed
      // over the lanes holding the key and folded into the running maximum.
      float hmax[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) hmax[cb] = 0.f;
#pragma unroll
      for (int rb = 0; rb < MAXRB; ++rb) {
        if (rb < nrb) {
          acc_t X[CB];
          mma_blk(X, b, rb, qoff);
          pool_blk(X, acc_s, rb, ln);
          if constexpr (!PIPE) __builtin_amdgcn_sched_barrier(0);
          if (Dsc.score_max && ((rb + 1) * M) % Dsc.nwin == 0) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
              float v = acc_s[cb];
#pragma unroll
              for (int o = M; o < 64; o <<= 1) v += __shfl_xor(v, o);
              hmax[cb] = fmaxf(hmax[cb], v);
              acc_s[cb] = 0.f;
            }
          }
        }
      }
      if (Dsc.score_max) {
        const float inv_w = 1.0f / (float)Dsc.nwin;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          if (lgrp == 0) srow[kb + cb * M + lrow] = hmax[cb] * inv_w;
        return;
      }
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float v = acc_s[cb];
#pragma unroll
      for (int o = M; o < 64; o <<= 1) v += __shfl_xor(v, o);
      if (lgrp == 0) srow[kb + cb * M + lrow] = v * inv_gw;
    }
  };
  frag_t b0[CB][NK], b1[CB][NK];
  if (wave < ngroups) load_keys(b0, wave);
  for (int grp = wave; grp < ngroups; grp += 2 * SCORE_WAVES) {
    const bool more = grp + SCORE_WAVES < ngroups;
    if (more) load_keys(b1, grp + SCORE_WAVES);
    group(b0, grp);
    if (!more) break;
    if (grp + 2 * SCORE_WAVES < ngroups) load_keys(b0, grp + 2 * SCORE_WAVES);
    group(b1, grp + SCORE_WAVES);
  }
}

// ---------------------------------------------------------------------------
// bf16, query-stationary form of both passes
// ---------------------------------------------------------------------------
// Each wave keeps two 32-query blocks of the unit in registers (A/B operand
// fragments, and in the pooling pass the LSE of every output row it holds)
// and the workgroup streams the tile's keys through LDS in chunks of 64 rows,
// double-buffered: the next chunk's global loads are in flight while the
// current one is consumed, one barrier per chunk.  Per MFMA this reads a
// quarter of the LDS bytes of the key-stationary form above (which re-reads
// every query block and its LSE values from LDS for each 32 keys), and no LSE
// value is read from LDS at all.  A K row sits in LDS with a 16-byte pad so
// that the 32 rows read by one fragment load fall in distinct bank groups.
template <int D>
struct QsCfg {
  static constexpr int CHUNK = 64;                   // keys per LDS chunk
  static constexpr int ROWB = D * 2;                 // bytes per bf16 K row
  static constexpr int RS = ROWB + 16;               // padded LDS row stride
  static constexpr int NK = D / 16;                  // MFMA k-steps
  static constexpr int PIECES = CHUNK * ROWB / 16;   // 16-byte pieces per chunk
};

// Waves of a query-stationary workgroup: two query blocks each.
template <int NBC>
struct QsWaves {
  static constexpr int NW = (NBC + 1) / 2;
  static constexpr int NT = 64 * NW;
  static constexpr int MINB = 8 / NW;                // two waves per SIMD
};

// Loads of one chunk (rows key0 .. key0+63 of the unit) into registers:
// thread t takes pieces t, t + NT, ... (consecutive threads, consecutive
// 16-byte pieces of a row).  Past the last piece a thread reloads it, so
// every register is written on every path and the array is never demoted
// to scratch memory.  The pieces' byte offsets within a chunk are computed
// once per tile (32-bit; the host bounds the token stride), and each chunk
// only moves the uniform base pointer, so the loads need no 64-bit vector
// address arithmetic.
typedef unsigned int qs_u32x4 __attribute__((ext_vector_type(4)));

template <int D, int NT>
struct QsLoader {
  static constexpr int PPR = QsCfg<D>::ROWB / 16;
  static constexpr int PER = (QsCfg<D>::PIECES + NT - 1) / NT;
  uint32_t off[PER];
  __device__ explicit QsLoader(int64_t kstride) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int p = min((int)threadIdx.x + j * NT, QsCfg<D>::PIECES - 1);
      const int row = p / PPR, pc = p - row * PPR;
      off[j] = (uint32_t)(row * kstride * 2 + pc * 16);
    }
  }
  __device__ void load(qs_u32x4 (&r)[PER], const uint16_t* ku, int64_t kstride, int key0) const {
    const char* base = reinterpret_cast<const char*>(ku + (int64_t)key0 * kstride);
#pragma unroll
    for (int j = 0; j < PER; ++j) r[j] = *reinterpret_cast<const qs_u32x4*>(base + off[j]);
  }
};

template <int D, int NT>
__device__ inline void qs_kstore(const qs_u32x4 (&r)[(QsCfg<D>::PIECES + NT - 1) / NT], char* buf) {
  constexpr int PPR = QsCfg<D>::ROWB / 16, PER = (QsCfg<D>::PIECES + NT - 1) / NT;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int p = (int)threadIdx.x + j * NT;
    if (QsCfg<D>::PIECES % NT == 0 || p < QsCfg<D>::PIECES) {
      const int row = p / PPR, pc = p - row * PPR;
      *reinterpret_cast<qs_u32x4*>(buf + row * QsCfg<D>::RS + pc * 16) = r[j];
    }
  }
}

// Fragment of 32 K rows (block kb of the chunk in LDS) for the lane: row
// kb*32 + lane%32, the lane half's permuted head-dimension range.
template <int D>
__device__ inline void qs_kfrag(bf16x8 (&f)[QsCfg<D>::NK], const char* buf, int kb, int lane) {
  const char* p = buf + (kb * 32 + (lane & 31)) * QsCfg<D>::RS + (lane >> 5) * D;
#pragma unroll
  for (int kk = 0; kk < QsCfg<D>::NK; ++kk) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p + kk * 16);
    __builtin_memcpy(&f[kk], &raw, 16);
  }
}

// The lane's fragments of query block qb (row qb*32 + lane%32, same
// permutation); zero past the unit's G*W queries.
template <int D>
__device__ inline void qs_qfrag(bf16x8 (&f)[QsCfg<D>::NK], const uint16_t* qg, int qb, int gw,
                                int lane) {
  const int row = qb * 32 + (lane & 31);
  const uint16_t* p = qg + (size_t)(row < gw ? row : 0) * D + (lane >> 5) * (D / 2);
#pragma unroll
  for (int kk = 0; kk < QsCfg<D>::NK; ++kk) {
    uint4 raw = row < gw ? reinterpret_cast<const uint4*>(p)[kk] : make_uint4(0, 0, 0, 0);
    __builtin_memcpy(&f[kk], &raw, 16);
  }
}

// Interleave the 8 MFMAs of one block with the VALU work of the previous
// block: 1 MFMA, then `n` VALU instructions, eight times.  A wave issues in
// order, so without this the exponentials of a block wait behind the next
// block's whole dependent MFMA chain.
#define QS_INTERLEAVE(n)                                   \
  do {                                                     \
    _Pragma("unroll") for (int _i = 0; _i < 8; ++_i) {     \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   \
      __builtin_amdgcn_sched_group_barrier(0x002, n, 0);   \
    }                                                      \
  } while (0)

// MAXP: max pooling over query heads (W a multiple of 32, so every 32-query
// block belongs to one head): the per-block sums are kept apart in LDS and
// combined per head, then maximised, at the end of the tile.  Otherwise the
// wave's two blocks are summed in-lane and the waves summed at the end.
template <int D, int NBC, bool MAXP>
__global__ __launch_bounds__(QsWaves<NBC>::NT, QsWaves<NBC>::MINB) void kvc_score_pool_qs_kernel(
    KvcDesc Dsc, int tile0, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const float* __restrict__ lse2, float* __restrict__ s) {
  using C = QsCfg<D>;
  constexpr int NW = QsWaves<NBC>::NW, NT = QsWaves<NBC>::NT, NK = C::NK;
  constexpr int NROWS = MAXP ? 2 * NW : NW;
  __shared__ __attribute__((aligned(16))) char sK[2][C::CHUNK * C::RS];
  __shared__ float sRed[NROWS][KVC_TILE_KEYS];
  const int tile = tile0 + xcd_local_tile_rev((int)blockIdx.x, (int)gridDim.x);
  const TileInfo ti = tile_info(Dsc, tile);
  if (ti.tail) return;  // kvc_score_tail_kernel
  const int gw = NBC * 32;
  const float c = kLog2e / sqrtf((float)D);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool two = 2 * wave + 1 < NBC;
  const uint16_t* qg = q + kvc_q_offset(Dsc, ti.seq, ti.l, ti.h);
  const uint16_t* ku = k + kvc_kv_offset(Dsc.ks, Dsc, ti.seq, ti.l, ti.h);

  // A operand (rows = queries) and minus the LSE of each output row the lane
  // holds: element i of the 32x32 block is row (i/4)*8 + (lane/32)*4 + i%4.
  // A wave with a single query block repeats it as its second block and
  // gives that copy -inf, so its terms are exactly zero.
  bf16x8 qf0[NK], qf1[NK];
  qs_qfrag<D>(qf0, qg, 2 * wave, gw, lane);
  qs_qfrag<D>(qf1, qg, two ? 2 * wave + 1 : 2 * wave, gw, lane);
  float nl0[16], nl1[16];
  {
    const float* lu = lse2 + (size_t)ti.u * gw;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      nl0[i] = -lu[(2 * wave) * 32 + row];
      nl1[i] = two ? -lu[(2 * wave + 1) * 32 + row] : -INFINITY;
    }
  }
  auto mma = [&](floatx16& acc, const bf16x8 (&qf)[NK], const bf16x8 (&kf)[NK]) {
    acc = floatx16{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[kk], kf[kk], acc, 0, 0, 0);
  };
  // Pairwise sum of the 16 terms: a serial chain of adds would leave the
  // VALU waiting on each add's latency.
  auto pool = [&](const floatx16& acc, const float (&nl)[16]) {
    float e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(acc[i], c, nl[i]));
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) e[i] = e[i] + e[i + w];
    return e[0];
  };
  // Both lane halves hold the same sum after the exchange and both write it
  // (same value, same address): no lane mask, no branch in the loop body.
  auto flush1 = [&](float sum, int row, int key) {
    sum += __shfl_xor(sum, 32);
    sRed[row][key + (lane & 31)] = sum;
  };
  // sums of the wave's blocks 0 and 1 for the 32 keys from `key` (tile-relative)
  auto flush = [&](float s_b0, float s_b1, int key) {
    if constexpr (MAXP) {
      flush1(s_b0, 2 * wave, key);
      flush1(s_b1, 2 * wave + 1, key);
    } else {
      flush1(s_b0 + s_b1, wave, key);
    }
  };

  // The loop body is branch-free so that the scheduling groups hold: the
  // last chunk reloads and restages itself into the idle buffer.
  const int nch = ti.keys / C::CHUNK;
  const QsLoader<D, NT> kl(Dsc.ks[2]);
  qs_u32x4 kr[(C::PIECES + NT - 1) / NT];
  kl.load(kr, ku, Dsc.ks[2], ti.key0);
  qs_kstore<D, NT>(kr, sK[0]);
  __syncthreads();
  floatx16 X, Y;          // X: query block 0, Y: query block 1 of the current key block
  bf16x8 kf0[NK], kf1[NK];
  float s0 = 0.f;         // pooled sum of the current key block (block 0 part)
  kl.load(kr, ku, Dsc.ks[2], ti.key0 + min(1, nch - 1) * C::CHUNK);
  qs_kfrag<D>(kf0, sK[0], 0, lane);
  mma(X, qf0, kf0);
  for (int ch = 0;;) {
    const char* buf = sK[ch & 1];
    // [B] keys 0-31 x block 1, beside keys 0-31 x block 0
    qs_kfrag<D>(kf1, buf, 1, lane);
    mma(Y, qf1, kf0);
    s0 = pool(X, nl0);
    QS_INTERLEAVE(6);
    // [C] keys 32-63 x block 0, beside keys 0-31 x block 1
    mma(X, qf0, kf1);
    flush(s0, pool(Y, nl1), ch * C::CHUNK);
    QS_INTERLEAVE(6);
    // [D] keys 32-63 x block 1, beside keys 32-63 x block 0
    mma(Y, qf1, kf1);
    s0 = pool(X, nl0);
    QS_INTERLEAVE(6);
    qs_kstore<D, NT>(kr, sK[(ch + 1) & 1]);
    __syncthreads();
    if (++ch == nch) break;
    kl.load(kr, ku, Dsc.ks[2], ti.key0 + min(ch + 1, nch - 1) * C::CHUNK);
    // [A] keys 0-31 of the new chunk x block 0, beside the last block of
    // the previous chunk
    qs_kfrag<D>(kf0, sK[ch & 1], 0, lane);
    const floatx16 Yp = Y;
    mma(X, qf0, kf0);
    flush(s0, pool(Yp, nl1), (ch - 1) * C::CHUNK + 32);
    QS_INTERLEAVE(6);
  }
  flush(s0, pool(Y, nl1), (nch - 1) * C::CHUNK + 32);
  __syncthreads();
  // Sum the waves' partial pools for every key of the tile.
  float* srow = s + Dsc.srow_base[ti.seq] + (int64_t)(ti.u - ti.seq * Dsc.upseq) * ti.L;
  if constexpr (MAXP) {
    const int bph = Dsc.nwin / 32;             // blocks per head
    const float inv_w = 1.0f / (float)Dsc.nwin;
    for (int j = threadIdx.x; j < ti.keys; j += NT) {
      float best = 0.f;
      for (int b0 = 0; b0 < NBC; b0 += bph) {
        float v = 0.f;
        for (int b = b0; b < b0 + bph; ++b) v += sRed[b][j];
        best = fmaxf(best, v);
      }
      srow[ti.key0 + j] = best * inv_w;
    }
  } else {
    const float inv_gw = 1.0f / (float)gw;
    for (int j = threadIdx.x; j < ti.keys; j += NT) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) v += sRed[w][j];
      srow[ti.key0 + j] = v * inv_gw;
    }
  }
}

// Statistics pass.  Fast path: each lane takes its reference maximum per
// query block from the tile's first 32 keys (one extra MFMA block) and sums
// exp2(l*c - m*c) over the whole tile with that fixed reference: no running
// maximum, no rescaling, the same VALU work per key as the pooling pass.
// Terms below the reference by more than the fp32 range underflow, which
// loses nothing next to the reference term itself (>= 1).  A sum can only go
// wrong by overflowing, when a later key's logit exceeds the reference by
// more than about 127 / c; the workgroup then recomputes the tile with the
// exact online maximum.
//
// BUDGET: the first nbw workgroups (a multiple of 8, so that every tile
// workgroup keeps its place on the XCDs) compute the budget pools instead
// (step 3 needs only the head scores), sharing the workgroup's LDS with the
// key chunks: the budget is then done within this pass instead of before it.
template <int D, int NBC, bool BUDGET = false>
__global__ __launch_bounds__(QsWaves<NBC>::NT, QsWaves<NBC>::MINB) void kvc_score_stats_qs_kernel(
    KvcDesc Dsc, int tile0, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    float2* __restrict__ partials, KvcBudgetArgs B, int nbw) {
  using C = QsCfg<D>;
  constexpr int NT = QsWaves<NBC>::NT, NK = C::NK;
  constexpr int KBYTES = 2 * C::CHUNK * C::RS;
  constexpr int SMEM =
      BUDGET && (int)sizeof(KvcBudgetSmem) > KBYTES ? (int)sizeof(KvcBudgetSmem) : KBYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  char(*sK)[C::CHUNK * C::RS] = reinterpret_cast<char(*)[C::CHUNK * C::RS]>(smem);
  __shared__ int sRedo;
  int bid = (int)blockIdx.x, nblk = (int)gridDim.x;
  if constexpr (BUDGET) {
    if (bid < nbw) {
      if (bid < Dsc.n_seq * (Dsc.upseq / Dsc.pool_size))
        kvc_budget_pool<NT>(Dsc, B.S, B.budgets, B.offsets, bid,
                            *reinterpret_cast<KvcBudgetSmem*>(smem));
      return;
    }
    bid -= nbw;
    nblk -= nbw;
  }
  const int tile = tile0 + xcd_local_tile(bid, nblk);
  const TileInfo ti = tile_info(Dsc, tile);
  if (ti.tail) return;  // kvc_score_tail_kernel
  const int gw = NBC * 32;
  const float c = kLog2e / sqrtf((float)D);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool two = 2 * wave + 1 < NBC;
  const uint16_t* qg = q + kvc_q_offset(Dsc, ti.seq, ti.l, ti.h);
  const uint16_t* ku = k + kvc_kv_offset(Dsc.ks, Dsc, ti.seq, ti.l, ti.h);

  // B operand (columns = queries): the wave's two query blocks (a wave with
  // one block repeats it and discards the copy's statistics).
  bf16x8 qf0[NK], qf1[NK];
  qs_qfrag<D>(qf0, qg, 2 * wave, gw, lane);
  qs_qfrag<D>(qf1, qg, two ? 2 * wave + 1 : 2 * wave, gw, lane);
  auto mma = [&](floatx16& acc, const bf16x8 (&kf)[NK], const bf16x8 (&qf)[NK]) {
    acc = floatx16{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[kk], acc, 0, 0, 0);
  };
  auto bmax = [&](const floatx16& acc) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = fmaxf(acc[i], acc[i + 8]);
#pragma unroll
    for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) t[i] = fmaxf(t[i], t[i + w]);
    return t[0];
  };
  auto esum = [&](const floatx16& acc, float nmc) {
    float e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(acc[i], c, nmc));
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int i = 0; i < w; ++i) e[i] = e[i] + e[i + w];
    return e[0];
  };

  const QsLoader<D, NT> kl(Dsc.ks[2]);
  const int nch = ti.keys / C::CHUNK;
  float m0, z0, m1, z1;
  // One pass over the tile through the LDS pipeline.  EXACT: online maximum
  // (rescaling z when it grows); otherwise the fixed references m0, m1.
  auto run = [&](auto exact_tag) {
    constexpr bool EXACT = decltype(exact_tag)::value;
    float n0 = -m0 * c, n1 = -m1 * c;
    auto stat = [&](const floatx16& acc, float& m, float& z, float& nmc) {
      if constexpr (EXACT) {
        const float mn = fmaxf(m, bmax(acc));
        const float nn = -mn * c;
        z = z * __builtin_amdgcn_exp2f((m - mn) * c) + esum(acc, nn);  // m = -inf: adds to 0
        m = mn;
        nmc = nn;
      } else {
        z += esum(acc, nmc);
      }
    };
    qs_u32x4 kr[(C::PIECES + NT - 1) / NT];
    kl.load(kr, ku, Dsc.ks[2], ti.key0);
    qs_kstore<D, NT>(kr, sK[0]);
    __syncthreads();
    floatx16 X, Y;
    bf16x8 kf0[NK], kf1[NK];
    kl.load(kr, ku, Dsc.ks[2], ti.key0 + min(1, nch - 1) * C::CHUNK);
    qs_kfrag<D>(kf0, sK[0], 0, lane);
    if constexpr (!EXACT) {
      // references from the tile's first 32 keys
      floatx16 R;
      mma(R, kf0, qf0);
      m0 = bmax(R);
      mma(R, kf0, qf1);
      m1 = bmax(R);
      n0 = -m0 * c;
      n1 = -m1 * c;
    }
    mma(X, kf0, qf0);
    for (int ch = 0;;) {
      const char* buf = sK[ch & 1];
      qs_kfrag<D>(kf1, buf, 1, lane);
      mma(Y, kf0, qf1);
      stat(X, m0, z0, n0);
      QS_INTERLEAVE(7);
      mma(X, kf1, qf0);
      stat(Y, m1, z1, n1);
      QS_INTERLEAVE(7);
      mma(Y, kf1, qf1);
      stat(X, m0, z0, n0);
      QS_INTERLEAVE(7);
      qs_kstore<D, NT>(kr, sK[(ch + 1) & 1]);
      __syncthreads();
      if (++ch == nch) break;
      kl.load(kr, ku, Dsc.ks[2], ti.key0 + min(ch + 1, nch - 1) * C::CHUNK);
      qs_kfrag<D>(kf0, sK[ch & 1], 0, lane);
      const floatx16 Yp = Y;
      mma(X, kf0, qf0);
      stat(Yp, m1, z1, n1);
      QS_INTERLEAVE(7);
    }
    stat(Y, m1, z1, n1);
  };

  z0 = z1 = 0.f;
  if (threadIdx.x == 0) sRedo = 0;
  run(std::integral_constant<bool, false>{});
  // An overflowed sum in any wave sends the whole workgroup (its barriers
  // must match) through the exact pass.
  if (!(z0 < INFINITY) || !(z1 < INFINITY)) sRedo = 1;
  __syncthreads();
  if (sRedo) {
    m0 = m1 = -INFINITY;
    z0 = z1 = 0.f;
    run(std::integral_constant<bool, true>{});
  }
  // The other lane half holds the other 16 keys of each 32-key block.
  {
    float m2 = __shfl_xor(m0, 32), z2 = __shfl_xor(z0, 32);
    merge_stat(m0, z0, m2, z2, c);
    m2 = __shfl_xor(m1, 32);
    z2 = __shfl_xor(z1, 32);
    merge_stat(m1, z1, m2, z2, c);
  }
  if (lane < 32) {
    partials[(size_t)tile * gw + (2 * wave) * 32 + lane] = make_float2(m0, z0);
    if (two) partials[(size_t)tile * gw + (2 * wave + 1) * 32 + lane] = make_float2(m1, z1);
  }
}

// The L % 64 keys of each unit past its last multiple of 64, split into
// KVC_TAIL_SPLITS ranges of at most KVC_TAIL_KEYS keys, one workgroup per
// (unit, range) and one thread per window query.  Mode 1: the statistics
// pass's (max, sum) per query over the range (a tile's partial, folded with
// the others); mode 2: the range's pooled scores.  Plain fp32 dot products,
// each query row read once and the keys broadcast from LDS.
template <class E, int D>
__global__ __launch_bounds__(KVC_MAX_GW) void kvc_score_tail_kernel(KvcDesc Dsc, int unit0,
                                                                    int mode,
                                                                    const E* __restrict__ q,
                                                                    const E* __restrict__ k,
                                                                    const float* __restrict__ lse2,
                                                                    float2* __restrict__ partials,
                                                                    float* __restrict__ s) {
  constexpr int NK = KVC_TAIL_KEYS;
  __shared__ __attribute__((aligned(16))) float sK[NK][D];
  __shared__ float sP[KVC_MAX_GW][NK + 1];
  __shared__ float sH[KVC_MAX_GW][NK];
  const int u = unit0 + (int)blockIdx.x / KVC_TAIL_SPLITS;
  const int split = (int)blockIdx.x % KVC_TAIL_SPLITS;
  const int seq = u / Dsc.upseq, within = u - seq * Dsc.upseq;
  const int l = within / Dsc.n_heads, h = within - l * Dsc.n_heads;
  const int L = Dsc.L[seq], L64 = L & ~63, nt = L - L64;
  if (nt == 0) return;   // (a launch over several sequences: this one has no tail tiles)
  const int per = (nt + KVC_TAIL_SPLITS - 1) / KVC_TAIL_SPLITS;
  const int j0 = L64 + split * per;
  const int nk = max(0, min(per, L - j0));
  const int gw = Dsc.gw;
  const float c = kLog2e / sqrtf((float)D);
  auto val = [](E x) -> float {
    if constexpr (sizeof(E) == 2) return __uint_as_float((uint32_t)x << 16);
    else return (float)x;
  };
  const E* qg = q + kvc_q_offset(Dsc, seq, l, h);
  const E* ku = k + kvc_kv_offset(Dsc.ks, Dsc, seq, l, h);
  // fp32 inputs: the range's key rows into LDS, a 16-byte piece per thread
  // (the bf16 path reads them as MFMA operands instead).
  constexpr int EP = 16 / (int)sizeof(E), PPR = D / EP;   // elements per piece, pieces per row
  for (int i = threadIdx.x; sizeof(E) != 2 && i < nk * PPR; i += KVC_MAX_GW) {
    const int j = i / PPR, pc = i - j * PPR;
    const uint4 raw = *reinterpret_cast<const uint4*>(ku + (int64_t)(j0 + j) * Dsc.ks[2] + pc * EP);
    E ev[EP];
    __builtin_memcpy(ev, &raw, 16);
#pragma unroll
    for (int e = 0; e < EP; ++e) sK[j][pc * EP + e] = val(ev[e]);
  }
  __syncthreads();
  const int r = threadIdx.x;
  float acc[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) acc[j] = 0.f;
  if constexpr (sizeof(E) == 2) {
    // bf16: the range's logits on v_mfma_f32_16x16x32_bf16, the window
    // queries as rows (16 per tile; wave w takes tiles w, w + 4, ...) and
    // the range's keys as the 16 columns, into LDS; then each thread reads
    // its query's row.  Lane l supplies row/column l % 16 and, at k-step
    // ks, head dims ks*32 + (l/16)*8 .. +7 of both operands.  Keys past the
    // range read its first key (their columns are never read back).
    typedef __bf16 tb_bf16x8 __attribute__((ext_vector_type(8)));
    typedef float tb_f4 __attribute__((ext_vector_type(4)));
    constexpr int KS = D / 32;
    __shared__ float sL[KVC_MAX_GW][NK + 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
    if (nk > 0) {
      tb_bf16x8 kb[KS];
      const E* kr = ku + (int64_t)(j0 + (col < nk ? col : 0)) * Dsc.ks[2] + grp * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 raw = *reinterpret_cast<const uint4*>(kr + ks * 32);
        __builtin_memcpy(&kb[ks], &raw, 16);
      }
      for (int qt = wave; qt * 16 < gw; qt += KVC_MAX_GW / 64) {
        const int qr = min(qt * 16 + col, gw - 1);
        const E* qp = qg + (size_t)qr * D + grp * 8;
        tb_f4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 raw = *reinterpret_cast<const uint4*>(qp + ks * 32);
          tb_bf16x8 qa;
          __builtin_memcpy(&qa, &raw, 16);
          t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kb[ks], t, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = qt * 16 + grp * 4 + i;
          if (q < gw) sL[q][col] = t[i];
        }
      }
    }
    __syncthreads();
    if (r < gw) {
#pragma unroll
      for (int j = 0; j < NK; ++j)
        if (j < nk) acc[j] = sL[r][j];
    }
  } else if (r < gw) {
    // The query row in pieces of 64 elements, each piece's 16-byte loads
    // issued together (the row is 16-byte aligned), then the dot products
    // over the piece in element order.
    constexpr int CH = 64, PL = CH * (int)sizeof(E) / 16;
    const uint4* qr = reinterpret_cast<const uint4*>(qg + (size_t)r * D);
#pragma unroll
    for (int c0 = 0; c0 < D; c0 += CH) {
      uint4 raw[PL];
#pragma unroll
      for (int i = 0; i < PL; ++i) raw[i] = qr[c0 * (int)sizeof(E) / 16 + i];
      E qe[CH];
      __builtin_memcpy(qe, raw, sizeof(qe));
#pragma unroll
      for (int e0 = 0; e0 < CH; e0 += 8) {
        float qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = val(qe[e0 + e]);
#pragma unroll
        for (int j = 0; j < NK; ++j) {
          if (j < nk) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[j] = fmaf(qv[e], sK[j][c0 + e0 + e], acc[j]);
          }
        }
      }
    }
  }
  if (mode == 1) {
    if (r < gw) {
      float m = -INFINITY, z = 0.f;
#pragma unroll
      for (int j = 0; j < NK; ++j)
        if (j < nk) merge_stat(m, z, acc[j], 1.0f, c);
      const int tile = Dsc.tile_base[seq] + within * kvc_tiles_per_unit(L) + kvc_main_tiles(L) +
                       split;
      partials[(size_t)tile * gw + r] = make_float2(m, z);
    }
    return;
  }
  if (nk == 0) return;
  if (r < gw) {
    const float lr = lse2[(size_t)u * gw + r];
#pragma unroll
    for (int j = 0; j < NK; ++j) sP[r][j] = __builtin_amdgcn_exp2f(fmaf(acc[j], c, -lr));
  }
  __syncthreads();
  // Per (head g, key j): the sum over the head's W window queries; then over
  // heads, the mean over all G W queries or the largest head mean.
  const int W = Dsc.nwin, G = gw / W;
  for (int x = threadIdx.x; x < G * NK; x += KVC_MAX_GW) {
    const int g = x / NK, j = x - g * NK;
    float v = 0.f;
    for (int rr = g * W; rr < (g + 1) * W; ++rr) v += sP[rr][j];
    sH[g][j] = v;
  }
  __syncthreads();
  if ((int)threadIdx.x < nk) {
    const int j = threadIdx.x;
    float a = 0.f;
    for (int g = 0; g < G; ++g) a = Dsc.score_max ? fmaxf(a, sH[g][j]) : a + sH[g][j];
    float* srow = s + Dsc.srow_base[seq] + (int64_t)within * L;
    srow[j0 + j] = Dsc.score_max ? a / (float)W : a / (float)gw;
  }
}

// First score tile of unit u (u = n_units: the total).  Units [u0, u1) may
// span sequences: the tiles of consecutive units are consecutive.
static int tile_of_unit(const KvcDesc& D, int u) {
  const int seq = u / D.upseq;
  if (seq >= D.n_seq) return D.tile_base[D.n_seq];
  return D.tile_base[seq] + (u - seq * D.upseq) * kvc_tiles_per_unit(D.L[seq]);
}

template <class E, int Dm>
static void launch_tail(const KvcDesc& D, int u0, int u1, int mode, const void* q, const void* k,
                        const float* lse2, float2* partials, float* s, hipStream_t st) {
  bool any = false;  // any unit of the range with tail keys
  for (int seq = u0 / D.upseq; seq <= (u1 - 1) / D.upseq; ++seq) any |= (D.L[seq] & 63) != 0;
  if (!any) return;
  hipLaunchKernelGGL((kvc_score_tail_kernel<E, Dm>), dim3((u1 - u0) * KVC_TAIL_SPLITS),
                     dim3(KVC_MAX_GW), 0, st, D, u0, mode, (const E*)q, (const E*)k, lse2,
                     partials, s);
}

size_t kvc_scores_workspace(const KvcDesc& D) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  return up(sizeof(float) * (size_t)D.n_units * D.gw) +
         up(sizeof(float2) * (size_t)D.total_tiles * D.gw);
}

// Units [u0, u1) must lie in one sequence.
template <class T, int Dm, int NBC>
static void launch_pair(const KvcDesc& D, int u0, int u1, const void* q, const void* k, float* s,
                        float2* partials, float* lse2, hipStream_t st, int which) {
  using elem_t = typename T::elem_t;
  const int t0 = tile_of_unit(D, u0);
  const int nt = tile_of_unit(D, u1) - t0;
  if (which & 1) {
    hipLaunchKernelGGL((kvc_score_stats_kernel<T, Dm, NBC>), dim3(nt), dim3(SCORE_THREADS), 0, st,
                       D, t0, (const elem_t*)q, (const elem_t*)k, partials);
    launch_tail<elem_t, Dm>(D, u0, u1, 1, q, k, lse2, partials, s, st);
    hipLaunchKernelGGL(kvc_score_lse_kernel, dim3(u1 - u0), dim3(KVC_MAX_GW), 0, st, D, u0,
                       kLog2e / sqrtf((float)Dm), (const float2*)partials, lse2);
  }
  if (which & 2) {
    hipLaunchKernelGGL((kvc_score_pool_kernel<T, Dm, NBC>), dim3(nt), dim3(SCORE_THREADS), 0, st,
                       D, t0, (const elem_t*)q, (const elem_t*)k, (const float*)lse2, s);
    launch_tail<elem_t, Dm>(D, u0, u1, 2, q, k, lse2, partials, s, st);
  }
}

// Query-stationary bf16 passes; units [u0, u1) in one sequence.
template <int Dm, int NBC>
static void launch_qs(const KvcDesc& D, int u0, int u1, const void* q, const void* k, float* s,
                      float2* partials, float* lse2, hipStream_t st, int which,
                      const KvcBudgetArgs* budget) {
  const int t0 = tile_of_unit(D, u0);
  const int nt = tile_of_unit(D, u1) - t0;
  constexpr int NT = QsWaves<NBC>::NT;
  if (which & 1) {
    if constexpr (QsWaves<NBC>::MINB <= 2) {
      if (budget) {
        const int nbw = (D.n_seq * (D.upseq / D.pool_size) + 7) & ~7;
        hipLaunchKernelGGL((kvc_score_stats_qs_kernel<Dm, NBC, true>), dim3(nt + nbw), dim3(NT),
                           0, st, D, t0, (const uint16_t*)q, (const uint16_t*)k, partials,
                           *budget, nbw);
      }
    }
    if (!budget || QsWaves<NBC>::MINB > 2)
      hipLaunchKernelGGL((kvc_score_stats_qs_kernel<Dm, NBC, false>), dim3(nt), dim3(NT), 0, st,
                         D, t0, (const uint16_t*)q, (const uint16_t*)k, partials,
                         KvcBudgetArgs{nullptr, nullptr, nullptr}, 0);
    launch_tail<uint16_t, Dm>(D, u0, u1, 1, q, k, lse2, partials, s, st);
    hipLaunchKernelGGL(kvc_score_lse_kernel, dim3(u1 - u0), dim3(KVC_MAX_GW), 0, st, D, u0,
                       kLog2e / sqrtf((float)Dm), (const float2*)partials, lse2);
  }
  if ((which & 2) && D.score_max)
    hipLaunchKernelGGL((kvc_score_pool_qs_kernel<Dm, NBC, true>), dim3(nt), dim3(NT), 0, st, D,
                       t0, (const uint16_t*)q, (const uint16_t*)k, (const float*)lse2, s);
  else if (which & 2)
    hipLaunchKernelGGL((kvc_score_pool_qs_kernel<Dm, NBC, false>), dim3(nt), dim3(NT), 0, st, D,
                       t0, (const uint16_t*)q, (const uint16_t*)k, (const float*)lse2, s);
  if (which & 2) launch_tail<uint16_t, Dm>(D, u0, u1, 2, q, k, lse2, partials, s, st);
}

template <int Dm>
static void launch_bf16(const KvcDesc& D, int u0, int u1, const void* q, const void* k, float* s,
                        float2* partials, float* lse2, hipStream_t st, int which,
                        const KvcBudgetArgs* b) {
  switch (D.gw / 32) {
    case 1: launch_qs<Dm, 1>(D, u0, u1, q, k, s, partials, lse2, st, which, b); break;
    case 2: launch_qs<Dm, 2>(D, u0, u1, q, k, s, partials, lse2, st, which, b); break;
    case 3: launch_qs<Dm, 3>(D, u0, u1, q, k, s, partials, lse2, st, which, b); break;
    case 4: launch_qs<Dm, 4>(D, u0, u1, q, k, s, partials, lse2, st, which, b); break;
    case 5: launch_qs<Dm, 5>(D, u0, u1, q, k, s, partials, lse2, st, which, b); break;
    case 6: launch_qs<Dm, 6>(D, u0, u1, q, k, s, partials, lse2, st, which, b); break;
    case 7: launch_qs<Dm, 7>(D, u0, u1, q, k, s, partials, lse2, st, which, b); break;
    default: launch_qs<Dm, 8>(D, u0, u1, q, k, s, partials, lse2, st, which, b); break;
  }
}

bool kvc_scores_host_budget(const KvcDesc& D) {
  // bf16, d = 128, seven or eight 32-query blocks: four waves per workgroup
  // and two workgroups per CU with or without the budget's LDS (smaller
  // kernels run more workgroups per CU than that LDS would allow)
  const int nbc = D.gw / 32 < 8 ? D.gw / 32 : 8;
  return D.dtype == 0 && D.d == 128 && nbc >= 7;
}

hipError_t kvc_launch_scores(const KvcDesc& D, int u0, int u1, const void* q, const void* k,
                             float* s, float2* partials, float* lse2, hipStream_t st, int which,
                             const KvcBudgetArgs* budget) {
  if (u1 <= u0) return hipSuccess;
  if (budget && (!kvc_scores_host_budget(D) || u0 != 0 || u1 != D.n_units || !(which & 1)))
    return hipErrorInvalidValue;
  if (D.dtype == 0 && D.d == 128)
    launch_bf16<128>(D, u0, u1, q, k, s, partials, lse2, st, which, budget);
  else if (D.dtype == 0 && D.d == 64)
    launch_bf16<64>(D, u0, u1, q, k, s, partials, lse2, st, which, budget);
  else if (D.dtype == 1 && D.d == 128) launch_pair<TF64, 128, 0>(D, u0, u1, q, k, s, partials, lse2, st, which);
  else if (D.dtype == 1 && D.d == 64) launch_pair<TF64, 64, 0>(D, u0, u1, q, k, s, partials, lse2, st, which);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
