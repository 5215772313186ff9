// wnw.hip -- decode-time chunk recall (WnW digest page, "WnW: Waxing-and-
// Waning KV Cache for Long-Form Speech LLMs": anchor, tidal and fixed KV
// heads; 4 s chunks with a 2 s stride, the top 3 chunks per step, release
// after 3 unselected steps) and the segment-wise selection of fixed heads.
//
// One decode step, all sequences at once:
//   wnw_logits_kernel      anchor logits q_g . k_j / sqrt(d) (log2 units) for
//                          every anchor's G query heads on the matrix cores
//                          (16x16x32 bf16 MFMA: the query heads as rows, 16
//                          keys as columns), and one (max, sum exp)
//                          partial per workgroup of 256 keys and query head.
//   wnw_lse_kernel         the partials folded into each head's LSE (one
//                          workgroup per head).
//   wnw_mass_kernel        per run of blocks: the positions' attention mass
//                          (sum over anchors of the mean over heads of
//                          exp2(l - LSE), i.e. the sum over all anchor heads
//                          divided by G) staged in LDS, the blocks' masses
//                          summed in position order, and the chunk scores
//                          (sums of m consecutive blocks; m - 1 blocks past
//                          the run are recomputed by the workgroup).
//   wnw_update_kernel      one 1024-thread workgroup per sequence: top-K by
//                          packed (score, index) maxima, idle counts,
//                          residency, slot release and assignment with
//                          block scans, the recall list.
//   wnw_recall_kernel      one workgroup per (tidal head, sequence): 16-byte
//                          copies of the recalled blocks' K and V rows from
//                          page-locked host memory (read over PCIe by the
//                          kernel itself, so no host round trip is needed to
//                          learn which blocks to fetch) into the slots.
// Decisions (top-K ties, slot order) are made in integers on one workgroup,
// so they are reproducible; the scores are fp32 sums in a fixed order.
#include <algorithm>
#include <cstring>

#include "kvc_internal.h"
#include "kvc_wnw.h"

#define WNW_MAX_SEQ 64
#define WNW_MAX_ANCHOR 64
#define WNW_MAX_UNITS 4096
#define WNW_MAX_CAP 131072
#define WNW_MAX_G 32
#define WNW_MAX_M 8
#define WNW_MAX_K 8
#define WNW_MAX_H 8
#define WNW_MAX_CHUNKS 65536
#define WNW_TILE 256
#define WNW_UT 1024
#define WNW_MAX_SLOTS (WNW_MAX_K * WNW_MAX_H * WNW_MAX_M)

static constexpr float kWnwLog2e = 1.4426950408889634f;

struct WnwDesc {
  int32_t n_seq, upseq, gqa, d;
  int32_t S, m, K, H, slot_cap, block_cap, chunk_cap;
  int32_t n_anchor, n_tidal, max_len, max_parts;
  int32_t len[WNW_MAX_SEQ];
  int32_t anchor_unit[WNW_MAX_ANCHOR];     // unit within a sequence: l * n_heads + h
  uint32_t tidal_mask[WNW_MAX_UNITS / 32];
  int64_t ks[2], hs[2], ss[2];
};

struct WnwState {
  int32_t *idle, *slot_of_block, *block_of_slot, *selected, *n_recalled, *recalled_block,
      *recalled_slot;
};

struct WnwWork {
  float* logits;   // [n_seq * n_anchor][G][max_len]
  float2* parts;   // [n_seq * n_anchor][G][max_parts], one per 256-key tile
  float* lse2;     // [n_seq * n_anchor][G]
  float* sigma;    // [n_seq][chunk_cap]
};

__device__ __forceinline__ float wnw_bf16(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

__device__ __forceinline__ void wnw_merge(float& m, float& z, float m2, float z2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  const float a = (m == -INFINITY) ? 0.f : z * __builtin_amdgcn_exp2f(m - mm);
  const float b = (m2 == -INFINITY) ? 0.f : z2 * __builtin_amdgcn_exp2f(m2 - mm);
  m = mm;
  z = a + b;
}

// ---------------------------------------------------------------------------
// Steps 1-2: anchor attention, block masses, chunk scores
// ---------------------------------------------------------------------------

typedef __bf16 wnw_bf16x8 __attribute__((ext_vector_type(8)));
typedef float wnw_f4 __attribute__((ext_vector_type(4)));

// One workgroup per (sequence, anchor) and 256 keys; wave w takes keys
// 64 w .. 64 w + 63 of the tile in four groups of 16.  A group's logits are
// one v_mfma_f32_16x16x32_bf16 chain per 16 query heads: A = the query heads
// (rows; zero past G), B = the 16 keys (columns).  Lane l supplies row or
// column l % 16 and, at k-step ks, head dims ks*32 + (l/16)*8 .. +7 of both
// operands, so every dim is contracted once and a lane reads 16-byte runs of
// its key row (64 contiguous bytes per key and k-step across the lane
// group).  Output lane l holds key l % 16 for query heads (l/16)*4 .. +3 of
// the block.  Keys past the sequence read its last row and are masked.
template <int D>
__global__ __launch_bounds__(WNW_TILE) void wnw_logits_kernel(WnwDesc W, const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              WnwWork X) {
  constexpr int KS = D / 32;
  constexpr int NWV = WNW_TILE / 64;
  __shared__ float2 sred[WNW_MAX_G][NWV];
  const int sa = blockIdx.y, seq = sa / W.n_anchor, a = sa - seq * W.n_anchor;
  const int n = W.len[seq], tile = blockIdx.x;
  if (tile * WNW_TILE >= n) return;
  const int G = W.gqa;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const uint16_t* qs = q + (size_t)sa * G * D;
  wnw_bf16x8 qa[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb * 16 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // rows past G: the last head's bits masked to zero (no branch)
      uint4 raw = *reinterpret_cast<const uint4*>(qs + (size_t)min(row, G - 1) * D + ks * 32 + grp * 8);
      const uint32_t keep = row < G ? 0xFFFFFFFFu : 0u;
      raw.x &= keep;
      raw.y &= keep;
      raw.z &= keep;
      raw.w &= keep;
      __builtin_memcpy(&qa[qb][ks], &raw, 16);
    }
  }
  const bool two = G > 16;
  const int64_t unit = (int64_t)seq * W.upseq + W.anchor_unit[a];
  const uint16_t* ku = k + unit * W.ks[0];
  const float c = kWnwLog2e / sqrtf((float)D);
  const int j0 = tile * WNW_TILE + wave * 64;
  // All 4 x KS fragment loads of the wave are issued before the first MFMA.
  uint4 kraw[4][KS];
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) {
    const int j = min(j0 + kg * 16 + col, n - 1);
    const uint16_t* kr = ku + (int64_t)j * W.ks[1] + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kraw[kg][ks] = *reinterpret_cast<const uint4*>(kr + ks * 32);
  }
  __builtin_amdgcn_sched_barrier(0);
  wnw_f4 acc[2][4];
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) {
    wnw_bf16x8 kb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) __builtin_memcpy(&kb[ks], &kraw[kg][ks], 16);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      wnw_f4 t = {0.f, 0.f, 0.f, 0.f};
      if (qb == 0 || two)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[qb][ks], kb[ks], t, 0, 0, 0);
      acc[qb][kg] = t;
    }
  }
  // Logits out, and this wave's (max, sum exp2) per query head over its 64
  // keys: the lane's four keys, then the 16 lanes of its group.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (qb == 1 && !two) break;   // (uniform: no second block of heads)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = qb * 16 + grp * 4 + i;   // uniform per lane group
      float l2[4], mx = -INFINITY;
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const int j = j0 + kg * 16 + col;
        l2[kg] = acc[qb][kg][i] * c;
        if (j < n) {
          mx = fmaxf(mx, l2[kg]);
          if (g < G) X.logits[((size_t)sa * G + g) * W.max_len + j] = l2[kg];
        }
      }
      mx = kvc_row16_max(mx);
      float z = 0.f;
#pragma unroll
      for (int kg = 0; kg < 4; ++kg)
        if (j0 + kg * 16 + col < n) z += __builtin_amdgcn_exp2f(l2[kg] - mx);
      z = kvc_row16_sum(z);
      if (col == 0 && g < G) sred[g][wave] = make_float2(mx, z);
    }
  }
  __syncthreads();
  // The tile's partial per query head (waves with no key past n give (-inf, 0)).
  if (threadIdx.x < G) {
    const int g = threadIdx.x;
    float m = -INFINITY, z = 0.f;
    for (int w = 0; w < NWV; ++w) wnw_merge(m, z, sred[g][w].x, sred[g][w].y);
    X.parts[((size_t)sa * G + g) * W.max_parts + tile] = make_float2(m, z);
  }
}

// One workgroup per (sequence, anchor, query head) row.
__global__ __launch_bounds__(256) void wnw_lse_kernel(WnwDesc W, WnwWork X) {
  __shared__ float2 sred[4];
  const size_t row = blockIdx.x;
  const int seq = (int)(row / ((size_t)W.n_anchor * W.gqa));
  const int nparts = (W.len[seq] + WNW_TILE - 1) / WNW_TILE;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float2* p = X.parts + row * W.max_parts;
  float m = -INFINITY, z = 0.f;
  for (int i = threadIdx.x; i < nparts; i += 256) wnw_merge(m, z, p[i].x, p[i].y);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), z2 = __shfl_xor(z, o);
    wnw_merge(m, z, m2, z2);
  }
  if (lane == 0) sred[wave] = make_float2(m, z);
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = sred[0].x, zz = sred[0].y;
    for (int w = 1; w < 4; ++w) wnw_merge(mm, zz, sred[w].x, sred[w].y);
    X.lse2[row] = mm + __builtin_amdgcn_logf(zz);
  }
}

// Chunk scores of chunks b0 .. b0 + nb - 1 of one sequence (nb = the blocks
// per workgroup; the grid covers chunk_cap, zeros past the sequence's C).
// Positions are taken WNW_MT at a time: a thread per position computes its
// mass into LDS, then a thread per block adds the block's positions of the
// tile in order to the block's running mass.  Every sum has a fixed order.
#define WNW_MT 256
__global__ __launch_bounds__(WNW_MT) void wnw_mass_kernel(WnwDesc W, WnwWork X, float* __restrict__ sigma,
                                                          int nb) {
  __shared__ float slse[WNW_MAX_ANCHOR * WNW_MAX_G];
  __shared__ float spm[WNW_MT];
  __shared__ float sbeta[WNW_MT + WNW_MAX_M];
  const int seq = blockIdx.y, tid = threadIdx.x;
  const int n = W.len[seq], S = W.S, m = W.m;
  const int B = (n + S - 1) / S, C = max(1, B - m + 1);
  const int b0 = blockIdx.x * nb;
  const int cend = min(W.chunk_cap, b0 + nb);
  float* sg = sigma + (size_t)seq * W.chunk_cap;
  if (b0 >= C) {
    for (int c = b0 + tid; c < cend; c += WNW_MT) sg[c] = 0.f;
    return;
  }
  const int G = W.gqa, ra = W.n_anchor * G;
  const size_t row0 = (size_t)seq * ra;
  for (int i = tid; i < ra; i += WNW_MT) slse[i] = X.lse2[row0 + i];
  const int nbw = min(B, b0 + nb + m - 1) - b0;   // blocks whose mass is needed
  for (int j = tid; j < nbw; j += WNW_MT) sbeta[j] = 0.f;
  __syncthreads();
  const float invG = 1.0f / (float)G;
  const int p_lo = b0 * S, p_hi = min(n, (b0 + nbw) * S);
  for (int t0 = p_lo; t0 < p_hi; t0 += WNW_MT) {
    const int p = t0 + tid;
    // The rows' terms summed in row order, then divided by G (every anchor
    // has G heads); eight rows' loads in flight at a time.
    float pm = 0.f;
    if (p < p_hi) {
      const float* lp = X.logits + row0 * W.max_len + p;
      int r = 0;
      for (; r + 8 <= ra; r += 8) {
        float l[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) l[i] = lp[(size_t)(r + i) * W.max_len];
#pragma unroll
        for (int i = 0; i < 8; ++i) pm += __builtin_amdgcn_exp2f(l[i] - slse[r + i]);
      }
      for (; r < ra; ++r) pm += __builtin_amdgcn_exp2f(lp[(size_t)r * W.max_len] - slse[r]);
      pm *= invG;
    }
    spm[tid] = pm;
    __syncthreads();
    const int t1 = min(p_hi, t0 + WNW_MT);
    const int jb0 = (t0 - p_lo) / S, jb1 = (t1 - 1 - p_lo) / S;
    for (int jb = jb0 + tid; jb <= jb1; jb += WNW_MT) {
      const int lo = max(t0, p_lo + jb * S), hi = min(t1, p_lo + (jb + 1) * S);
      float sb = 0.f;
      for (int x = lo; x < hi; ++x) sb += spm[x - t0];
      sbeta[jb] += sb;
    }
    __syncthreads();
  }
  for (int c = b0 + tid; c < cend; c += WNW_MT) {
    float sc = 0.f;
    if (c < C)
      for (int b = c; b < min(c + m, B); ++b) sc += sbeta[b - b0];
    sg[c] = sc;
  }
}

// Blocks per mass workgroup: as many as fit one tile of positions with the
// m - 1 blocks recomputed past them, at least one.
static int wnw_mass_blocks(const WnwDesc& W) {
  return std::max(1, (WNW_MT - (W.m - 1) * W.S) / W.S);
}

// ---------------------------------------------------------------------------
// Steps 3-4: selection, residency, slots (one workgroup per sequence)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wnw_order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive scan over the workgroup's WNW_UT threads; *total gets the sum.
__device__ __forceinline__ int wnw_scan(int v, int* sw, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sw[w] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < WNW_UT / 64; ++i) {
    const int x = sw[i];
    if (i < w) before += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

__global__ __launch_bounds__(WNW_UT) void wnw_update_kernel(WnwDesc W, const float* __restrict__ sigma,
                                                            WnwState in, WnwState out) {
  __shared__ unsigned long long sbest[WNW_UT / 64];
  __shared__ int ssel[WNW_MAX_K];
  __shared__ int sfree[WNW_MAX_SLOTS];
  __shared__ int sw[WNW_UT / 64];
  const int seq = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = W.len[seq], B = (n + W.S - 1) / W.S, C = max(1, B - W.m + 1);
  const float* sg = sigma + (size_t)seq * W.chunk_cap;
  const size_t oc = (size_t)seq * W.chunk_cap, ob = (size_t)seq * W.block_cap,
               os = (size_t)seq * W.slot_cap;
  // Top-K: the largest (score, -index) key, K times.
  const int nsel = min(W.K, C);
  for (int r = 0; r < nsel; ++r) {
    unsigned long long best = 0;
    for (int c = t; c < C; c += WNW_UT) {
      bool taken = false;
      for (int i = 0; i < r; ++i) taken |= (ssel[i] == c);
      if (taken) continue;
      const unsigned long long key =
          ((unsigned long long)wnw_order_key(sg[c]) << 32) | (unsigned long long)(0xffffffffu - (uint32_t)c);
      best = key > best ? key : best;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long y = __shfl_xor(best, o);
      best = y > best ? y : best;
    }
    if (lane == 0) sbest[wave] = best;
    __syncthreads();
    if (t == 0) {
      unsigned long long bb = 0;
      for (int i = 0; i < WNW_UT / 64; ++i) bb = sbest[i] > bb ? sbest[i] : bb;
      ssel[r] = (int)(0xffffffffu - (uint32_t)(bb & 0xffffffffull));
    }
    __syncthreads();
  }
  if (t < W.K) out.selected[(size_t)seq * W.K + t] = t < nsel ? ssel[t] : -1;
  // Idle counts.
  for (int c = t; c < W.chunk_cap; c += WNW_UT) {
    int z = -1;
    if (c < C) {
      bool s = false;
      for (int i = 0; i < nsel; ++i) s |= (ssel[i] == c);
      const int z0 = in.idle[oc + c];
      z = s ? 0 : (z0 >= 0 ? (z0 + 1 >= W.H ? -1 : z0 + 1) : -1);
    }
    out.idle[oc + c] = z;
  }
  __syncthreads();
  auto resident = [&](int b) {
    bool r = false;
    for (int c = max(0, b - W.m + 1); c <= min(b, C - 1); ++c) r |= out.idle[oc + c] >= 0;
    return r;
  };
  // Kept slots stay, the others are free.
  bool fr = false;
  if (t < W.slot_cap) {
    const int blk = in.block_of_slot[os + t];
    const bool keep = blk >= 0 && blk < B && resident(blk);
    out.block_of_slot[os + t] = keep ? blk : -1;
    fr = !keep;
  }
  int nfree;
  const int fr_rank = wnw_scan(fr ? 1 : 0, sw, &nfree);
  if (fr) sfree[fr_rank] = t;
  __syncthreads();
  // Blocks: kept slot, none, or the next free slot (ascending blocks).
  int base = 0;
  for (int b0 = 0; b0 < W.block_cap; b0 += WNW_UT) {
    const int b = b0 + t;
    bool isnew = false;
    int slot = -1;
    if (b < B && resident(b)) {
      slot = in.slot_of_block[ob + b];
      isnew = slot < 0;
    }
    int tot;
    const int r = wnw_scan(isnew ? 1 : 0, sw, &tot) + base;
    if (isnew) {
      slot = r < nfree ? sfree[r] : -1;
      if (slot >= 0) {
        out.block_of_slot[os + slot] = b;
        out.recalled_block[os + r] = b;
        out.recalled_slot[os + r] = slot;
      }
    }
    if (b < W.block_cap) out.slot_of_block[ob + b] = slot;
    base += tot;
  }
  const int nrec = min(base, nfree);
  for (int r = nrec + t; r < W.slot_cap; r += WNW_UT) {
    out.recalled_block[os + r] = -1;
    out.recalled_slot[os + r] = -1;
  }
  if (t == 0) out.n_recalled[seq] = nrec;
}

// ---------------------------------------------------------------------------
// Step 5: recall copies, host -> slots
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void wnw_recall_kernel(WnwDesc W, WnwState st,
                                                         const uint16_t* __restrict__ hk,
                                                         const uint16_t* __restrict__ hv,
                                                         uint16_t* __restrict__ sk,
                                                         uint16_t* __restrict__ sv) {
  __shared__ int sunit;
  const int tid = blockIdx.x, seq = blockIdx.y;
  if (threadIdx.x == 0) {
    // the tid-th tidal unit of the role table
    int seen = 0, u = -1;
    for (int w = 0; w < (W.upseq + 31) / 32 && u < 0; ++w) {
      const uint32_t m = W.tidal_mask[w];
      const int pc = __popc(m);
      if (seen + pc > tid) {
        uint32_t mm = m;
        for (int i = 0; i < tid - seen; ++i) mm &= mm - 1;
        u = w * 32 + __ffs(mm) - 1;
      }
      seen += pc;
    }
    sunit = u;
  }
  __syncthreads();
  const int uw = sunit;
  if (uw < 0) return;
  const int64_t unit = (int64_t)seq * W.upseq + uw;
  const int n = W.len[seq], B = (n + W.S - 1) / W.S;
  // (a state from elsewhere is range-checked entry by entry)
  const int nrec = min(max(st.n_recalled[seq], 0), W.slot_cap);
  constexpr int PR = D / 8;  // 16-byte pieces per row
  const size_t os = (size_t)seq * W.slot_cap;
  for (int r = 0; r < nrec; ++r) {
    const int b = st.recalled_block[os + r], s = st.recalled_slot[os + r];
    if (b < 0 || b >= B || s < 0 || s >= W.slot_cap) continue;
    const int rows = min(W.S, n - b * W.S);
    const uint16_t* hkb = hk + unit * W.hs[0] + (int64_t)b * W.S * W.hs[1];
    const uint16_t* hvb = hv + unit * W.hs[0] + (int64_t)b * W.S * W.hs[1];
    uint16_t* skb = sk + unit * W.ss[0] + (int64_t)s * W.S * W.ss[1];
    uint16_t* svb = sv + unit * W.ss[0] + (int64_t)s * W.S * W.ss[1];
    for (int i = threadIdx.x; i < rows * PR; i += 256) {
      const int row = i / PR, p = i - row * PR;
      const uint4 kx = reinterpret_cast<const uint4*>(hkb + (int64_t)row * W.hs[1])[p];
      const uint4 vx = reinterpret_cast<const uint4*>(hvb + (int64_t)row * W.hs[1])[p];
      reinterpret_cast<uint4*>(skb + (int64_t)row * W.ss[1])[p] = kx;
      reinterpret_cast<uint4*>(svb + (int64_t)row * W.ss[1])[p] = vx;
    }
  }
}

__global__ void wnw_fill_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ---------------------------------------------------------------------------
// Fixed heads: segment-wise selection at prefill.  Grid (unit, group of
// WNW_SEGS segments); one wave per segment of at most 64 positions.  Each
// segment's quota and its first output slot are closed forms, so the
// segments need no exchange.
// ---------------------------------------------------------------------------
#define WNW_SEGS 16

__global__ __launch_bounds__(256) void wnw_fixed_select_kernel(KvcDesc D, int seg,
                                                               const float* __restrict__ s_hat,
                                                               const int32_t* __restrict__ budgets,
                                                               const int64_t* __restrict__ offsets,
                                                               int32_t* __restrict__ idx_out) {
  __shared__ __attribute__((aligned(16))) uint32_t skey[4][64];
  const int u = blockIdx.x;
  const int seq = u / D.upseq, within = u - seq * D.upseq;
  const int L = D.L[seq], w = D.window, ncand = L - w;
  // (budgets hold w <= b <= L, as for kvc_select; clamped all the same)
  const int k = min(max(budgets[u] - w, 0), max(ncand, 0));
  int32_t* out = idx_out + offsets[u];
  if (blockIdx.y == 0)
    for (int i = threadIdx.x; i < w; i += 256) out[k + i] = ncand + i;
  if (k <= 0) return;
  const float* row = s_hat + D.srow_base[seq] + (int64_t)within * L;
  // Quotas: every full segment has the same floor and remainder, the short
  // last one (if any) its own; the R leftovers go by remainder, then index.
  const int64_t nfull = ncand / seg, last = ncand - nfull * seg;
  const int64_t qf = (int64_t)k * seg / ncand, rf = (int64_t)k * seg % ncand;
  const int64_t ql = last ? (int64_t)k * last / ncand : 0, rl = last ? (int64_t)k * last % ncand : 0;
  const int64_t R = k - nfull * qf - ql;
  const bool last_first = last && rl > rf;
  const int64_t rfull =  // full segments with +1
      std::max<int64_t>(0, std::min<int64_t>(nfull, last_first ? R - 1 : R));
  const int64_t qlast = ql + ((last_first && R >= 1) || (!last_first && R > nfull) ? 1 : 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t J = nfull + (last ? 1 : 0);
  const int64_t j1 = std::min<int64_t>(J, (int64_t)(blockIdx.y + 1) * WNW_SEGS);
  for (int64_t j = (int64_t)blockIdx.y * WNW_SEGS + wave; j < j1; j += 4) {
    const int lo = (int)(j * seg), len = (int)std::min<int64_t>(seg, ncand - j * seg);
    const int64_t quota = (j < nfull) ? qf + (j < rfull ? 1 : 0) : qlast;
    const int64_t before = (j < nfull) ? j * qf + std::min<int64_t>(j, rfull) : nfull * qf + rfull;
    const bool valid = lane < len;
    const uint32_t key = valid ? wnw_order_key(row[lo + lane]) : 0u;
    skey[wave][lane] = key;   // the wave's own row: no barrier needed
    __builtin_amdgcn_wave_barrier();
    // Rank = keys above, then equal keys at lower positions.  The padding
    // (key 0) is above no key, so the first count needs no bound.  Without
    // equal keys the ranks of the segment are 0 .. len-1 once each, and
    // equal keys share a rank, which lowers the sum: only then is the
    // tie-breaking count run (a uniform branch).
    int rank = 0;
    for (int o = 0; o < len; o += 4) {
      const uint4 kq = *reinterpret_cast<const uint4*>(&skey[wave][o]);   // same for every lane
      rank += (kq.x > key) + (kq.y > key) + (kq.z > key) + (kq.w > key);
    }
    int rsum = 0;
#pragma unroll
    for (int b = 0; b < 6; ++b) rsum += __popcll(__ballot(valid && ((rank >> b) & 1))) << b;
    if (rsum != len * (len - 1) / 2) {
      rank = 0;
      for (int o = 0; o < len; o += 4) {
        const uint4 kq = *reinterpret_cast<const uint4*>(&skey[wave][o]);
        const uint32_t ko[4] = {kq.x, kq.y, kq.z, kq.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rank += (o + e < len) && ((ko[e] > key) || (ko[e] == key && o + e < lane));
      }
    }
    __builtin_amdgcn_wave_barrier();
    const bool take = valid && rank < quota;
    const unsigned long long mask = __ballot(take);
    const int pos = __popcll(mask & ((1ull << lane) - 1ull));
    if (take) out[before + pos] = lo + lane;
  }
}

hipError_t kvc_launch_wnw_fixed_select(const KvcDesc& D, int seg, const float* s_hat,
                                       const int32_t* budgets, const int64_t* offsets,
                                       int32_t* idx_out, hipStream_t st) {
  int jmax = 1;
  for (int i = 0; i < D.n_seq; ++i) jmax = max(jmax, (D.L[i] - D.window + seg - 1) / seg);
  const dim3 grid((unsigned)D.n_units, (unsigned)((jmax + WNW_SEGS - 1) / WNW_SEGS));
  hipLaunchKernelGGL(wnw_fixed_select_kernel, grid, dim3(256), 0, st, D, seg, s_hat, budgets,
                     offsets, idx_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static size_t wnw_up(size_t x) { return (x + 255) & ~size_t(255); }

static kvc_status wnw_hip(hipError_t e) {
  if (e == hipSuccess) return KVC_OK;
  kvc_note_hip_error((int)e);
  return KVC_ERR_HIP;
}

static kvc_status wnw_desc(const kvc_wnw_problem* p, const kvc_wnw_params* prm, WnwDesc* W) {
  if (!p || !prm || !W || !p->len || !p->role) return KVC_ERR_INVALID_ARG;
  if (p->n_seq < 1 || p->n_layers < 1 || p->n_kv_heads < 1 || p->gqa_group < 1 ||
      p->head_dim < 1 || p->capacity < 1)
    return KVC_ERR_INVALID_ARG;
  const int S = prm->chunk_stride, Wc = prm->chunk_len;
  if (S < 1 || Wc < S || Wc % S != 0 || prm->top_chunks < 1 || prm->release_after < 1)
    return KVC_ERR_INVALID_ARG;
  if (Wc / S > WNW_MAX_M || prm->top_chunks > WNW_MAX_K || prm->release_after > WNW_MAX_H)
    return KVC_ERR_UNSUPPORTED;
  if (p->n_seq > WNW_MAX_SEQ || p->capacity > WNW_MAX_CAP) return KVC_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return KVC_ERR_UNSUPPORTED;
  if (p->gqa_group > WNW_MAX_G) return KVC_ERR_UNSUPPORTED;
  const int64_t upseq = (int64_t)p->n_layers * p->n_kv_heads;
  if (upseq > WNW_MAX_UNITS) return KVC_ERR_UNSUPPORTED;
  memset(W, 0, sizeof(*W));
  int na = 0, nt = 0;
  for (int64_t u = 0; u < upseq; ++u) {
    const uint8_t r = p->role[u];
    if (r > KVC_WNW_TIDAL) return KVC_ERR_INVALID_ARG;
    if (r == KVC_WNW_ANCHOR) {
      if (na == WNW_MAX_ANCHOR) return KVC_ERR_UNSUPPORTED;
      W->anchor_unit[na++] = (int32_t)u;
    } else if (r == KVC_WNW_TIDAL) {
      W->tidal_mask[u / 32] |= 1u << (u % 32);
      ++nt;
    }
  }
  if (na < 1) return KVC_ERR_INVALID_ARG;
  for (int a = 0; a < 2; ++a)
    if (p->k_stride[a] < 0 || p->host_stride[a] < 0 || p->slot_stride[a] < 0 ||
        p->k_stride[a] % 8 || p->host_stride[a] % 8 || p->slot_stride[a] % 8)
      return KVC_ERR_INVALID_ARG;
  const int m = Wc / S;
  const int64_t slot_cap = (int64_t)prm->top_chunks * prm->release_after * m;
  if (p->k_stride[1] < p->head_dim || p->k_stride[0] < p->k_stride[1] * p->capacity)
    return KVC_ERR_INVALID_ARG;
  if (nt > 0) {
    if (p->host_stride[1] < p->head_dim || p->host_stride[0] < p->host_stride[1] * p->capacity)
      return KVC_ERR_INVALID_ARG;
    if (p->slot_stride[1] < p->head_dim || p->slot_stride[0] < p->slot_stride[1] * slot_cap * S)
      return KVC_ERR_INVALID_ARG;
  }
  int max_len = 1, bcap = 1, ccap = 1;
  for (int i = 0; i < p->n_seq; ++i) {
    const int64_t n = p->len[i];
    if (n < 1 || n > p->capacity) return KVC_ERR_INVALID_ARG;
    const int64_t B = (n + S - 1) / S, C = std::max<int64_t>(1, B - m + 1);
    if (C > WNW_MAX_CHUNKS) return KVC_ERR_UNSUPPORTED;
    W->len[i] = (int32_t)n;
    max_len = std::max<int>(max_len, (int)n);
    bcap = std::max<int>(bcap, (int)B);
    ccap = std::max<int>(ccap, (int)C);
  }
  W->n_seq = p->n_seq;
  W->upseq = (int32_t)upseq;
  W->gqa = p->gqa_group;
  W->d = p->head_dim;
  W->S = S;
  W->m = m;
  W->K = prm->top_chunks;
  W->H = prm->release_after;
  W->slot_cap = (int32_t)slot_cap;
  W->block_cap = bcap;
  W->chunk_cap = ccap;
  W->n_anchor = na;
  W->n_tidal = nt;
  W->max_len = max_len;
  W->max_parts = (max_len + WNW_TILE - 1) / WNW_TILE;
  for (int a = 0; a < 2; ++a) {
    W->ks[a] = p->k_stride[a];
    W->hs[a] = p->host_stride[a];
    W->ss[a] = p->slot_stride[a];
  }
  return KVC_OK;
}

static void wnw_layout(const WnwDesc& W, kvc_wnw_layout* L) {
  memset(L, 0, sizeof(*L));
  const size_t N = (size_t)W.n_seq;
  L->n_anchor = W.n_anchor;
  L->n_tidal = W.n_tidal;
  L->block_cap = W.block_cap;
  L->chunk_cap = W.chunk_cap;
  L->slot_cap = W.slot_cap;
  size_t o = 0;
  L->idle = o;           o += wnw_up(4 * N * W.chunk_cap);
  L->slot_of_block = o;  o += wnw_up(4 * N * W.block_cap);
  L->block_of_slot = o;  o += wnw_up(4 * N * W.slot_cap);
  L->selected = o;       o += wnw_up(4 * N * W.K);
  L->n_recalled = o;     o += wnw_up(4 * N);
  L->recalled_block = o; o += wnw_up(4 * N * W.slot_cap);
  L->recalled_slot = o;  o += wnw_up(4 * N * W.slot_cap);
  L->state_bytes = o;
  const size_t SA = N * W.n_anchor * W.gqa;
  L->workspace_bytes = wnw_up(4 * SA * W.max_len) + wnw_up(8 * SA * W.max_parts) +
                       wnw_up(4 * SA) + wnw_up(4 * N * W.chunk_cap);
}

static WnwState wnw_state(const kvc_wnw_layout& L, const void* p) {
  char* b = (char*)p;
  WnwState s;
  s.idle = (int32_t*)(b + L.idle);
  s.slot_of_block = (int32_t*)(b + L.slot_of_block);
  s.block_of_slot = (int32_t*)(b + L.block_of_slot);
  s.selected = (int32_t*)(b + L.selected);
  s.n_recalled = (int32_t*)(b + L.n_recalled);
  s.recalled_block = (int32_t*)(b + L.recalled_block);
  s.recalled_slot = (int32_t*)(b + L.recalled_slot);
  return s;
}

static WnwWork wnw_work(const WnwDesc& W, void* p) {
  char* b = (char*)p;
  const size_t N = (size_t)W.n_seq, SA = N * W.n_anchor * W.gqa;
  WnwWork X;
  X.logits = (float*)b;  b += wnw_up(4 * SA * W.max_len);
  X.parts = (float2*)b;  b += wnw_up(8 * SA * W.max_parts);
  X.lse2 = (float*)b;    b += wnw_up(4 * SA);
  X.sigma = (float*)b;
  return X;
}

static bool wnw_a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool wnw_a256(const void* p) { return ((uintptr_t)p & 255u) == 0; }

// Page-locked host memory the device can read; its device-side address.
static bool wnw_host_ptr(const void* p, const void** dev) {
  if (!p || !wnw_a16(p)) return false;
  hipPointerAttribute_t a;
  memset(&a, 0, sizeof(a));
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (a.type != hipMemoryTypeHost || !a.devicePointer) return false;
  *dev = a.devicePointer;
  return wnw_a16(*dev);
}

extern "C" kvc_status kvc_wnw_plan(const kvc_wnw_problem* prob, const kvc_wnw_params* params,
                                   kvc_wnw_layout* layout) {
  WnwDesc W;
  const kvc_status st = wnw_desc(prob, params, &W);
  if (st != KVC_OK) return st;
  if (!layout) return KVC_ERR_INVALID_ARG;
  wnw_layout(W, layout);
  return KVC_OK;
}

extern "C" kvc_status kvc_wnw_init(const kvc_wnw_problem* prob, const kvc_wnw_params* params,
                                   void* state, void* stream) {
  WnwDesc W;
  kvc_status rs = wnw_desc(prob, params, &W);
  if (rs != KVC_OK) return rs;
  if (!state || !wnw_a256(state)) return KVC_ERR_INVALID_ARG;
  kvc_wnw_layout L;
  wnw_layout(W, &L);
  hipStream_t st = (hipStream_t)stream;
  const int64_t words = (int64_t)(L.state_bytes / 4);
  hipLaunchKernelGGL(wnw_fill_kernel, dim3(256), dim3(256), 0, st, (int32_t*)state, words, -1);
  hipLaunchKernelGGL(wnw_fill_kernel, dim3(1), dim3(64), 0, st,
                     (int32_t*)((char*)state + L.n_recalled), (int64_t)W.n_seq, 0);
  return wnw_hip(hipGetLastError());
}

static hipError_t wnw_launch_scores(const WnwDesc& W, const void* q, const void* k, float* sigma,
                                    const WnwWork& X, hipStream_t st) {
  const dim3 g1((unsigned)((W.max_len + WNW_TILE - 1) / WNW_TILE), (unsigned)(W.n_seq * W.n_anchor));
  if (W.d == 128)
    hipLaunchKernelGGL(wnw_logits_kernel<128>, g1, dim3(WNW_TILE), 0, st, W, (const uint16_t*)q,
                       (const uint16_t*)k, X);
  else
    hipLaunchKernelGGL(wnw_logits_kernel<64>, g1, dim3(WNW_TILE), 0, st, W, (const uint16_t*)q,
                       (const uint16_t*)k, X);
  hipLaunchKernelGGL(wnw_lse_kernel, dim3((unsigned)(W.n_seq * W.n_anchor * W.gqa)), dim3(256), 0,
                     st, W, X);
  const int nb = wnw_mass_blocks(W);
  hipLaunchKernelGGL(wnw_mass_kernel, dim3((unsigned)((W.chunk_cap + nb - 1) / nb), (unsigned)W.n_seq),
                     dim3(WNW_MT), 0, st, W, X, sigma, nb);
  return hipGetLastError();
}

static hipError_t wnw_launch_recall(const WnwDesc& W, const WnwState& s, const void* hk,
                                    const void* hv, void* sk, void* sv, hipStream_t st) {
  if (W.n_tidal == 0) return hipSuccess;
  const dim3 g((unsigned)W.n_tidal, (unsigned)W.n_seq);
  if (W.d == 128)
    hipLaunchKernelGGL(wnw_recall_kernel<128>, g, dim3(256), 0, st, W, s, (const uint16_t*)hk,
                       (const uint16_t*)hv, (uint16_t*)sk, (uint16_t*)sv);
  else
    hipLaunchKernelGGL(wnw_recall_kernel<64>, g, dim3(256), 0, st, W, s, (const uint16_t*)hk,
                       (const uint16_t*)hv, (uint16_t*)sk, (uint16_t*)sv);
  return hipGetLastError();
}

// Checks the host copies and slots of a call that recalls; their device
// addresses in *dk, *dv.
static kvc_status wnw_check_recall(const WnwDesc& W, const void* hk, const void* hv,
                                   const void* sk, const void* sv, const void** dk,
                                   const void** dv) {
  *dk = *dv = nullptr;
  if (W.n_tidal == 0) return KVC_OK;
  if (!sk || !sv || !wnw_a16(sk) || !wnw_a16(sv)) return KVC_ERR_INVALID_ARG;
  if (!wnw_host_ptr(hk, dk) || !wnw_host_ptr(hv, dv)) return KVC_ERR_INVALID_ARG;
  return KVC_OK;
}

extern "C" kvc_status kvc_wnw_chunk_scores(const kvc_wnw_problem* prob, const kvc_wnw_params* params,
                                           const void* q, const void* k, float* sigma,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  WnwDesc W;
  kvc_status rs = wnw_desc(prob, params, &W);
  if (rs != KVC_OK) return rs;
  if (!q || !k || !sigma || !workspace || !wnw_a16(q) || !wnw_a16(k) || !wnw_a256(workspace))
    return KVC_ERR_INVALID_ARG;
  kvc_wnw_layout L;
  wnw_layout(W, &L);
  if (workspace_bytes < L.workspace_bytes) return KVC_ERR_WORKSPACE;
  return wnw_hip(wnw_launch_scores(W, q, k, sigma, wnw_work(W, workspace), (hipStream_t)stream));
}

extern "C" kvc_status kvc_wnw_update(const kvc_wnw_problem* prob, const kvc_wnw_params* params,
                                     const float* sigma, const void* state_in, void* state_out,
                                     void* stream) {
  WnwDesc W;
  kvc_status rs = wnw_desc(prob, params, &W);
  if (rs != KVC_OK) return rs;
  if (!sigma || !state_in || !state_out || state_in == state_out || !wnw_a256(state_in) ||
      !wnw_a256(state_out))
    return KVC_ERR_INVALID_ARG;
  kvc_wnw_layout L;
  wnw_layout(W, &L);
  hipLaunchKernelGGL(wnw_update_kernel, dim3((unsigned)W.n_seq), dim3(WNW_UT), 0,
                     (hipStream_t)stream, W, sigma, wnw_state(L, state_in), wnw_state(L, state_out));
  return wnw_hip(hipGetLastError());
}

extern "C" kvc_status kvc_wnw_recall(const kvc_wnw_problem* prob, const kvc_wnw_params* params,
                                     const void* state, const void* host_k, const void* host_v,
                                     void* slot_k, void* slot_v, void* stream) {
  WnwDesc W;
  kvc_status rs = wnw_desc(prob, params, &W);
  if (rs != KVC_OK) return rs;
  if (!state || !wnw_a256(state)) return KVC_ERR_INVALID_ARG;
  const void *dk, *dv;
  if ((rs = wnw_check_recall(W, host_k, host_v, slot_k, slot_v, &dk, &dv)) != KVC_OK) return rs;
  kvc_wnw_layout L;
  wnw_layout(W, &L);
  return wnw_hip(wnw_launch_recall(W, wnw_state(L, state), dk, dv, slot_k, slot_v,
                                   (hipStream_t)stream));
}

extern "C" kvc_status kvc_wnw_step(const kvc_wnw_problem* prob, const kvc_wnw_params* params,
                                   const void* q, const void* k, const void* state_in,
                                   void* state_out, const void* host_k, const void* host_v,
                                   void* slot_k, void* slot_v, float* sigma, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  WnwDesc W;
  kvc_status rs = wnw_desc(prob, params, &W);
  if (rs != KVC_OK) return rs;
  if (!q || !k || !state_in || !state_out || state_in == state_out || !workspace)
    return KVC_ERR_INVALID_ARG;
  if (!wnw_a16(q) || !wnw_a16(k) || !wnw_a256(state_in) || !wnw_a256(state_out) ||
      !wnw_a256(workspace))
    return KVC_ERR_INVALID_ARG;
  const void *dk, *dv;
  if ((rs = wnw_check_recall(W, host_k, host_v, slot_k, slot_v, &dk, &dv)) != KVC_OK) return rs;
  kvc_wnw_layout L;
  wnw_layout(W, &L);
  if (workspace_bytes < L.workspace_bytes) return KVC_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const WnwWork X = wnw_work(W, workspace);
  float* sg = sigma ? sigma : X.sigma;
  hipError_t e = wnw_launch_scores(W, q, k, sg, X, st);
  if (e != hipSuccess) return wnw_hip(e);
  const WnwState so = wnw_state(L, state_out);
  hipLaunchKernelGGL(wnw_update_kernel, dim3((unsigned)W.n_seq), dim3(WNW_UT), 0, st, W,
                     (const float*)sg, wnw_state(L, state_in), so);
  if ((e = hipGetLastError()) != hipSuccess) return wnw_hip(e);
  return wnw_hip(wnw_launch_recall(W, so, dk, dv, slot_k, slot_v, st));
}
