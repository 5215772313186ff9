// voxzip.hip -- decode-time decayed KV-cache eviction (kvc_voxzip.h).
//
// VoxZip digest page, method overview, second stage "Temporally Decayed KV
// Cache Eviction": every decode step adds the new token's attention row to
// an exponentially decayed running score A, and whenever a cache exceeds
// its budget it keeps its first T rows, its last M rows and the N middle
// rows of largest A, concatenated in order.
//
// Four kernels per step, every cache u = (sequence, layer, KV head):
//   logits  one workgroup per (cache, 256-row part): the G x 256 logits
//           (log2 units, c = log2(e)/sqrt(d) folded in) into workspace, and
//           per query head the part's (max, sum of exp2).  bf16 on
//           v_mfma_f32_16x16x32_bf16 with the G query heads as A rows (16
//           per block, zero past G) and 16 cache rows as B columns, every
//           fragment load of a wave in flight before its first MFMA; fp32
//           inputs on fp64 VALU dot products.
//   accum   one workgroup per (cache, 1024-row chunk): fold the parts'
//           statistics into each head's LSE (a wave per head, lanes over
//           the parts) and write A = gamma * [A_prev, 0] +
//           mean_g exp2(l_g - LSE_g).
//   evict   one 1024-lane workgroup per cache: radix select of the N largest
//           A among the middle rows (four 8-bit digit passes over
//           order-preserving u32 keys), then an ordered compaction that
//           lists the kept positions ascending, equal keys taken lowest
//           position first.
//   gather  K, V rows and A entries of the kept positions into the output
//           buffers, 16 bytes per lane.
// The decode step reads each cache once for the logits and once for the
// gather; the logits round trip (G x n floats) stays far below the cache's
// own bytes and mostly in the 256 MB infinity cache.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "../../include/kvc_voxzip.h"
#include "kvc_internal.h"


#define VZ_CHUNK 1024
#define VZ_PART 256                       // rows per logits workgroup and partial
#define VZ_THREADS 256
#define VZ_SEL_THREADS 1024
#define VZ_MAX_SEQ 64
#define VZ_MAX_CAP 65536
#define VZ_MAX_G 32

static constexpr float kVzLog2e = 1.4426950408889634f;

struct VzDesc {
  int32_t n_seq, upseq, gqa, d, dtype, n_sink;
  int32_t n_units, nch;             // nch = chunks per cache at capacity
  int32_t npart;                    // VZ_PART-row parts per cache at capacity
  float gamma;
  int64_t cap;
  int64_t ks[2], vs[2];             // element strides: cache, row
  int32_t len[VZ_MAX_SEQ];          // n of every cache of sequence i
  int32_t budget[VZ_MAX_SEQ];       // B
  int32_t recent[VZ_MAX_SEQ];       // M
  int32_t mid[VZ_MAX_SEQ];          // N
};

// ---------------------------------------------------------------------------
// Logits and part statistics
// ---------------------------------------------------------------------------
// Fold (m2, z2) into (m, z): z = sum of exp2(l - m) over the values seen.
__device__ inline void vz_merge(float& m, float& z, float m2, float z2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  const float a = (m == -INFINITY) ? 0.f : z * exp2f(m - mm);
  const float b = (m2 == -INFINITY) ? 0.f : z2 * exp2f(m2 - mm);
  m = mm;
  z = a + b;
}

typedef __bf16 vz_bf16x8v __attribute__((ext_vector_type(8)));
typedef float vz_f4 __attribute__((ext_vector_type(4)));

// Wave w takes rows row0 + 64 w .. +63 of the part in four groups of 16.  A
// group's logits are one v_mfma_f32_16x16x32_bf16 chain per 16 query heads:
// lane l supplies head (A) or row (B) l % 16 and, at k-step ks, head dims
// ks*32 + (l/16)*8 .. +7 of both operands (so a row is read as 64-byte
// runs); output lane l holds row l % 16 for heads (l/16)*4 .. +3 of the
// block.  Rows past n read row n - 1 and are masked.
// STAGED (the in-place step, where nothing reads the rows again): every load
// instruction reads whole rows (PPR lanes per row, full 128-byte lines) with
// non-temporal loads into LDS, and each lane then reads its fragments in the
// MFMA layout from rows padded by 16 bytes.  Otherwise (the compacting step,
// whose gather re-reads nearly every row right after and finds part of them
// still in the caches) each lane loads its fragments straight from memory.
template <int D, bool STAGED>
__global__ __launch_bounds__(VZ_THREADS) void vz_logits_bf16_kernel(
    VzDesc V, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    float* __restrict__ lg, float2* __restrict__ part) {
  constexpr int KS = D / 32;
  constexpr int NWV = VZ_THREADS / 64;
  constexpr int PPR = D / 8, RPI = 64 / PPR, NLD = 64 / RPI;   // pieces per row, rows per load, loads
  constexpr int RS = 2 * D + 16;                                 // padded LDS row stride, bytes
  __shared__ float2 sst[VZ_MAX_G][NWV];
  const int u = blockIdx.x, pi = blockIdx.y;
  const int seq = u / V.upseq;
  const int n = V.len[seq];
  const int row0 = pi * VZ_PART;
  if (row0 >= n) return;
  const int G = V.gqa;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const float c = kVzLog2e / sqrtf((float)D);
  const uint16_t* qs = q + (size_t)u * G * D;
  vz_bf16x8v qa[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = qb * 16 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // heads past G: the last head's bits masked to zero (no branch)
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
  const uint16_t* kc = k + (int64_t)u * V.ks[0];
  float* lgu = lg + (size_t)u * G * V.cap;
  const int j0 = row0 + wave * 64;
  // Rows past n reload row n - 1 (masked below).
  uint4 kraw[4][KS];
  if constexpr (STAGED) {
    __shared__ __attribute__((aligned(16))) char sKr[NWV][64 * RS];
    const int pc = lane % PPR;
    uint4 kl[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int j = min(j0 + i * RPI + lane / PPR, n - 1);
      kl[i] = kvc_nt_load16(kc + (int64_t)j * V.ks[1] + pc * 8);
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i)
      *reinterpret_cast<uint4*>(sKr[wave] + (i * RPI + lane / PPR) * RS + pc * 16) = kl[i];
    __syncthreads();
#pragma unroll
    for (int kg = 0; kg < 4; ++kg)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kraw[kg][ks] = *reinterpret_cast<const uint4*>(sKr[wave] + (kg * 16 + col) * RS + (ks * 32 + grp * 8) * 2);
  } else {
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int j = min(j0 + kg * 16 + col, n - 1);
      const uint16_t* kr = kc + (int64_t)j * V.ks[1] + grp * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kraw[kg][ks] = *reinterpret_cast<const uint4*>(kr + ks * 32);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  vz_f4 acc[2][4];
#pragma unroll
  for (int kg = 0; kg < 4; ++kg) {
    vz_bf16x8v kb[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) __builtin_memcpy(&kb[ks], &kraw[kg][ks], 16);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      vz_f4 t = {0.f, 0.f, 0.f, 0.f};
      if (qb == 0 || two)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[qb][ks], kb[ks], t, 0, 0, 0);
      acc[qb][kg] = t;
    }
  }
  // Logits out; the wave's (max, sum exp2) per head over its 64 rows: the
  // lane's four rows, then the 16 lanes of its group.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (qb == 1 && !two) break;   // (uniform: no second block of heads)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = qb * 16 + grp * 4 + i;
      float l2[4], mx = -INFINITY;
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const int j = j0 + kg * 16 + col;
        l2[kg] = acc[qb][kg][i] * c;
        if (j < n) {
          mx = fmaxf(mx, l2[kg]);
          if (g < G) lgu[(size_t)g * V.cap + j] = l2[kg];
        }
      }
      mx = kvc_row16_max(mx);
      float z = 0.f;
#pragma unroll
      for (int kg = 0; kg < 4; ++kg)
        if (j0 + kg * 16 + col < n) z += exp2f(l2[kg] - mx);
      z = kvc_row16_sum(z);
      if (col == 0 && g < G) sst[g][wave] = make_float2(mx, z);
    }
  }
  // A wave with no rows in the part leaves (-inf, 0), which folds as empty.
  __syncthreads();
  if ((int)threadIdx.x < G) {
    float mm = -INFINITY, zz = 0.f;
    for (int w = 0; w < NWV; ++w) vz_merge(mm, zz, sst[threadIdx.x][w].x, sst[threadIdx.x][w].y);
    part[((size_t)u * V.npart + pi) * G + threadIdx.x] = make_float2(mm, zz);
  }
}

// fp32 inputs: one row per thread per pass, the G dot products in fp64.
template <int D>
__global__ __launch_bounds__(VZ_THREADS) void vz_logits_f32_kernel(
    VzDesc V, const float* __restrict__ q, const float* __restrict__ k,
    float* __restrict__ lg, float2* __restrict__ part) {
  const int u = blockIdx.x, pi = blockIdx.y;
  const int seq = u / V.upseq;
  const int n = V.len[seq];
  const int row0 = pi * VZ_PART;
  if (row0 >= n) return;
  const int G = V.gqa;
  __shared__ float sq[VZ_MAX_G * D];
  for (int i = threadIdx.x; i < G * D; i += VZ_THREADS) sq[i] = q[(size_t)u * G * D + i];
  __syncthreads();
  const double c = 1.4426950408889634 / sqrt((double)D);
  const float* kc = k + (int64_t)u * V.ks[0];
  float* lgu = lg + (size_t)u * G * V.cap;
  const int wave = threadIdx.x >> 6;
  __shared__ float2 sst[4][VZ_MAX_G];
  for (int g = 0; g < G; ++g) {
    float m = -INFINITY, z = 0.f;
    for (int r = row0 + threadIdx.x; r < n && r < row0 + VZ_PART; r += VZ_THREADS) {
      const float* kp = kc + (int64_t)r * V.ks[1];
      double dot = 0.0;
#pragma unroll 8
      for (int e = 0; e < D; ++e) dot = fma((double)sq[g * D + e], (double)kp[e], dot);
      const float l2 = (float)(dot * c);
      lgu[(size_t)g * V.cap + r] = l2;
      vz_merge(m, z, l2, 1.f);
    }
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m, o);
      const float z2 = __shfl_xor(z, o);
      vz_merge(m, z, m2, z2);
    }
    if ((threadIdx.x & 63) == 0) sst[wave][g] = make_float2(m, z);
  }
  __syncthreads();
  if ((int)threadIdx.x < G) {
    float mm = -INFINITY, zz = 0.f;
    for (int w = 0; w < 4; ++w) vz_merge(mm, zz, sst[w][threadIdx.x].x, sst[w][threadIdx.x].y);
    part[((size_t)u * V.npart + pi) * G + threadIdx.x] = make_float2(mm, zz);
  }
}

// ---------------------------------------------------------------------------
// A = gamma * [A_prev, 0] + mean over heads of exp2(l - LSE)
// ---------------------------------------------------------------------------
// INPLACE: a_prev and a_t are one buffer indexed by cache slot, and every
// slot's previous value is decayed (the step that freed a slot for the new
// token zeroed it); otherwise row n-1 is the new token, which has none.
template <bool INPLACE>
__global__ __launch_bounds__(VZ_THREADS) void vz_accum_kernel(
    VzDesc V, const float* __restrict__ lg, const float2* __restrict__ part,
    const float* a_prev, float* a_t) {
  const int u = blockIdx.x, chunk = blockIdx.y;
  const int seq = u / V.upseq;
  const int n = V.len[seq];
  const int row0 = chunk * VZ_CHUNK;
  if (row0 >= n) return;
  const int G = V.gqa;
  __shared__ float lse[VZ_MAX_G];
  // Each head's LSE: a wave per head, lanes over the parts.
  {
    const int np = (n + VZ_PART - 1) / VZ_PART;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int g = wave; g < G; g += VZ_THREADS / 64) {
      float m = -INFINITY, z = 0.f;
      for (int p = lane; p < np; p += 64) {
        const float2 pp = part[((size_t)u * V.npart + p) * G + g];
        vz_merge(m, z, pp.x, pp.y);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float m2 = __shfl_xor(m, o), z2 = __shfl_xor(z, o);
        vz_merge(m, z, m2, z2);
      }
      if (lane == 0) lse[g] = m + log2f(z);
    }
  }
  __syncthreads();
  const float inv_g = 1.0f / (float)G;
  const float* lgu = lg + (size_t)u * G * V.cap;
  const float* ap = a_prev + (size_t)u * V.cap;
  float* at = a_t + (size_t)u * V.cap;
  const int rend = min(n, row0 + VZ_CHUNK);
  for (int r = row0 + threadIdx.x; r < rend; r += VZ_THREADS) {
    // the heads' terms in head order, eight heads' loads in flight at a time
    float s = 0.f;
    int g = 0;
    for (; g + 8 <= G; g += 8) {
      float l[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) l[i] = lgu[(size_t)(g + i) * V.cap + r];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += exp2f(l[i] - lse[g + i]);
    }
    for (; g < G; ++g) s += exp2f(lgu[(size_t)g * V.cap + r] - lse[g]);
    const float prev = (INPLACE || r < n - 1) ? V.gamma * ap[r] : 0.f;
    at[r] = prev + s * inv_g;
  }
}

// ---------------------------------------------------------------------------
// Eviction: N largest A among [T, n - M), positions ascending
// ---------------------------------------------------------------------------
// Order-preserving key of a float (-0.0 first mapped to +0.0).
__device__ inline uint32_t vz_key(float x) {
  const uint32_t b = __float_as_uint(x + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Exclusive prefix count of `flag` over the workgroup in thread order, and
// the total.  Two barriers; `scratch` holds one count per wave.
__device__ inline int vz_block_scan(bool flag, int* scratch, int* total) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long m = __ballot(flag);
  const int before = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) scratch[wave] = __popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < VZ_SEL_THREADS / 64; ++w) {
    const int c = scratch[w];
    off += w < wave ? c : 0;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + before;
}

__global__ __launch_bounds__(VZ_SEL_THREADS) void vz_evict_kernel(
    VzDesc V, const float* __restrict__ a_t, int32_t* __restrict__ idx) {
  const int u = blockIdx.x;
  const int seq = u / V.upseq;
  const int n = V.len[seq], B = V.budget[seq];
  int32_t* ix = idx + (size_t)u * V.cap;
  const int tid = threadIdx.x;
  if (n <= B) {
    for (int t = tid; t < n; t += VZ_SEL_THREADS) ix[t] = t;
    return;
  }
  const int T = V.n_sink, M = V.recent[seq], N = V.mid[seq];
  for (int t = tid; t < T; t += VZ_SEL_THREADS) ix[t] = t;
  for (int t = tid; t < M; t += VZ_SEL_THREADS) ix[T + N + t] = n - M + t;
  if (N == 0) return;
  const float* x = a_t + (size_t)u * V.cap;
  const int lo = T, hi = n - M;                 // candidates [lo, hi), hi - lo > N

  __shared__ uint32_t hist[VZ_SEL_THREADS / 64][256];
  __shared__ uint32_t s_digit, s_above;
  __shared__ int scan_a[VZ_SEL_THREADS / 64], scan_b[VZ_SEL_THREADS / 64];
  const int wave = tid >> 6, lane = tid & 63;
  uint32_t prefix = 0, pmask = 0;
  uint32_t want = (uint32_t)N;                  // rank still to place, 1-based
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = lane; b < 256; b += 64) hist[wave][b] = 0;
    __syncthreads();
    for (int j = lo + tid; j < hi; j += VZ_SEL_THREADS) {
      const uint32_t key = vz_key(x[j]);
      if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // Lane l owns bins 255-4l .. 252-4l (descending); counts summed over
      // the waves, then an inclusive scan from the top bin down.
      uint32_t c4[4], own = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 255 - 4 * lane - e;
        uint32_t s = 0;
        for (int w = 0; w < VZ_SEL_THREADS / 64; ++w) s += hist[w][b];
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
      if (excl < want && want <= incl) {
        uint32_t run = excl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (run < want && want <= run + c4[e]) {
            s_digit = (uint32_t)(255 - 4 * lane - e);
            s_above = run;
          }
          run += c4[e];
        }
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    want -= s_above;
    __syncthreads();
  }
  // Keys above `prefix` are all kept, plus the first `want` equal ones.
  const uint32_t kth = prefix;
  int taken = 0, eq_seen = 0;
  for (int base = lo; base < hi; base += VZ_SEL_THREADS) {
    const int j = base + tid;
    const bool valid = j < hi;
    const uint32_t key = valid ? vz_key(x[j]) : 0u;
    const bool gt = valid && key > kth;
    const bool eq = valid && key == kth;
    int eq_tot, take_tot;
    const int eq_rank = vz_block_scan(eq, scan_a, &eq_tot) + eq_seen;
    const bool take = gt || (eq && eq_rank < (int)want);
    const int pos = vz_block_scan(take, scan_b, &take_tot) + taken;
    if (take) ix[T + pos] = j;
    eq_seen += eq_tot;
    taken += take_tot;
  }
}

// ---------------------------------------------------------------------------
// Eviction in place (kvc_vz_step_inplace): at most one row leaves a cache per
// step, so the kept rows stay in their slots and only the leaving row's slot
// changes hands.  Slot s of cache u holds the row whose place in the
// page's concatenated order is pos[s] (older rows lower); with one row in
// and one out per step, the T sinks are the T lowest places and the M
// recent rows the M highest, and the middle row to drop is the one of
// smallest A, the latest place among equal values (the complement of the
// N kept).  The freed slot gets A = 0 and the next place, ready for the
// next token's row.  One 1024-thread workgroup per cache, eight slots' loads
// in flight per thread in each pass.
// ---------------------------------------------------------------------------
__device__ inline void vz_min_pair(unsigned long long& k, int& s, unsigned long long k2, int s2) {
  if (k2 < k) {
    k = k2;
    s = s2;
  }
}

#define VZ_EVICT_T 1024
#define VZ_EVICT_KB 8
__global__ __launch_bounds__(VZ_EVICT_T) void vz_slot_evict_kernel(VzDesc V, float* a,
                                                                   int32_t* pos,
                                                                   int32_t* free_slot) {
  constexpr int NW = VZ_EVICT_T / 64, KB = VZ_EVICT_KB;
  __shared__ int s_min[NW], s_max[NW];
  __shared__ unsigned long long s_key[NW];
  __shared__ int s_slot[NW];
  const int u = blockIdx.x, seq = u / V.upseq;
  const int n = V.len[seq], B = V.budget[seq];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float* au = a + (size_t)u * V.cap;
  int32_t* pu = pos + (size_t)u * V.cap;
  // lowest and highest place
  int pmin = INT32_MAX, pmax = INT32_MIN;
  for (int s0 = tid; s0 < n; s0 += KB * VZ_EVICT_T) {
    int p[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) p[i] = pu[min(s0 + i * VZ_EVICT_T, n - 1)];   // (clamped)
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      pmin = min(pmin, p[i]);
      pmax = max(pmax, p[i]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    pmin = min(pmin, __shfl_xor(pmin, o));
    pmax = max(pmax, __shfl_xor(pmax, o));
  }
  if (lane == 0) {
    s_min[wave] = pmin;
    s_max[wave] = pmax;
  }
  __syncthreads();
  pmin = s_min[0];
  pmax = s_max[0];
  for (int w = 1; w < NW; ++w) {
    pmin = min(pmin, s_min[w]);
    pmax = max(pmax, s_max[w]);
  }
  int out = -1;
  if (n > B) {
    // middle places: not among the T lowest nor the M highest
    const int T = V.n_sink, M = V.recent[seq];
    unsigned long long best = ~0ull;
    int bslot = -1;
    for (int s0 = tid; s0 < n; s0 += KB * VZ_EVICT_T) {
      int p[KB];
      float av[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const int s = min(s0 + i * VZ_EVICT_T, n - 1);   // (clamped; masked below)
        p[i] = pu[s];
        av[i] = au[s];
      }
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const int s = s0 + i * VZ_EVICT_T;
        if (s >= n || p[i] - pmin < T || p[i] > pmax - M) continue;
        // smallest A first; among equal A the latest place (largest p)
        const unsigned long long key =
            ((unsigned long long)vz_key(av[i]) << 32) | (unsigned long long)(~(uint32_t)p[i]);
        vz_min_pair(best, bslot, key, s);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const unsigned long long k2 = __shfl_xor(best, o);
      const int s2 = __shfl_xor(bslot, o);
      vz_min_pair(best, bslot, k2, s2);
    }
    if (lane == 0) {
      s_key[wave] = best;
      s_slot[wave] = bslot;
    }
    __syncthreads();
    best = s_key[0];
    bslot = s_slot[0];
    for (int w = 1; w < NW; ++w) vz_min_pair(best, bslot, s_key[w], s_slot[w]);
    out = bslot;
  } else if (n < V.cap) {
    out = n;                                  // the cache still grows: next slot
  }
  if (tid == 0) {
    if (out >= 0) {
      au[out] = 0.0f;
      pu[out] = pmax + 1;
    }
    free_slot[u] = out;
  }
}

// ---------------------------------------------------------------------------
// Gather kept rows of K, V and entries of A
// ---------------------------------------------------------------------------
// One workgroup per (cache, run of 64 output rows for 256-byte rows), the
// runs of a cache consecutive in dispatch order so that neighbouring
// workgroups stream neighbouring rows; the output is written with
// non-temporal stores (it is not read again here).
template <int ROWB>
__global__ __launch_bounds__(VZ_THREADS) void vz_gather_kernel(
    VzDesc V, int blocks_per_cache, const char* __restrict__ k, const char* __restrict__ v,
    const float* __restrict__ a_t, const int32_t* __restrict__ idx, char* __restrict__ k_out,
    char* __restrict__ v_out, float* __restrict__ a_out) {
  constexpr int CH = ROWB / 16;
  constexpr int RPP = VZ_THREADS / CH;          // rows per pass
  constexpr int PASSES = 4;
  const int u = blockIdx.x / blocks_per_cache;
  const int t0 = (blockIdx.x - u * blocks_per_cache) * RPP * PASSES;
  const int seq = u / V.upseq;
  const int n = V.len[seq];
  const int nl = min(n, V.budget[seq]);
  if (t0 >= nl) return;
  const int esz = V.dtype == 0 ? 2 : 4;
  const int ch = threadIdx.x % CH;
  const int32_t* ix = idx + (size_t)u * V.cap;
  uint4 kv[PASSES], vv[PASSES];
  int src[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + p * RPP + threadIdx.x / CH;
    src[p] = 0;
    if (t >= nl) continue;
    int s = ix[t];
    if ((unsigned)s >= (unsigned)n) s = 0;
    src[p] = s;
    kv[p] = kvc_nt_load16(k + (u * V.ks[0] + s * V.ks[1]) * esz + ch * 16);
    vv[p] = kvc_nt_load16(v + (u * V.vs[0] + s * V.vs[1]) * esz + ch * 16);
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int t = t0 + p * RPP + threadIdx.x / CH;
    if (t >= nl) continue;
    uint4* ko = reinterpret_cast<uint4*>(k_out + (u * V.ks[0] + (int64_t)t * V.ks[1]) * esz + ch * 16);
    uint4* vo = reinterpret_cast<uint4*>(v_out + (u * V.vs[0] + (int64_t)t * V.vs[1]) * esz + ch * 16);
    __builtin_nontemporal_store(kv[p].x, &ko->x);
    __builtin_nontemporal_store(kv[p].y, &ko->y);
    __builtin_nontemporal_store(kv[p].z, &ko->z);
    __builtin_nontemporal_store(kv[p].w, &ko->w);
    __builtin_nontemporal_store(vv[p].x, &vo->x);
    __builtin_nontemporal_store(vv[p].y, &vo->y);
    __builtin_nontemporal_store(vv[p].z, &vo->z);
    __builtin_nontemporal_store(vv[p].w, &vo->w);
    if (ch == 0)
      __builtin_nontemporal_store(a_t[(size_t)u * V.cap + src[p]], &a_out[(size_t)u * V.cap + t]);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static kvc_status vz_hip(hipError_t e) {
  if (e == hipSuccess) return KVC_OK;
  kvc_note_hip_error((int)e);
  return KVC_ERR_HIP;
}

static size_t vz_up(size_t x) { return (x + 255) & ~size_t(255); }

static kvc_status vz_desc(const kvc_vz_problem* p, const kvc_vz_params* prm, VzDesc* V) {
  if (!p || !prm || !V || !p->len || !p->budget) return KVC_ERR_INVALID_ARG;
  if (p->n_seq < 1 || p->n_layers < 1 || p->n_kv_heads < 1 || p->gqa_group < 1 ||
      p->head_dim < 1 || p->capacity < 1)
    return KVC_ERR_INVALID_ARG;
  if (p->dtype != KVC_BF16 && p->dtype != KVC_F32) return KVC_ERR_INVALID_ARG;
  if (!(prm->gamma >= 0.0 && prm->gamma < INFINITY)) return KVC_ERR_INVALID_ARG;
  if (!(prm->recent_frac >= 0.0 && prm->recent_frac <= 1.0) || prm->n_sink < 0)
    return KVC_ERR_INVALID_ARG;
  const int esz = p->dtype == KVC_BF16 ? 2 : 4;
  for (int a = 0; a < 2; ++a) {
    if (p->k_stride[a] < 0 || p->v_stride[a] < 0) return KVC_ERR_INVALID_ARG;
    if ((p->k_stride[a] * esz) % 16 || (p->v_stride[a] * esz) % 16) return KVC_ERR_INVALID_ARG;
  }
  if (p->k_stride[1] < p->head_dim || p->v_stride[1] < p->head_dim) return KVC_ERR_INVALID_ARG;
  if (p->k_stride[0] < p->k_stride[1] * p->capacity || p->v_stride[0] < p->v_stride[1] * p->capacity)
    return KVC_ERR_INVALID_ARG;
  if (p->n_seq > VZ_MAX_SEQ || p->capacity > VZ_MAX_CAP) return KVC_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return KVC_ERR_UNSUPPORTED;
  if (p->gqa_group > VZ_MAX_G) return KVC_ERR_UNSUPPORTED;
  const int64_t upseq = (int64_t)p->n_layers * p->n_kv_heads;
  if (upseq > KVC_MAX_UNITS_PER_SEQ) return KVC_ERR_UNSUPPORTED;
  memset(V, 0, sizeof(*V));
  for (int i = 0; i < p->n_seq; ++i) {
    const int64_t n = p->len[i], B = p->budget[i];
    if (n < 1 || n > p->capacity || B < 1) return KVC_ERR_INVALID_ARG;
    const int64_t M = (int64_t)floor(prm->recent_frac * (double)B);
    const int64_t N = B - prm->n_sink - M;
    if (N < 0) return KVC_ERR_BUDGET;
    V->len[i] = (int32_t)n;
    V->budget[i] = (int32_t)B;
    V->recent[i] = (int32_t)M;
    V->mid[i] = (int32_t)N;
  }
  V->n_seq = p->n_seq;
  V->upseq = (int32_t)upseq;
  V->gqa = p->gqa_group;
  V->d = p->head_dim;
  V->dtype = p->dtype == KVC_BF16 ? 0 : 1;
  V->n_sink = prm->n_sink;
  V->n_units = (int32_t)(upseq * p->n_seq);
  V->cap = p->capacity;
  V->nch = (int32_t)((p->capacity + VZ_CHUNK - 1) / VZ_CHUNK);
  V->npart = (int32_t)((p->capacity + VZ_PART - 1) / VZ_PART);
  V->gamma = (float)prm->gamma;
  for (int a = 0; a < 2; ++a) {
    V->ks[a] = p->k_stride[a];
    V->vs[a] = p->v_stride[a];
  }
  return KVC_OK;
}

struct VzCarve {
  float* lg;
  float2* part;
  float* a_t;
};

static size_t vz_ws_logits(const VzDesc& V) {
  return vz_up(sizeof(float) * (size_t)V.n_units * V.gqa * V.cap) +
         vz_up(sizeof(float2) * (size_t)V.n_units * V.npart * V.gqa);
}

static VzCarve vz_carve(const VzDesc& V, void* ws) {
  VzCarve c;
  char* p = (char*)ws;
  c.lg = (float*)p;
  p += vz_up(sizeof(float) * (size_t)V.n_units * V.gqa * V.cap);
  c.part = (float2*)p;
  p += vz_up(sizeof(float2) * (size_t)V.n_units * V.npart * V.gqa);
  c.a_t = (float*)p;
  return c;
}

static bool vz_a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static hipError_t vz_launch_accumulate(const VzDesc& V, const void* q, const void* k,
                                       const float* a_prev, float* a_t, const VzCarve& c,
                                       hipStream_t st) {
  const dim3 pgrid(V.n_units, V.npart), grid(V.n_units, V.nch);
  if (V.dtype == 0) {
    const uint16_t* qq = (const uint16_t*)q;
    const uint16_t* kk = (const uint16_t*)k;
    const bool inplace = a_prev == a_t;
    if (V.d == 128 && inplace)
      hipLaunchKernelGGL((vz_logits_bf16_kernel<128, true>), pgrid, dim3(VZ_THREADS), 0, st, V, qq, kk, c.lg, c.part);
    else if (V.d == 128)
      hipLaunchKernelGGL((vz_logits_bf16_kernel<128, false>), pgrid, dim3(VZ_THREADS), 0, st, V, qq, kk, c.lg, c.part);
    else if (inplace)
      hipLaunchKernelGGL((vz_logits_bf16_kernel<64, true>), pgrid, dim3(VZ_THREADS), 0, st, V, qq, kk, c.lg, c.part);
    else
      hipLaunchKernelGGL((vz_logits_bf16_kernel<64, false>), pgrid, dim3(VZ_THREADS), 0, st, V, qq, kk, c.lg, c.part);
  } else {
    const float* qq = (const float*)q;
    const float* kk = (const float*)k;
    if (V.d == 128)
      hipLaunchKernelGGL((vz_logits_f32_kernel<128>), pgrid, dim3(VZ_THREADS), 0, st, V, qq, kk, c.lg, c.part);
    else
      hipLaunchKernelGGL((vz_logits_f32_kernel<64>), pgrid, dim3(VZ_THREADS), 0, st, V, qq, kk, c.lg, c.part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a_prev == a_t)
    hipLaunchKernelGGL(vz_accum_kernel<true>, grid, dim3(VZ_THREADS), 0, st, V,
                       (const float*)c.lg, (const float2*)c.part, a_prev, a_t);
  else
    hipLaunchKernelGGL(vz_accum_kernel<false>, grid, dim3(VZ_THREADS), 0, st, V,
                       (const float*)c.lg, (const float2*)c.part, a_prev, a_t);
  return hipGetLastError();
}

static hipError_t vz_launch_evict(const VzDesc& V, const float* a_t, int32_t* idx, hipStream_t st) {
  hipLaunchKernelGGL(vz_evict_kernel, dim3(V.n_units), dim3(VZ_SEL_THREADS), 0, st, V, a_t, idx);
  return hipGetLastError();
}

static hipError_t vz_launch_gather(const VzDesc& V, const void* k, const void* v, const float* a_t,
                                   const int32_t* idx, void* k_out, void* v_out, float* a_out,
                                   hipStream_t st) {
  const int rowb = V.d * (V.dtype == 0 ? 2 : 4);
  int maxnl = 1;
  for (int i = 0; i < V.n_seq; ++i) maxnl = std::max(maxnl, std::min(V.len[i], V.budget[i]));
  const int rows_per_block = (VZ_THREADS / (rowb / 16)) * 4;
  const int bpc = (maxnl + rows_per_block - 1) / rows_per_block;
  const dim3 grid((unsigned)((int64_t)V.n_units * bpc));
  const char* kc = (const char*)k;
  const char* vc = (const char*)v;
  char* ko = (char*)k_out;
  char* vo = (char*)v_out;
  switch (rowb) {
    case 128: hipLaunchKernelGGL((vz_gather_kernel<128>), grid, dim3(VZ_THREADS), 0, st, V, bpc, kc, vc, a_t, idx, ko, vo, a_out); break;
    case 256: hipLaunchKernelGGL((vz_gather_kernel<256>), grid, dim3(VZ_THREADS), 0, st, V, bpc, kc, vc, a_t, idx, ko, vo, a_out); break;
    default: hipLaunchKernelGGL((vz_gather_kernel<512>), grid, dim3(VZ_THREADS), 0, st, V, bpc, kc, vc, a_t, idx, ko, vo, a_out); break;
  }
  return hipGetLastError();
}

extern "C" kvc_status kvc_vz_plan(const kvc_vz_problem* prob, const kvc_vz_params* params,
                                  int64_t* new_len, size_t* workspace_bytes) {
  VzDesc V;
  const kvc_status st = vz_desc(prob, params, &V);
  if (st != KVC_OK) return st;
  if (new_len)
    for (int i = 0; i < V.n_seq; ++i) new_len[i] = std::min(V.len[i], V.budget[i]);
  if (workspace_bytes)
    *workspace_bytes = vz_ws_logits(V) + vz_up(sizeof(float) * (size_t)V.n_units * V.cap);
  return KVC_OK;
}

extern "C" kvc_status kvc_vz_accumulate(const kvc_vz_problem* prob, const kvc_vz_params* params,
                                        const void* q, const void* k, const float* a_prev,
                                        float* a, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  VzDesc V;
  const kvc_status st = vz_desc(prob, params, &V);
  if (st != KVC_OK) return st;
  if (!q || !k || !a_prev || !a || !workspace) return KVC_ERR_INVALID_ARG;
  if (!vz_a16(q) || !vz_a16(k) || ((uintptr_t)workspace & 255u) || ((uintptr_t)a & 3u) ||
      ((uintptr_t)a_prev & 3u))
    return KVC_ERR_INVALID_ARG;
  if (workspace_bytes < vz_ws_logits(V)) return KVC_ERR_WORKSPACE;
  return vz_hip(vz_launch_accumulate(V, q, k, a_prev, a, vz_carve(V, workspace),
                                     (hipStream_t)stream));
}

extern "C" kvc_status kvc_vz_evict(const kvc_vz_problem* prob, const kvc_vz_params* params,
                                   const float* a, int32_t* idx_out, void* stream) {
  VzDesc V;
  const kvc_status st = vz_desc(prob, params, &V);
  if (st != KVC_OK) return st;
  if (!a || !idx_out || ((uintptr_t)a & 3u) || ((uintptr_t)idx_out & 3u)) return KVC_ERR_INVALID_ARG;
  return vz_hip(vz_launch_evict(V, a, idx_out, (hipStream_t)stream));
}

extern "C" kvc_status kvc_vz_gather(const kvc_vz_problem* prob, const kvc_vz_params* params,
                                    const void* k, const void* v, const float* a,
                                    const int32_t* idx, void* k_out, void* v_out, float* a_out,
                                    void* stream) {
  VzDesc V;
  const kvc_status st = vz_desc(prob, params, &V);
  if (st != KVC_OK) return st;
  if (!k || !v || !a || !idx || !k_out || !v_out || !a_out) return KVC_ERR_INVALID_ARG;
  if (!vz_a16(k) || !vz_a16(v) || !vz_a16(k_out) || !vz_a16(v_out) || ((uintptr_t)a & 3u) ||
      ((uintptr_t)a_out & 3u) || ((uintptr_t)idx & 3u))
    return KVC_ERR_INVALID_ARG;
  return vz_hip(vz_launch_gather(V, k, v, a, idx, k_out, v_out, a_out, (hipStream_t)stream));
}

extern "C" kvc_status kvc_vz_step(const kvc_vz_problem* prob, const kvc_vz_params* params,
                                  const void* q, const void* k, const void* v,
                                  const float* a_prev, void* k_out, void* v_out, float* a_out,
                                  int32_t* idx_out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  VzDesc V;
  const kvc_status st = vz_desc(prob, params, &V);
  if (st != KVC_OK) return st;
  if (!q || !k || !v || !a_prev || !k_out || !v_out || !a_out || !idx_out || !workspace)
    return KVC_ERR_INVALID_ARG;
  if (!vz_a16(q) || !vz_a16(k) || !vz_a16(v) || !vz_a16(k_out) || !vz_a16(v_out) ||
      ((uintptr_t)workspace & 255u) || ((uintptr_t)a_prev & 3u) || ((uintptr_t)a_out & 3u) ||
      ((uintptr_t)idx_out & 3u))
    return KVC_ERR_INVALID_ARG;
  const size_t need = vz_ws_logits(V) + vz_up(sizeof(float) * (size_t)V.n_units * V.cap);
  if (workspace_bytes < need) return KVC_ERR_WORKSPACE;
  const VzCarve c = vz_carve(V, workspace);
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = vz_launch_accumulate(V, q, k, a_prev, c.a_t, c, s);
  if (e == hipSuccess) e = vz_launch_evict(V, c.a_t, idx_out, s);
  if (e == hipSuccess) e = vz_launch_gather(V, k, v, c.a_t, idx_out, k_out, v_out, a_out, s);
  return vz_hip(e);
}

extern "C" kvc_status kvc_vz_step_inplace(const kvc_vz_problem* prob,
                                          const kvc_vz_params* params, const void* q,
                                          const void* k, float* a, int32_t* pos,
                                          int32_t* free_slot, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  VzDesc V;
  const kvc_status st = vz_desc(prob, params, &V);
  if (st != KVC_OK) return st;
  if (!q || !k || !a || !pos || !free_slot || !workspace) return KVC_ERR_INVALID_ARG;
  if (!vz_a16(q) || !vz_a16(k) || ((uintptr_t)workspace & 255u) || ((uintptr_t)a & 3u) ||
      ((uintptr_t)pos & 3u) || ((uintptr_t)free_slot & 3u))
    return KVC_ERR_INVALID_ARG;
  for (int i = 0; i < V.n_seq; ++i)
    if (V.len[i] > V.budget[i] + 1) return KVC_ERR_UNSUPPORTED;  // one row out per step
  if (workspace_bytes < vz_ws_logits(V)) return KVC_ERR_WORKSPACE;
  const VzCarve c = vz_carve(V, workspace);
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = vz_launch_accumulate(V, q, k, a, a, c, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(vz_slot_evict_kernel, dim3(V.n_units), dim3(VZ_EVICT_T), 0, s, V, a, pos,
                       free_slot);
    e = hipGetLastError();
  }
  return vz_hip(e);
}
