// sss_select.hip -- Spectral Score Smoothing (step 2) and per-head top-k
// selection (step 4), one 1024-thread workgroup per unit.
//
// AudioKV article, section 2.2: F = rfft(s) of the length-L score row; the
// cumulative energy E(k) = sum_{i<=k} |F_i|^2; the smallest k* with
// E(k*) >= rho E(L/2); a low-pass mask keeping bins 0..k*; the blend
// s_hat = (1 - alpha) s + alpha irfft(F masked).  The article runs the FFTs
// with cuFFT; here they are hand-written for one gfx950 workgroup:
//
//  * The real length-L transform is a complex length-N = L/2 transform of
//    z_m = s_{2m} + i s_{2m+1}, split into the real spectrum afterwards
//    (and merged back before the inverse).
//  * Complex FFTs use the Stockham autosort formulation (each radix-R pass
//    reads x[j + r N/R] and writes its R outputs to (j - j mod Ns) R +
//    j mod Ns + m Ns, natural order after the last pass; Govindaraju et al.,
//    SC 2008).  Every thread keeps V = 8, 16 or 32 values in registers and
//    runs radix-V butterflies on them; passes exchange data through one
//    LDS buffer (N complex values, or for N = 32768 (L = 65536) N floats
//    with the real and imaginary parts in turn, 128 KiB), so every length
//    fits one workgroup without a multi-pass global variant.  The buffer is
//    not padded: the first pass's strided writes conflict on LDS banks
//    (counters: about 3 conflict cycles per LDS instruction over the
//    kernel at L = 32768), but one pad slot per 16 pairs, as tried, made
//    the addresses nonlinear in the slot index and raised the register
//    spills at L = 32768 from 10 to 55 VGPRs per lane.
//  * E(k) is summed in fp64 from the fp32 spectrum; k* is the first bin
//    whose prefix reaches rho E(N), found with a block scan.
//
// Selection (step 4): the b_u - w largest s_hat among positions [0, L-w)
// plus the window [L-w, L), ascending.  s_hat is mapped to order-preserving
// 32-bit keys (-0 folded into +0); a bitwise search for the largest key T
// with count(key >= T) >= k finds the k-th largest value, positions equal to
// T are taken from the lowest position upward, and a block scan writes the
// kept positions in ascending order.  Each thread transposes its keys into
// 32-bit planes once (bit s of plane b = bit b of its key s), so a round of
// the search costs a popcount per 32 keys instead of 32 compares, and the
// search leaves the masks of the keys above and equal to T.
#include "kvc_internal.h"

#define SSS_T KVC_SSS_THREADS
#define SSS_WAVES (SSS_T / 64)

// e^{-2 pi i m / 32} for m = 0..15: cos and sin of 2 pi m / 32.
static constexpr float kCos32[16] = {
    1.0f, 0.98078528040323044913f, 0.92387953251128675613f, 0.83146961230254523708f,
    0.70710678118654752440f, 0.55557023301960222474f, 0.38268343236508977173f,
    0.19509032201612826785f, 0.0f, -0.19509032201612826785f, -0.38268343236508977173f,
    -0.55557023301960222474f, -0.70710678118654752440f, -0.83146961230254523708f,
    -0.92387953251128675613f, -0.98078528040323044913f};
static constexpr float kSin32[16] = {
    0.0f, 0.19509032201612826785f, 0.38268343236508977173f, 0.55557023301960222474f,
    0.70710678118654752440f, 0.83146961230254523708f, 0.92387953251128675613f,
    0.98078528040323044913f, 1.0f, 0.98078528040323044913f, 0.92387953251128675613f,
    0.83146961230254523708f, 0.70710678118654752440f, 0.55557023301960222474f,
    0.38268343236508977173f, 0.19509032201612826785f};


__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

template <int R>
__host__ __device__ constexpr int bitrev(int i) {
  int r = 0;
  for (int b = 1; b < R; b <<= 1) {
    r = (r << 1) | (i & 1);
    i >>= 1;
  }
  return r;
}

// In-register forward DFT of size R (power of two <= 32), natural order.
template <int R>
__device__ __forceinline__ void dft_small(float2 (&v)[R]) {
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int j = bitrev<R>(i);
    if (j > i) {
      const float2 t = v[i];
      v[i] = v[j];
      v[j] = t;
    }
  }
#pragma unroll
  for (int len = 2; len <= R; len <<= 1) {
#pragma unroll
    for (int i = 0; i < R; i += len) {
#pragma unroll
      for (int m = 0; m < len / 2; ++m) {
        const int ti = m * (32 / len);
        const float2 w = make_float2(kCos32[ti], -kSin32[ti]);
        const float2 a = v[i + m];
        const float2 b = cmul(v[i + m + len / 2], w);
        v[i + m] = make_float2(a.x + b.x, a.y + b.y);
        v[i + m + len / 2] = make_float2(a.x - b.x, a.y - b.y);
      }
    }
  }
}

// One Stockham pass of radix R on the V values a thread holds (V/R
// butterflies j = t + b T, T = N/V threads).
template <int V, int R, int T, int Ns>
__device__ __forceinline__ void fft_pass(float (&re)[V], float (&im)[V], int t) {
#pragma unroll
  for (int b = 0; b < V / R; ++b) {
    const int j = t + b * T;
    int k = j & (Ns - 1);
    // The forward and inverse transforms use the same twiddles; an empty asm
    // keeps the compiler from carrying them across the whole kernel.
    asm volatile("" : "+v"(k));
    float2 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) v[r] = make_float2(re[b * R + r], im[b * R + r]);
    if constexpr (Ns > 1) {
      // w^r, w = e^{-2 pi i k / (Ns R)}: v_sin/v_cos (which take revolutions;
      // k r / (Ns R) is an exact dyadic fraction) at every 8th power, the
      // powers in between by one complex multiply each.
      constexpr float inv = 1.0f / (float)(Ns * R);
      const float x1 = (float)k * inv;
      const float2 w1 = make_float2(__builtin_amdgcn_cosf(x1), -__builtin_amdgcn_sinf(x1));
      float2 w = w1;
#pragma unroll
      for (int r = 1; r < R; ++r) {
        if (r > 1) {
          if (r % 8 == 0) {
            const float x = (float)(k * r) * inv;
            w = make_float2(__builtin_amdgcn_cosf(x), -__builtin_amdgcn_sinf(x));
          } else {
            w = cmul(w, w1);
          }
        }
        v[r] = cmul(v[r], w);
      }
    }
    dft_small<R>(v);
#pragma unroll
    for (int m = 0; m < R; ++m) {
      re[b * R + m] = v[m].x;
      im[b * R + m] = v[m].y;
    }
  }
}

// Position of value slot s in the input of a radix-R pass, and in the output
// of a radix-R pass whose sub-transforms have length Ns.
template <int R, int T, int N>
__device__ __forceinline__ int in_index(int s, int t) {
  return t + (s / R) * T + (s % R) * (N / R);
}
template <int R, int T, int Ns>
__device__ __forceinline__ int out_index(int s, int t) {
  const int j = t + (s / R) * T;
  const int k = j & (Ns - 1);
  return (j - k) * R + k + (s % R) * Ns;
}

// Exchange through LDS: the value in slot s moves from position widx(s) to
// the slot whose position is ridx(s).  Real parts first, then imaginary
// parts.  One optional extra value per thread is written at position xw and
// one read from position xr (-1: none).
struct Extra {
  int xw, xr;
  float wre, wim, rre, rim;
};

template <int V, class WF, class RF>
__device__ __forceinline__ void exchange(float (&re)[V], float (&im)[V], float* lds, bool act,
                                         WF widx, RF ridx, Extra& x) {
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) lds[widx(s)] = re[s];
    if (x.xw >= 0) lds[x.xw] = x.wre;
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) re[s] = lds[ridx(s)];
    if (x.xr >= 0) x.rre = lds[x.xr];
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) lds[widx(s)] = im[s];
    if (x.xw >= 0) lds[x.xw] = x.wim;
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) im[s] = lds[ridx(s)];
    if (x.xr >= 0) x.rim = lds[x.xr];
  }
  __syncthreads();
}

// Same exchange with real and imaginary parts moved together (when the LDS
// buffer holds N complex values): two barriers instead of four.  PAD: see
// xchg.
template <int V, bool PAD, class WF, class RF>
__device__ __forceinline__ void exchange2(float (&re)[V], float (&im)[V], float2* lds, bool act,
                                          WF widx, RF ridx, Extra& x) {
  auto phys2 = [](int a) {
    if constexpr (!PAD) return a;
    asm volatile("" : "+v"(a));  // computed at its use, not shared across exchanges
    return a + (a >> 4);
  };
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) lds[phys2(widx(s))] = make_float2(re[s], im[s]);
    if (x.xw >= 0) lds[phys2(x.xw)] = make_float2(x.wre, x.wim);
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const float2 v = lds[phys2(ridx(s))];
      re[s] = v.x;
      im[s] = v.y;
    }
    if (x.xr >= 0) {
      const float2 v = lds[phys2(x.xr)];
      x.rre = v.x;
      x.rim = v.y;
    }
  }
  __syncthreads();
}

// LDS buffer: N complex values when they fit (N <= 16384, 128 KiB), else N
// floats with the two parts exchanged in turn.
template <int N>
struct Xbuf {
  static constexpr bool kPair = N <= 16384;
  static constexpr int kFloats = kPair ? 2 * N : N;            // positions, in floats
  static constexpr int kPhys = kPair ? kFloats + kFloats / 16 : kFloats;  // with the pads
};

// PAD: the exchange's positions sit in LDS with one unused slot after every
// 16 complex values (128 bytes, one pass over the banks).  A side of an
// exchange that steps through positions 16 apart across lanes (a first
// radix-16 pass's output) then falls on distinct banks instead of on one,
// while runs of consecutive positions stay consecutive.  The
// buffer holds data only within one exchange, so each exchange picks its
// own layout.  Which exchanges take it is chosen per kernel: the padded
// address costs registers, and these kernels sit at their register limit.
template <int N, int V, bool PAD = false, class WF, class RF>
__device__ __forceinline__ void xchg(float (&re)[V], float (&im)[V], float* lds, bool act, WF widx,
                                     RF ridx, Extra& x) {
  static_assert(!PAD || Xbuf<N>::kPair, "the padded layout is for complex-pair buffers");
  if constexpr (Xbuf<N>::kPair)
    exchange2<V, PAD>(re, im, reinterpret_cast<float2*>(lds), act, widx, ridx, x);
  else
    exchange<V>(re, im, lds, act, widx, ridx, x);
}

// Radix of the pass that follows sub-length Ns: V values per thread, at most
// RM (a smaller RM trades an extra pass for fewer live registers).
__host__ __device__ constexpr int fft_radix(int N, int V, int Ns, int RM) {
  return (N / Ns) < (V < RM ? V : RM) ? (N / Ns) : (V < RM ? V : RM);
}

// Forward complex FFT of length N = T V, passes from sub-length Ns on.  On
// entry slot s holds x[in_index<fft_radix(N, V, 1, RM), T, N>(s)]; on exit
// slot s holds X[ridx_final(s)] (plus the extra read of `xf`, if any).
// PAD1: the first pass's exchange uses the padded layout (the buffer then
// needs Xbuf<N>::kPhys floats).
template <int N, int V, int Ns, int RM = 32, bool PAD1 = false, class RF>
__device__ __forceinline__ void fft_stages(float (&re)[V], float (&im)[V], float* lds, int t,
                                           bool act, RF ridx_final, Extra& xf) {
  constexpr int T = N / V;
  constexpr int R = fft_radix(N, V, Ns, RM);
  constexpr int Nn = Ns * R;
  if (act) fft_pass<V, R, T, Ns>(re, im, t);
  auto wf = [&](int s) { return out_index<R, T, Ns>(s, t); };
  if constexpr (Nn >= N) {
    xchg<N, V, PAD1 && Ns == 1>(re, im, lds, act, wf, ridx_final, xf);
  } else {
    constexpr int R2 = fft_radix(N, V, Nn, RM);
    Extra none{-1, -1, 0.f, 0.f, 0.f, 0.f};
    xchg<N, V, PAD1 && Ns == 1>(re, im, lds, act, wf,
                                [&](int s) { return in_index<R2, T, N>(s, t); }, none);
    fft_stages<N, V, Nn, RM>(re, im, lds, t, act, ridx_final, xf);
  }
}

// Block-wide exclusive scan (sum) over all SSS_T threads; *total gets the sum.
template <class X>
__device__ __forceinline__ X block_scan(X v, X* sw, X* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  X incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const X y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sw[w] = incl;
  __syncthreads();
  X before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < SSS_WAVES; ++i) {
    const X x = sw[i];
    if (i < w) before += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

// Wave sum and wave exclusive prefix of small non-negative ints (v <
// 2^BITS), one ballot per bit of v: a few scalar and VALU instructions
// instead of a chain of cross-lane permutes through LDS.  The sum is
// wave-uniform.
template <int BITS>
__device__ __forceinline__ int wave_sum_small(int v) {
  int s = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) s += __popcll(__ballot((v >> b) & 1)) << b;
  return s;
}
template <int BITS>
__device__ __forceinline__ int wave_prefix_small(int v, int* wave_total) {
  int p = 0, s = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const uint64_t m = __ballot((v >> b) & 1);
    const int below = (int)__builtin_amdgcn_mbcnt_hi(
        (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    p += below << b;
    s += __popcll(m) << b;
  }
  *wave_total = s;
  return p;
}
// block_scan for ints in [0, 2^BITS).
template <int BITS>
__device__ __forceinline__ int block_scan_small(int v, int* sw, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int wt;
  const int p = wave_prefix_small<BITS>(v, &wt);
  if (lane == 0) sw[w] = wt;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < SSS_WAVES; ++i) {
    const int x = sw[i];
    if (i < w) before += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return before + p;
}

// Bits of a count of at most n.
__host__ __device__ constexpr int count_bits(int n) { return n < 2 ? 1 : 1 + count_bits(n / 2); }

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 and +0 are equal
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct SssShared {
  double sd[SSS_WAVES];
  int si[SSS_WAVES];
  int bitcnt[32];   // per threshold bit: keys hit over the block
  int kstar;
  int kstar2;       // the second unit's, where two units share a transform
};

// e^{i pi x} as (cos, sin); v_sin/v_cos take revolutions (x/2).
__device__ __forceinline__ float2 cispi(float x) {
  const float rev = 0.5f * x;
  return make_float2(__builtin_amdgcn_cosf(rev), __builtin_amdgcn_sinf(rev));
}

// ---------------------------------------------------------------------------
// Smoothing of one unit's row.  On return re[s], im[s] hold s_hat at
// positions 2(tV + s) and 2(tV + s) + 1.
// ---------------------------------------------------------------------------
template <int N, int V>
__device__ __forceinline__ void smooth_unit(const KvcDesc& D, int mode, int u, const float* srow,
                            float* shrow, int32_t* kstar_out, float (&re)[V], float (&im)[V],
                            float* lds, SssShared& sh, int t, bool act) {
  constexpr int T = N / V;
  constexpr int L = 2 * N;
  constexpr int RM = 32;
  constexpr int R0 = fft_radix(N, V, 1, RM);
  const int hv = V / 2;
  // z_m = s_{2m} + i s_{2m+1}, in the order of the first pass.
  if (act) {
    const float2* z = reinterpret_cast<const float2*>(srow);
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const float2 v = z[in_index<R0, T, N>(s, t)];
      re[s] = v.x;
      im[s] = v.y;
    }
  }
  if (t == 0) sh.kstar = N;

  // Forward FFT; end in the pair layout: slot s < V/2 holds Z_k with
  // k = t V/2 + s, slot V/2 + s holds Z_{(N - k) mod N}; thread 0 also reads
  // the self-paired bin N/2.
  auto pair_idx = [&](int s) {
    const int k = t * hv + (s % hv);
    return s < hv ? k : ((N - k) & (N - 1));
  };
  Extra xf{-1, (t == 0) ? N / 2 : -1, 0.f, 0.f, 0.f, 0.f};
  fft_stages<N, V, 1, RM, Xbuf<N>::kPair>(re, im, lds, t, act, pair_idx, xf);

  // Real spectrum: F_k = A_k + e^{-2 pi i k/L} B_k with
  // A_k = (Z_k + conj Z_{N-k})/2, B_k = (Z_k - conj Z_{N-k})/(2i); the mirror
  // bin N-k uses the same pair.  Energies |F|^2 in fp64.
  double lo_sum = 0.0, hi_sum = 0.0, pmid = 0.0;
  float2 fmid = make_float2(0.f, 0.f);
  if (act) {
    const float2 Wstep = cispi(-2.0f / (float)L);
    float2 W = make_float2(1.f, 0.f);
#pragma unroll
    for (int s = 0; s < hv; ++s) {
      const int k = t * hv + s;
      const float2 zk = make_float2(re[s], im[s]);
      const float2 zm = make_float2(re[hv + s], im[hv + s]);
      const float2 A = make_float2(0.5f * (zk.x + zm.x), 0.5f * (zk.y - zm.y));
      const float2 B = make_float2(0.5f * (zk.y + zm.y), -0.5f * (zk.x - zm.x));
      if (s % 8 == 0) W = cispi(-2.0f * (float)k / (float)L);
      else W = cmul(W, Wstep);
      const float2 WB = cmul(W, B);
      const float2 Fk = make_float2(A.x + WB.x, A.y + WB.y);
      // mirror: A' = conj(A), B' = (Z_{N-k} - conj Z_k)/(2i) = conj(B)... with
      // twiddle e^{-2 pi i (N-k)/L} = -conj(W)
      const float2 Bm = make_float2(B.x, -B.y);
      const float2 Wm = make_float2(-W.x, W.y);
      const float2 WBm = cmul(Wm, Bm);
      const float2 Fm = make_float2(A.x + WBm.x, -A.y + WBm.y);
      re[s] = Fk.x;
      im[s] = Fk.y;
      re[hv + s] = Fm.x;
      im[hv + s] = Fm.y;
      lo_sum += (double)Fk.x * Fk.x + (double)Fk.y * Fk.y;
      hi_sum += (double)Fm.x * Fm.x + (double)Fm.y * Fm.y;
    }
    if (t == 0) {
      fmid = make_float2(xf.rre, -xf.rim);  // F_{N/2} = conj(Z_{N/2})
      pmid = (double)fmid.x * fmid.x + (double)fmid.y * fmid.y;
    }
  }
  // The spectrum values wait in LDS (free between the forward FFT's last
  // exchange and the inverse's first) while the block scans run, so that
  // the registers they occupy are not spilled to scratch across the scans:
  // all 2V floats of a thread when the buffer holds them (N <= 16384), else
  // the mirror bins' V floats.  Slot j of thread t at j*T + t (consecutive
  // threads, consecutive words).
  constexpr int PARK = 2 * V * T <= Xbuf<N>::kFloats ? 2 * V : V;
  static_assert(PARK * T <= Xbuf<N>::kFloats, "parked values fit the exchange buffer");
  auto park_slot = [&](int j) -> float& {
    // PARK == 2V: re[0..V) then im[0..V); PARK == V: re, im of slots hv..V
    if constexpr (PARK == 2 * V) return j < V ? re[j] : im[j - V];
    else return j < hv ? re[hv + j] : im[j];
  };
  if (act) {
#pragma unroll
    for (int j = 0; j < PARK; ++j) lds[j * T + t] = park_slot(j);
  }
  // Natural bin order: lower chunks (t ascending), bin N/2, upper chunks
  // (t descending).  Prefix energies from two block scans.
  double lo_tot, hi_tot;
  const double lo_before = block_scan<double>(lo_sum, sh.sd, &lo_tot);
  const double hi_incl = block_scan<double>(hi_sum, sh.sd, &hi_tot) + hi_sum;
  if (act) {
#pragma unroll
    for (int j = 0; j < PARK; ++j) park_slot(j) = lds[j * T + t];
  }
  if (t == 0) sh.sd[0] = pmid;
  __syncthreads();
  const double pm = sh.sd[0];
  __syncthreads();
  const double total = lo_tot + pm + hi_tot;
  const double target = (double)D.rho * total;
  if (act) {
    // Recompute the bin energies below rather than keeping 2V doubles live.
#pragma unroll
    for (int s = 0; s < V; ++s) asm volatile("" : "+v"(re[s]), "+v"(im[s]));
    int cand = N;
    double e = lo_before;
#pragma unroll
    for (int s = 0; s < hv; ++s) {
      e += (double)re[s] * re[s] + (double)im[s] * im[s];
      if (e >= target && cand == N) cand = t * hv + s;
    }
    if (t == 0 && cand == N && lo_tot + pm >= target) cand = N / 2;
    if (cand == N) {
      e = lo_tot + pm + (hi_tot - hi_incl);
#pragma unroll
      for (int s = hv - 1; s >= 0; --s) {
        e += (double)re[hv + s] * re[hv + s] + (double)im[hv + s] * im[hv + s];
        const int kk = N - (t * hv + s);
        if (e >= target && cand == N) cand = kk;
      }
    }
    if (cand < N) atomicMin(&sh.kstar, cand);
  }
  __syncthreads();
  const int kstar = sh.kstar;
  if ((mode & 4) && t == 0) kstar_out[u] = kstar;

  // Mask bins above k*, then merge back to the half-length sequence:
  // Z'_k = A'_k + i B'_k, A'_k = (F_k + conj F_{N-k})/2,
  // B'_k = e^{+2 pi i k/L} (F_k - conj F_{N-k})/2.
  Extra xi{-1, -1, 0.f, 0.f, 0.f, 0.f};
  if (act) {
    const float2 Wstep = cispi(2.0f / (float)L);
    float2 W = make_float2(1.f, 0.f);
#pragma unroll
    for (int s = 0; s < hv; ++s) {
      const int k = t * hv + s;
      const int km = N - k;  // N when k == 0
      const float2 Fk = (k <= kstar) ? make_float2(re[s], im[s]) : make_float2(0.f, 0.f);
      const float2 Fm =
          (km <= kstar) ? make_float2(re[hv + s], im[hv + s]) : make_float2(0.f, 0.f);
      const float2 A = make_float2(0.5f * (Fk.x + Fm.x), 0.5f * (Fk.y - Fm.y));
      const float2 Dd = make_float2(0.5f * (Fk.x - Fm.x), 0.5f * (Fk.y + Fm.y));
      if (s % 8 == 0) W = cispi(2.0f * (float)k / (float)L);
      else W = cmul(W, Wstep);
      const float2 B = cmul(W, Dd);
      // Z'_k = A + i B
      re[s] = A.x - B.y;
      im[s] = A.y + B.x;
      // Z'_{N-k}: A'' = conj(A), B'' = e^{+2 pi i (N-k)/L} (F_{N-k} - conj F_k)/2
      //         = (-conj W) * (-conj Dd) = conj(W Dd) = conj(B)
      re[hv + s] = A.x - (-B.y);
      im[hv + s] = -A.y + B.x;
    }
    if (t == 0) {
      // Z'_{N/2} = conj(F'_{N/2})
      const bool keep = (N / 2) <= kstar;
      xi.xw = N / 2;
      xi.wre = keep ? fmid.x : 0.f;
      xi.wim = keep ? -fmid.y : 0.f;
    }
  }
  // To the inverse's first-pass order.  Slot V/2 of thread 0 (k = 0) maps to
  // index 0 again and carries the same value as slot 0.
  xchg<N, V>(re, im, lds, act, pair_idx, [&](int s) { return in_index<R0, T, N>(s, t); }, xi);

  // Inverse FFT as conj(FFT(conj(x))) / N, ending in natural chunks
  // (slot s holds index tV + s).
#pragma unroll
  for (int s = 0; s < V; ++s) im[s] = -im[s];
  Extra none{-1, -1, 0.f, 0.f, 0.f, 0.f};
  fft_stages<N, V, 1, RM, Xbuf<N>::kPair>(re, im, lds, t, act, [&](int s) { return t * V + s; },
                                          none);

  // Blend with the raw row: s_hat = (1 - alpha) s + alpha lowpass.
  const float invN = 1.0f / (float)N;
  const float a = D.alpha, oma = 1.0f - D.alpha;
  if (act) {
    const float2* sr = reinterpret_cast<const float2*>(srow);
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const float2 sv = sr[t * V + s];
      const float lpe = re[s] * invN, lpo = -im[s] * invN;
      re[s] = oma * sv.x + a * lpe;
      im[s] = oma * sv.y + a * lpo;
    }
    if (mode & 4) {
      float2* o = reinterpret_cast<float2*>(shrow);
#pragma unroll
      for (int s = 0; s < V; ++s) o[t * V + s] = make_float2(re[s], im[s]);
    }
  }
}

// One level of a 32 x 32 bit-matrix transpose (row k = A[k], column j = bit
// j): rows k and k + J (bit J of k clear) exchange the high J-bit half of
// each 2J-bit group of row k with the low half of row k + J.
template <int J, uint32_t M>
__device__ __forceinline__ void transpose_level(uint32_t (&A)[32]) {
#pragma unroll
  for (int k = 0; k < 32; ++k)
    if (!(k & J)) {
      const uint32_t x = ((A[k] >> J) ^ A[k + J]) & M;
      A[k + J] ^= x;
      A[k] ^= x << J;
    }
}
// Afterwards bit s of A[b] is bit b of the original A[s].
__device__ __forceinline__ void transpose32(uint32_t (&A)[32]) {
  transpose_level<16, 0x0000FFFFu>(A);
  transpose_level<8, 0x00FF00FFu>(A);
  transpose_level<4, 0x0F0F0F0Fu>(A);
  transpose_level<2, 0x33333333u>(A);
  transpose_level<1, 0x55555555u>(A);
}

// ---------------------------------------------------------------------------
// Selection for one unit of L positions from s_hat held as in smooth_unit's
// output (thread t: positions 2 V t + 2 s in re[s], 2 V t + 2 s + 1 in
// im[s]; positions >= L are not part of the row).  stage: kStage ints of
// LDS, free for the output staging.
// ---------------------------------------------------------------------------
template <int V>
__device__ __forceinline__ void select_unit(const KvcDesc& D, int u, int L, float (&re)[V],
                            float (&im)[V], const int32_t* budgets, const int64_t* offsets,
                            int32_t* idx_out, SssShared& sh, int* stage, int kStage, int t,
                            bool act) {
  static_assert(2 * V <= 64, "the selection masks hold 64 positions per thread");
  const int w = D.window;
  const int ncand = L - w;
  const int b = budgets[u];
  const int k = b - w;
  const int64_t off = offsets[u];
  // A row kept whole (k >= ncand: every position) or down to its window
  // (k <= 0: positions ncand .. L-1) is a run of consecutive positions:
  // written directly, with no threshold search and no staging.
  if (k >= ncand || k <= 0) {
    const int lo = k >= ncand ? 0 : max(0, ncand);
    const int n = min(b, L - lo);
    for (int i = threadIdx.x; i < n; i += SSS_T) idx_out[off + i] = lo + i;
    return;
  }
  // Order-preserving keys of the thread's slots s (position p0 + s; slot
  // s is re[s/2] for even s, im[s/2] for odd s), transposed into planes per
  // group of 32 slots.  Slots past the row or the candidates never enter
  // the masks.
  constexpr int NG = (2 * V + 31) / 32;
  const int p0 = 2 * V * t;  // first position held by this thread
  uint32_t P[NG][32];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int sl = 32 * g + j;
      P[g][j] = sl < 2 * V ? order_key((sl & 1) ? im[sl >> 1] : re[sl >> 1]) : 0u;
    }
    transpose32(P[g]);
  }
  const int nval = act ? min(2 * V, max(0, ncand - p0)) : 0;
  uint32_t match[NG], above[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int nv = min(32, max(0, nval - 32 * g));
    match[g] = nv >= 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u);
    above[g] = 0u;
  }

  // Largest T with #{key >= T} >= k, bit by bit from the top; one barrier
  // per bit.  Per bit, the keys still equal to T's prefix with that bit set
  // are `hit`: they stay equal if T takes the bit, else they are above T
  // from then on.  Each wave adds its count of hits to the bit's LDS
  // counter; `A` counts the keys above T so far over the whole block.  Both
  // are wave-uniform (scalar registers), so the decision is a scalar
  // branch.
  constexpr int CB = count_bits(2 * V);  // a thread holds at most 2V keys
  if (threadIdx.x < 32) sh.bitcnt[threadIdx.x] = 0;
  __syncthreads();
  int A = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    uint32_t hit[NG];
    int h = 0;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      hit[g] = match[g] & P[g][bit];
      h += __popc(hit[g]);
    }
    const int hw = wave_sum_small<CB>(h);
    if ((threadIdx.x & 63) == 0) atomicAdd(&sh.bitcnt[bit], hw);
    __syncthreads();
    const int tot = A + __builtin_amdgcn_readfirstlane(sh.bitcnt[bit]);
    if (tot >= k) {
#pragma unroll
      for (int g = 0; g < NG; ++g) match[g] = hit[g];
    } else {
      A = tot;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        above[g] |= hit[g];
        match[g] &= ~P[g][bit];
      }
    }
  }
  // Counts above and at the threshold (the masks hold candidates only).
  int ngt = 0, neq = 0;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    ngt += __popc(above[g]);
    neq += __popc(match[g]);
  }
  int gt_total, eq_total;
  const int eq_before = block_scan_small<CB>(neq, sh.si, &eq_total);
  block_scan_small<CB>(ngt, sh.si, &gt_total);
  (void)eq_total;
  const int need = k - gt_total;  // positions equal to thr to keep, lowest first

  int nsel = 0, er = eq_before;
  uint32_t selmask_lo = 0, selmask_hi = 0;
  if (act) {
#pragma unroll
    for (int s = 0; s < 2 * V; ++s) {
      const int p = p0 + s;
      const bool gt = (above[s >> 5] >> (s & 31)) & 1u;
      const bool eq = (match[s >> 5] >> (s & 31)) & 1u;
      bool sel;
      if (p >= ncand) sel = p < L;
      else if (gt) sel = true;
      else if (eq) sel = (er++ < need);
      else sel = false;
      if (sel) {
        if (s < 32) selmask_lo |= 1u << s;
        else selmask_hi |= 1u << (s - 32);
        ++nsel;
      }
    }
  }
  int nsel_total;
  const int base = block_scan_small<CB>(nsel, sh.si, &nsel_total);
  // Staged output: position j of the segment at LDS int j + j/32, so that
  // threads whose runs start 32 apart (dense selections) write to distinct
  // banks.
  auto sidx = [](int j) { return j + (j >> 5); };
  if (b + (b >> 5) <= kStage) {
    // Compact into LDS, then one coalesced copy of the b positions.
    if (act) {
      int o = 0;
#pragma unroll
      for (int s = 0; s < 2 * V; ++s) {
        const bool sel = (s < 32) ? ((selmask_lo >> s) & 1u) : ((selmask_hi >> (s - 32)) & 1u);
        if (sel && base + o < b) stage[sidx(base + (o++))] = p0 + s;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < b; i += SSS_T) idx_out[off + i] = stage[sidx(i)];
  } else if (act) {
    int o = 0;
#pragma unroll
    for (int s = 0; s < 2 * V; ++s) {
      const bool sel = (s < 32) ? ((selmask_lo >> s) & 1u) : ((selmask_hi >> (s - 32)) & 1u);
      // (base + o < b always holds for finite input; the guard keeps a
      // non-finite row from writing past the unit's segment)
      if (sel && base + o < b) idx_out[off + base + (o++)] = p0 + s;
    }
  }
}

// Values per thread for a half-length N: at most 1024 threads, at least 8
// values each.
__host__ __device__ constexpr int kvc_sss_v(int N) {
  return N >= 32 * SSS_T ? 32 : N >= 16 * SSS_T ? 16 : 8;
}

template <int LOG2N>
__global__ __launch_bounds__(SSS_T) void kvc_sss_select_kernel(
    KvcDesc D, int mode, KvcSeqGroup G, const float* __restrict__ s_in, float* __restrict__ s_hat_out,
    int32_t* __restrict__ kstar_out, const int32_t* __restrict__ budgets,
    const int64_t* __restrict__ offsets, int32_t* __restrict__ idx_out) {
  constexpr int N = 1 << LOG2N;
  constexpr int L = 2 * N;
  constexpr int V = kvc_sss_v(N);
  constexpr int T = N / V;
  __shared__ __attribute__((aligned(16))) float lds[Xbuf<N>::kPhys];
  __shared__ SssShared sh;
  // This launch covers the group's units, all of one length.
  const int u = kvc_group_unit(G, D.upseq, (int)blockIdx.x);
  const int seq = u / D.upseq;
  const int within = u - seq * D.upseq;
  const int64_t row = D.srow_base[seq] + (int64_t)within * L;
  const int t = threadIdx.x;
  const bool act = t < T;
  float re[V], im[V];
  if (mode & 1) {
    smooth_unit<N, V>(D, mode, u, s_in + row, s_hat_out ? s_hat_out + row : nullptr, kstar_out,
                      re, im, lds, sh, t, act);
  } else if (act) {
    const float2* z = reinterpret_cast<const float2*>(s_in + row);
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const float2 v = z[t * V + s];
      re[s] = v.x;
      im[s] = v.y;
    }
  }
  if (mode & 2) {
    __syncthreads();  // the exchange buffer becomes the output staging area
    select_unit<V>(D, u, L, re, im, budgets, offsets, idx_out, sh, reinterpret_cast<int*>(lds),
                   Xbuf<N>::kPhys, t, act);
  }
}

// ---------------------------------------------------------------------------
// Lengths that are not powers of two
// ---------------------------------------------------------------------------
// The real transform of length L is a complex one of length Np (L/2 packed
// values for even L, L real values for odd L), computed with Bluestein's
// algorithm: X_k = conj(w_k) sum_n (x_n conj(w_n)) w_{k-n}, w_m = e^{i pi
// m^2 / Np}, the convolution taken with power-of-two FFTs of length
// M >= 2 Np - 1 (the Stockham passes above).  A per-launch prologue computes
// the table conj(w_n), n < Np, and FFT_M of the chirp filter; each unit's
// packed spectrum and its L/2 + 1 real bins go through global scratch
// (2 Np + 2 complex values per unit).  Selection then runs on the smoothed
// row in registers, as for powers of two.

// Scratch regions of one launch, 256-byte aligned: FFT_M of the chirp filter
// (M values), the chirp table (Np values), then the units' rows.
struct BluesteinScratch {
  size_t chirp_off, rows_off, bytes_per_unit;
};
__host__ __device__ inline size_t kvc_up256(size_t x) { return (x + 255) & ~size_t(255); }
__host__ inline BluesteinScratch kvc_bluestein_scratch(int Np, int M) {
  BluesteinScratch b;
  b.chirp_off = kvc_up256(sizeof(float2) * (size_t)M);
  b.rows_off = b.chirp_off + kvc_up256(sizeof(float2) * (size_t)Np);
  b.bytes_per_unit = sizeof(float2) * (2 * (size_t)Np + 2);
  return b;
}

// Largest radix of the Bluestein FFTs: radix-32 passes over 32 values per
// thread exceed the 128 registers a 1024-thread workgroup leaves each lane.
__host__ __device__ constexpr int kvc_bluestein_rm(int M) { return M >= 32 * SSS_T ? 16 : 32; }

// e^{i pi m^2 / Np}, the exponent reduced modulo 2 Np in integers first
// (m < 65536, so m^2 fits 32 bits unsigned).
__device__ __forceinline__ float2 kvc_chirp(int m, int Np) {
  const uint32_t r = ((uint32_t)m * (uint32_t)m) % (uint32_t)(2 * Np);
  return cispi((float)r / (float)Np);
}

__device__ __forceinline__ float2 conjf2(float2 a) { return make_float2(a.x, -a.y); }

// Forward DFT of length Np of in(n) (n < Np).  On exit slot s of thread t
// holds X_k, k = t V + s (meaningful for k < Np).  bhat: FFT_M of the chirp
// filter, natural order; cw: conj(w_n), n < Np.
template <int M, int V, class IN>
__device__ __forceinline__ void kvc_bluestein(IN in, int Np, const float2* __restrict__ bhat,
                                              const float2* __restrict__ cw, float* lds, int t,
                                              bool act, float (&re)[V], float (&im)[V]) {
  constexpr int T = M / V;
  constexpr int RM = kvc_bluestein_rm(M);
  constexpr int R0 = fft_radix(M, V, 1, RM);
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const int n = in_index<R0, T, M>(s, t);
      const float2 a = n < Np ? cmul(in(n), cw[n]) : make_float2(0.f, 0.f);
      re[s] = a.x;
      im[s] = a.y;
    }
  }
  Extra none{-1, -1, 0.f, 0.f, 0.f, 0.f};
  fft_stages<M, V, 1, RM>(re, im, lds, t, act, [&](int s) { return in_index<R0, T, M>(s, t); }, none);
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const float2 p = cmul(make_float2(re[s], im[s]), bhat[in_index<R0, T, M>(s, t)]);
      re[s] = p.x;
      im[s] = -p.y;  // conj: the inverse FFT as conj(FFT(conj(.))) / M
    }
  }
  fft_stages<M, V, 1, RM>(re, im, lds, t, act, [&](int s) { return t * V + s; }, none);
  if (act) {
    const float invM = 1.0f / (float)M;
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const int k = t * V + s;
      const float2 c = make_float2(re[s] * invM, -im[s] * invM);
      const float2 x = k < Np ? cmul(cw[k], c) : make_float2(0.f, 0.f);
      re[s] = x.x;
      im[s] = x.y;
    }
  }
}

// The launch prologue: cw[n] = conj(w_n) for n < Np, and FFT_M of the chirp
// filter b (b_m = w_m for 0 <= m < Np, b_{M-m} = w_m for 0 < m < Np, zero
// between), natural order; one workgroup.
template <int LOGM>
__global__ __launch_bounds__(SSS_T) void kvc_sss_chirp_kernel(int Np, float2* __restrict__ bhat,
                                                              float2* __restrict__ cw) {
  constexpr int M = 1 << LOGM;
  constexpr int V = kvc_sss_v(M);
  constexpr int T = M / V;
  constexpr int RM = kvc_bluestein_rm(M);
  constexpr int R0 = fft_radix(M, V, 1, RM);
  __shared__ __attribute__((aligned(16))) float lds[Xbuf<M>::kFloats];
  const int t = threadIdx.x;
  const bool act = t < T;
  for (int n = t; n < Np; n += SSS_T) cw[n] = conjf2(kvc_chirp(n, Np));
  float re[V], im[V];
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const int m = in_index<R0, T, M>(s, t);
      const int mm = m < Np ? m : (M - m < Np ? M - m : -1);
      const float2 b = mm >= 0 ? kvc_chirp(mm, Np) : make_float2(0.f, 0.f);
      re[s] = b.x;
      im[s] = b.y;
    }
  }
  Extra none{-1, -1, 0.f, 0.f, 0.f, 0.f};
  fft_stages<M, V, 1, RM>(re, im, lds, t, act, [&](int s) { return in_index<R0, T, M>(s, t); }, none);
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) bhat[in_index<R0, T, M>(s, t)] = make_float2(re[s], im[s]);
  }
}

template <int LOGM>
__global__ __launch_bounds__(SSS_T) void kvc_sss_general_kernel(
    KvcDesc D, int mode, KvcSeqGroup G, const float* __restrict__ s_in, float* __restrict__ s_hat_out,
    int32_t* __restrict__ kstar_out, const int32_t* __restrict__ budgets,
    const int64_t* __restrict__ offsets, int32_t* __restrict__ idx_out, float2* __restrict__ rows,
    const float2* __restrict__ bhat, const float2* __restrict__ cw) {
  constexpr int M = 1 << LOGM;
  constexpr int V = kvc_sss_v(M);
  constexpr int T = M / V;
  __shared__ __attribute__((aligned(16))) float lds[Xbuf<M>::kFloats];
  __shared__ SssShared sh;
  const int u = kvc_group_unit(G, D.upseq, (int)blockIdx.x);
  const int seq = u / D.upseq;
  const int within = u - seq * D.upseq;
  const int L = D.L[seq];
  const int64_t row = D.srow_base[seq] + (int64_t)within * L;
  const float* srow = s_in + row;
  const bool even = (L & 1) == 0;
  const int Np = even ? L / 2 : L;
  const int t = threadIdx.x;
  const bool act = t < T;
  // Values for the selection: position 2 VS t + 2 s in kr[s], the next in
  // ki[s] (T threads cover 2 VS T >= L positions).
  constexpr int VS = V < 16 ? V : 16;
  static_assert(2 * VS * T >= M, "selection layout covers the row");
  float kr[VS], ki[VS];
  if (mode & 1) {
    float re[V], im[V];
    float2* X = rows + (size_t)blockIdx.x * (2 * Np + 2);
    float2* Y = X + Np;  // L/2 + 1 <= Np + 1 bins
    // Spectrum of the row.
    auto in_row = [&](int n) {
      return even ? make_float2(srow[2 * n], srow[2 * n + 1]) : make_float2(srow[n], 0.f);
    };
    kvc_bluestein<M, V>(in_row, Np, bhat, cw, lds, t, act, re, im);
    if (act) {
#pragma unroll
      for (int s = 0; s < V; ++s)
        if (t * V + s < Np) X[t * V + s] = make_float2(re[s], im[s]);
    }
    if (t == 0) sh.kstar = L / 2;  // the last bin, should rounding leave E short of rho E(L/2)
    __syncthreads();
    // Real bins F_0 .. F_{L/2} (unpacked for even L), their energies in fp64.
    const int nb = L / 2 + 1;
    const int per = (nb + SSS_T - 1) / SSS_T;
    const int k0 = min(nb, t * per), k1 = min(nb, k0 + per);
    double esum = 0.0;
    for (int kk = k0; kk < k1; ++kk) {
      float2 F;
      if (even) {
        const float2 zk = X[kk % Np], zm = X[(Np - kk % Np) % Np];
        const float2 A = make_float2(0.5f * (zk.x + zm.x), 0.5f * (zk.y - zm.y));
        const float2 B = make_float2(0.5f * (zk.y + zm.y), -0.5f * (zk.x - zm.x));
        const float2 W = cispi(-2.0f * (float)kk / (float)L);
        const float2 WB = cmul(W, B);
        F = make_float2(A.x + WB.x, A.y + WB.y);
      } else {
        F = X[kk];
      }
      Y[kk] = F;
      esum += (double)F.x * F.x + (double)F.y * F.y;
    }
    double total;
    const double before = block_scan<double>(esum, sh.sd, &total);
    const double target = (double)D.rho * total;
    {
      double e = before;
      int cand = L;
      for (int kk = k0; kk < k1; ++kk) {
        const float2 F = Y[kk];
        e += (double)F.x * F.x + (double)F.y * F.y;
        if (e >= target && cand == L) cand = kk;
      }
      if (cand < L) atomicMin(&sh.kstar, cand);
    }
    __syncthreads();
    const int kstar = sh.kstar;
    if ((mode & 4) && t == 0) kstar_out[u] = kstar;
    // Masked spectrum, back to the complex sequence the inverse transforms.
    auto Fm = [&](int kk) { return kk <= kstar ? Y[kk] : make_float2(0.f, 0.f); };
    for (int kk = t; kk < Np; kk += SSS_T) {
      float2 z;
      if (even) {
        const float2 Fk = Fm(kk), Fr = Fm(Np - kk);
        const float2 A = make_float2(0.5f * (Fk.x + Fr.x), 0.5f * (Fk.y - Fr.y));
        const float2 Dd = make_float2(0.5f * (Fk.x - Fr.x), 0.5f * (Fk.y + Fr.y));
        const float2 B = cmul(cispi(2.0f * (float)kk / (float)L), Dd);
        z = make_float2(A.x - B.y, A.y + B.x);
      } else {
        z = kk <= (L - 1) / 2 ? Fm(kk) : conjf2(Fm(L - kk));
      }
      X[kk] = conjf2(z);  // the inverse DFT as conj(DFT(conj(.))) / Np
    }
    __syncthreads();
    kvc_bluestein<M, V>([&](int n) { return X[n]; }, Np, bhat, cw, lds, t, act, re, im);
    // Blend with the raw row: s_hat = (1 - alpha) s + alpha lowpass, into
    // LDS by position for the selection.
    const float invNp = 1.0f / (float)Np, a = D.alpha, oma = 1.0f - D.alpha;
    float* hrow = (mode & 4) ? s_hat_out + row : nullptr;
    if (act) {
#pragma unroll
      for (int s = 0; s < V; ++s) {
        const int m = t * V + s;
        const float lre = re[s] * invNp, lim = -im[s] * invNp;
        if (even) {
          if (m < Np) {
            // (rows of a sequence after one of odd length may start at an odd
            // float offset: scalar accesses)
            const float h0 = oma * srow[2 * m] + a * lre, h1 = oma * srow[2 * m + 1] + a * lim;
            lds[2 * m] = h0;
            lds[2 * m + 1] = h1;
            if (hrow) {
              hrow[2 * m] = h0;
              hrow[2 * m + 1] = h1;
            }
          }
        } else if (m < L) {
          const float h = oma * srow[m] + a * lre;
          lds[m] = h;
          if (hrow) hrow[m] = h;
        }
      }
    }
    if (!(mode & 2)) return;
    __syncthreads();
    if (act) {
#pragma unroll
      for (int s = 0; s < VS; ++s) {
        const int p = 2 * VS * t + 2 * s;
        kr[s] = p < L ? lds[p] : 0.f;
        ki[s] = p + 1 < L ? lds[p + 1] : 0.f;
      }
    }
  } else if (act) {
#pragma unroll
    for (int s = 0; s < VS; ++s) {
      const int p = 2 * VS * t + 2 * s;
      kr[s] = p < L ? srow[p] : 0.f;
      ki[s] = p + 1 < L ? srow[p + 1] : 0.f;
    }
  }
  if (mode & 2) {
    __syncthreads();  // the exchange buffer becomes the output staging area
    select_unit<VS>(D, u, L, kr, ki, budgets, offsets, idx_out, sh, reinterpret_cast<int*>(lds),
                    Xbuf<M>::kFloats, t, act);
  }
}

// ---------------------------------------------------------------------------
// Bluestein sizes M >= 32768: the transforms split across workgroups
// ---------------------------------------------------------------------------
// One workgroup cannot hold an M-point transform for M > 32768 (its values
// in registers and one part in LDS), and at M = 32768 the single-workgroup
// kernel above runs out of registers.  These lengths (even L > 16384, odd
// L > 8192, up to 65536) split each M-point FFT into S = M / H transforms of
// H = 32768 points, by one radix-S step of decimation in frequency for the
// forward FFT of the premultiplied sequence a and one of decimation in time
// for the second FFT (W_n = e^{-2 pi i / n}):
//   FFT_M(a)_{S k + r} = FFT_H(y_r)_k,  y_r[j] = W_M^{j r} sum_q a_{j+qH} W_S^{q r}
//   FFT_M(P)_m = sum_r W_M^{r m} FFT_H(P_{S k + r})_{m mod H}
// so the product with FFT_M of the chirp filter is formed in the decimated
// order in which the first FFT leaves it, which is the order the second one
// takes.  Kernels per smoothing launch: the chirp filter's split and
// sub-FFTs (once), then per unit the first convolution (one workgroup per
// sub-sequence: the split from the score row, FFT, product, FFT), the
// spectrum (one workgroup per unit: combine, real bins, fp64 energies, k*,
// mask, back to the inverse's split), the second convolution, and the
// finish (combine, blend, selection).  A sub-sequence's two FFTs run in the
// same 1024-thread workgroup (Stockham passes, 32 values per thread), the
// first leaving its output in the order the second starts from, so only
// the convolution results go through global scratch.
#define KVC_BIG_LOGH 15
#define KVC_BIG_H (1 << KVC_BIG_LOGH)

// Scratch of a long-length launch, in float2 units: FFT_M of the chirp
// filter in decimated order (sub-transform r's bins at r H ..), the chirp
// table conj(w_n) (n < Np), then per unit: the M sub-sequence values, the
// Np-bin spectrum (also the smoothed row's staging area) and the L/2 + 1
// real bins.
struct BigScratch {
  size_t cw_off, rows_off, ustride;
};
__host__ __device__ inline BigScratch kvc_big_scratch(int Np, int M) {
  auto up32 = [](size_t x) { return (x + 31) & ~size_t(31); };
  BigScratch b;
  b.cw_off = up32((size_t)M);
  b.rows_off = b.cw_off + up32((size_t)Np);
  b.ustride = up32((size_t)M + 2 * (size_t)Np + 2);
  return b;
}

// e^{-2 pi i f} for f = x / M given as an integer x (any sign), exact
// revolutions after reduction modulo M (M a power of two).
__device__ __forceinline__ float2 kvc_twiddle(int x, int M) {
  const float f = (float)(x & (M - 1)) / (float)M;
  return make_float2(__builtin_amdgcn_cosf(f), -__builtin_amdgcn_sinf(f));
}

// v * W_S^e for S in {1, 2, 4}: multiples of a quarter turn, exact.
__device__ __forceinline__ float2 kvc_quarter(float2 v, int e, int S) {
  const int qt = (e * (4 / S)) & 3;  // quarter turns clockwise
  return qt == 0 ? v : qt == 1 ? make_float2(v.y, -v.x) : qt == 2 ? make_float2(-v.x, -v.y)
                                                                    : make_float2(-v.y, v.x);
}

// Odd lengths have no half-length packing (L real values, Np = L), so two
// units share each transform instead: the rows of the group's units 2p and
// 2p + 1 are the real and imaginary parts of one length-L complex sequence
// (the last unit of an odd count pairs with itself).  The DFT Z of
// x1 + i x2 gives X1_k = (Z_k + conj Z_{L-k}) / 2 and
// X2_k = (Z_k - conj Z_{L-k}) / (2i); the inverse of G1 + i G2 for two
// Hermitian spectra is g1 + i g2 with both parts real.  Each row enters
// scaled by 2^-e, e chosen so that its L2 norm is in [1, 2): the rounding
// of one part then stays at the size of the other's (rows of very different
// sizes would otherwise lose the smaller one's accuracy), and a power of
// two commutes with every rounding, so the energies, k* and the low-pass
// row (scaled back by 2^e) come out as without it.  A pair's values live in
// the scratch slot of its first unit; every unit's exponent in the last
// value of its own slot.  Even lengths: one unit per slot, no scaling.
__host__ __device__ inline int kvc_big_items(int nwg, bool paired) {
  return paired ? (nwg + 1) / 2 : nwg;
}
__host__ __device__ inline size_t kvc_big_exp_index(int Np, int M) {
  return (size_t)M + 2 * (size_t)Np + 1;   // within the slot (BigScratch::ustride)
}

// Value n of the premultiplied sequence of the first forward transform:
// a_n = in(n) conj(w_n), in(n) = (s_2n, s_2n+1) for even L,
// (s_n 2^-e1, s2_n 2^-e2) for odd L (s2: the pair's second row).
__device__ __forceinline__ float2 kvc_big_in(const float* srow, const float* srow2, bool even,
                                             int n, float2 c, int e1, int e2) {
  const float2 x = even ? make_float2(srow[2 * n], srow[2 * n + 1])
                        : make_float2(ldexpf(srow[n], -e1), ldexpf(srow2[n], -e2));
  return cmul(x, c);
}

// The score row of group unit b.
__device__ __forceinline__ const float* kvc_big_row(const KvcDesc& D, const KvcSeqGroup& G,
                                                    const float* s_in, int b) {
  const int u = kvc_group_unit(G, D.upseq, b);
  const int seq = u / D.upseq, within = u - seq * D.upseq;
  return s_in + D.srow_base[seq] + (int64_t)within * D.L[seq];
}

// Odd L: each unit's scale exponent e (L2 norm of the row times 2^-e in
// [1, 2); 0 for a zero or non-finite norm), into the last value of its
// slot.  One 1024-thread workgroup per unit, eight loads in flight per
// thread.
__global__ __launch_bounds__(SSS_T) void kvc_big_scale_kernel(KvcDesc D, KvcSeqGroup G, int Np,
                                                              int M, const float* __restrict__ s_in,
                                                              float2* __restrict__ base) {
  __shared__ float part[SSS_WAVES];
  const int b = (int)blockIdx.x;
  const int L = D.L[G.seq[0]];
  const float* srow = kvc_big_row(D, G, s_in, b);
  float acc = 0.f;
  for (int n0 = threadIdx.x; n0 < L; n0 += 8 * SSS_T) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + i * SSS_T;
      v[i] = n < L ? srow[n] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf(v[i], v[i], acc);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float ss = 0.f;
    for (int w = 0; w < SSS_WAVES; ++w) ss += part[w];
    int e = 0;
    if (ss > 0.f && ss < INFINITY) {
      frexpf(sqrtf(ss), &e);   // sqrt(ss) = f 2^e, f in [0.5, 1)
      e -= 1;                  // 2^-e sqrt(ss) in [1, 2)
    }
    const BigScratch bs = kvc_big_scratch(Np, M);
    float2* slot = base + bs.rows_off + (size_t)b * bs.ustride;
    slot[kvc_big_exp_index(Np, M)] = make_float2(__int_as_float(e), 0.f);
  }
}
__device__ __forceinline__ int kvc_big_exp(const float2* slot_base, int Np, int M) {
  return __float_as_int(slot_base[kvc_big_exp_index(Np, M)].x);
}

// The radix-S split y_r[j] (r < S) of a length-M sequence given by `val`
// (val(n) for n < M), written to Y[r H + j].
template <int S, class F>
__device__ __forceinline__ void kvc_big_split(float2* __restrict__ Y, int j, int M, F val) {
  float2 a[S];
#pragma unroll
  for (int q = 0; q < S; ++q) a[q] = val(j + q * KVC_BIG_H);
#pragma unroll
  for (int r = 0; r < S; ++r) {
    float2 y = make_float2(0.f, 0.f);
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const float2 v = kvc_quarter(a[q], q * r, S);
      y = make_float2(y.x + v.x, y.y + v.y);
    }
    Y[(size_t)r * KVC_BIG_H + j] = r == 0 ? y : cmul(y, kvc_twiddle(j * r, M));
  }
}

// sum_r W_M^{r m} E_r[m mod H]: bin m of the M-point FFT from the
// sub-transforms' outputs.
template <int S>
__device__ __forceinline__ float2 kvc_big_combine(const float2* __restrict__ Y, int m, int M) {
  const int k = m & (KVC_BIG_H - 1);
  float2 q = Y[k];
#pragma unroll
  for (int r = 1; r < S; ++r) {
    const float2 v = cmul(Y[(size_t)r * KVC_BIG_H + k], kvc_twiddle(r * m, M));
    q = make_float2(q.x + v.x, q.y + v.y);
  }
  return q;
}

// Split of the chirp filter (b_m = w_m for m < Np, b_{M-m} = w_m for
// 0 < m < Np, zero between) into the bhat region, and the table
// cw[n] = conj(w_n).  grid H / 256, 256 threads.
template <int S>
__global__ __launch_bounds__(256) void kvc_big_chirp_split_kernel(int Np,
                                                                  float2* __restrict__ base) {
  constexpr int M = S * KVC_BIG_H;
  const int j = blockIdx.x * 256 + threadIdx.x;
  const BigScratch bs = kvc_big_scratch(Np, M);
  float2* cw = base + bs.cw_off;
  for (int n = j; n < Np; n += KVC_BIG_H) cw[n] = conjf2(kvc_chirp(n, Np));
  kvc_big_split<S>(base, j, M, [&](int m) {
    const int mm = m < Np ? m : (M - m < Np ? M - m : -1);
    return mm >= 0 ? kvc_chirp(mm, Np) : make_float2(0.f, 0.f);
  });
}

// The chirp filter's H-point sub-FFTs in place: sub-sequence blockIdx.x of
// the bhat region, natural order (sub-transform r then holds bins S k + r).
template <int S>
__global__ __launch_bounds__(SSS_T) void kvc_big_chirp_fft_kernel(float2* __restrict__ base) {
  constexpr int N = KVC_BIG_H, V = 32, T = N / V, RM = 16;
  constexpr int R0 = fft_radix(N, V, 1, RM);
  static_assert(T == SSS_T, "one value slot set per thread");
  __shared__ __attribute__((aligned(16))) float lds[Xbuf<N>::kFloats];
  float2* y = base + (size_t)blockIdx.x * N;
  const int t = threadIdx.x;
  float re[V], im[V];
#pragma unroll
  for (int s = 0; s < V; ++s) {
    const float2 v = y[in_index<R0, T, N>(s, t)];
    re[s] = v.x;
    im[s] = v.y;
  }
  Extra none{-1, -1, 0.f, 0.f, 0.f, 0.f};
  fft_stages<N, V, 1, RM>(re, im, lds, t, true, [&](int s) { return t * V + s; }, none);
  // (every value of y was read before the first exchange's barrier)
  float4* o = reinterpret_cast<float4*>(y + t * V);
#pragma unroll
  for (int s = 0; s < V; s += 2) o[s / 2] = make_float4(re[s], im[s], re[s + 1], im[s + 1]);
}

// One sub-sequence's share of a whole convolution in one workgroup: its
// H-point FFT (left in the first pass's input order, which is where the
// second FFT starts), the product with the chirp filter's spectrum and the
// conjugation, the second H-point FFT (the decimation-in-time sub-transform
// of the same sub-sequence), stored in place in natural order.  FROM_ROW:
// the input is split on the fly from the unit's score row (the first
// transform); else read from the unit's split values (the second).  One
// workgroup per (slot item, sub-sequence): units for even L, unit pairs for
// odd L.
template <int S, bool FROM_ROW>
__global__ __launch_bounds__(SSS_T) void kvc_big_conv_kernel(KvcDesc D, KvcSeqGroup G, int Np,
                                                             const float* __restrict__ s_in,
                                                             float2* __restrict__ base) {
  constexpr int N = KVC_BIG_H, V = 32, T = N / V, RM = 16, M = S * N;
  constexpr int R0 = fft_radix(N, V, 1, RM);
  static_assert(T == SSS_T, "one value slot set per thread");
  __shared__ __attribute__((aligned(16))) float lds[Xbuf<N>::kFloats];
  const BigScratch bs = kvc_big_scratch(Np, M);
  const float2* bhat = base;
  const float2* cw = base + bs.cw_off;
  const int nwg = G.n * (G.hi - G.lo);
  const bool even = (D.L[G.seq[0]] & 1) == 0;   // (one length per group)
  const int item = (int)blockIdx.x / S, r = (int)blockIdx.x % S;
  const int slot = even ? item : 2 * item;
  float2* y = base + bs.rows_off + (size_t)slot * bs.ustride + (size_t)r * N;
  const int t = threadIdx.x;
  float re[V], im[V];
  if constexpr (FROM_ROW) {
    const float* srow = kvc_big_row(D, G, s_in, slot);
    const int slot2 = min(slot + 1, nwg - 1);
    const float* srow2 = even ? srow : kvc_big_row(D, G, s_in, slot2);
    const float2* slots = base + bs.rows_off;
    const int e1 = even ? 0 : kvc_big_exp(slots + (size_t)slot * bs.ustride, Np, M);
    const int e2 = even ? 0 : kvc_big_exp(slots + (size_t)slot2 * bs.ustride, Np, M);
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const int j = in_index<R0, T, N>(s, t);
      float2 acc = make_float2(0.f, 0.f);
#pragma unroll
      for (int q = 0; q < S; ++q) {
        const int n = j + q * N;
        if (n < Np) {
          const float2 v =
              kvc_quarter(kvc_big_in(srow, srow2, even, n, cw[n], e1, e2), q * r, S);
          acc = make_float2(acc.x + v.x, acc.y + v.y);
        }
      }
      if (r) acc = cmul(acc, kvc_twiddle(j * r, M));
      re[s] = acc.x;
      im[s] = acc.y;
    }
  } else {
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const float2 v = y[in_index<R0, T, N>(s, t)];
      re[s] = v.x;
      im[s] = v.y;
    }
  }
  Extra none{-1, -1, 0.f, 0.f, 0.f, 0.f};
  fft_stages<N, V, 1, RM>(re, im, lds, t, true, [&](int s) { return in_index<R0, T, N>(s, t); },
                          none);
  {
    // (an opaque copy of the thread index: the compiler would otherwise keep
    // the first FFT's output indices live into the second)
    int tt = t;
    asm volatile("" : "+v"(tt));
    const float2* bh = bhat + (size_t)r * N;
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const float2 p = cmul(make_float2(re[s], im[s]), bh[in_index<R0, T, N>(s, tt)]);
      re[s] = p.x;
      im[s] = -p.y;
    }
  }
  fft_stages<N, V, 1, RM>(re, im, lds, t, true, [&](int s) { return t * V + s; }, none);
  float4* o = reinterpret_cast<float4*>(y + t * V);
#pragma unroll
  for (int s = 0; s < V; s += 2) o[s / 2] = make_float4(re[s], im[s], re[s + 1], im[s + 1]);
}

// Loads in these per-unit kernels go out in batches (a batch's loads, then
// its arithmetic and stores): their loops read and write one scratch area,
// so the compiler would otherwise wait on every load.  KB: batch size.
template <int S>
__host__ __device__ constexpr int kvc_big_batch() { return S >= 4 ? 4 : 8; }

// After the first convolution, per slot item (a unit for even L, a unit
// pair for odd L), in three launches spread over the whole chip:
//  A (kvc_big_bins_kernel): the real bins F_0 .. F_{L/2} (odd L: of both
//    units), each from the spectrum values Z_k and Z_{Np-k} combined from the
//    sub-transforms, and the fp64 energy sum of each of KVC_BIG_CH chunks of
//    consecutive bins;
//  B (kvc_big_kstar_kernel): k* from the chunk sums and a block scan of the
//    one chunk in which the cumulative energy reaches rho of the total;
//  C (kvc_big_merge_kernel): the masked spectrum merged back to the complex
//    sequence the inverse transforms (G1 + i G2 for a pair), conjugated and
//    premultiplied by conj(w_n), and its split into the sub-sequences.
// In the item's slot: the chunk sums and k* from M on, the bins from
// M + Np on.
#define KVC_BIG_CH 16

// Spectrum value k < Np of the first transform from the sub-transforms:
// Z_k = conj(w_k) conj(sum_r W_M^{rk} E_r[k mod H]) / M.
template <int S>
__device__ __forceinline__ float2 kvc_big_spec(const float2* __restrict__ Y,
                                               const float2* __restrict__ cw, int k, int M) {
  const int kh = k & (KVC_BIG_H - 1);
  float2 q = Y[kh];
#pragma unroll
  for (int r = 1; r < S; ++r) {
    const float2 v = cmul(Y[(size_t)r * KVC_BIG_H + kh], kvc_twiddle(r * k, M));
    q = make_float2(q.x + v.x, q.y + v.y);
  }
  const float invM = 1.0f / (float)M;
  return cmul(cw[k], make_float2(q.x * invM, -q.y * invM));
}

// The slot of item `item`, the chunk sums (two per chunk: unit 1, unit 2)
// and k* (two) within it.
struct BigItem {
  float2* Y;
  float2* Fb;
  float2* Fb2;
  double* sums;
  int* kst;
};
__device__ __forceinline__ BigItem kvc_big_item(float2* base, int Np, int M, int L, int slot) {
  const BigScratch bs = kvc_big_scratch(Np, M);
  BigItem it;
  it.Y = base + bs.rows_off + (size_t)slot * bs.ustride;
  it.Fb = it.Y + M + Np;
  it.Fb2 = it.Fb + (L / 2 + 1);   // odd L: the second unit's bins (Np = L)
  it.sums = reinterpret_cast<double*>(it.Y + M);
  it.kst = reinterpret_cast<int*>(it.sums + 2 * KVC_BIG_CH);
  return it;
}

template <int S>
__global__ __launch_bounds__(256) void kvc_big_bins_kernel(KvcDesc D, KvcSeqGroup G, int Np,
                                                           float2* __restrict__ base) {
  constexpr int M = S * KVC_BIG_H, KB = 4;
  __shared__ double part[2][4];
  const int L = D.L[G.seq[0]];   // (one length per group)
  const bool even = (L & 1) == 0;
  const int item = (int)blockIdx.x / KVC_BIG_CH, c = (int)blockIdx.x % KVC_BIG_CH;
  const BigItem it = kvc_big_item(base, Np, M, L, even ? item : 2 * item);
  const float2* cw = base + kvc_big_scratch(Np, M).cw_off;
  const int nb = L / 2 + 1, per = (nb + KVC_BIG_CH - 1) / KVC_BIG_CH;
  const int k0 = min(nb, c * per), k1 = min(nb, k0 + per);
  double e1 = 0.0, e2 = 0.0;
  // (KB bins per thread at a time: their loads, then arithmetic and stores)
  for (int kb = k0 + (int)threadIdx.x; kb < k1; kb += KB * 256) {
    float2 zk[KB], zm[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int k = min(kb + i * 256, k1 - 1);   // (clamped: every load in bounds)
      zk[i] = kvc_big_spec<S>(it.Y, cw, k % Np, M);
      zm[i] = kvc_big_spec<S>(it.Y, cw, (Np - k % Np) % Np, M);
    }
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int k = kb + i * 256;
      if (k >= k1) continue;
      // A = (Z_k + conj Z_{Np-k}) / 2, B = (Z_k - conj Z_{Np-k}) / (2i)
      const float2 A = make_float2(0.5f * (zk[i].x + zm[i].x), 0.5f * (zk[i].y - zm[i].y));
      const float2 B = make_float2(0.5f * (zk[i].y + zm[i].y), -0.5f * (zk[i].x - zm[i].x));
      if (even) {
        const float2 WB = cmul(cispi(-2.0f * (float)k / (float)L), B);
        const float2 F = make_float2(A.x + WB.x, A.y + WB.y);
        it.Fb[k] = F;
        e1 += (double)F.x * F.x + (double)F.y * F.y;
      } else {
        it.Fb[k] = A;    // the pair's first unit
        it.Fb2[k] = B;   // and its second
        e1 += (double)A.x * A.x + (double)A.y * A.y;
        e2 += (double)B.x * B.x + (double)B.y * B.y;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    e1 += __shfl_xor(e1, o);
    e2 += __shfl_xor(e2, o);
  }
  if ((threadIdx.x & 63) == 0) {
    part[0][threadIdx.x >> 6] = e1;
    part[1][threadIdx.x >> 6] = e2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    it.sums[2 * c] = ((part[0][0] + part[0][1]) + part[0][2]) + part[0][3];
    it.sums[2 * c + 1] = ((part[1][0] + part[1][1]) + part[1][2]) + part[1][3];
  }
}

// k* of each unit of the item: the first bin at which the cumulative fp64
// energy reaches rho of the total (the last bin, should rounding leave the
// total short).  One 1024-thread workgroup per item.
template <int S>
__global__ __launch_bounds__(SSS_T) void kvc_big_kstar_kernel(KvcDesc D, int mode, KvcSeqGroup G,
                                                              int Np, float2* __restrict__ base,
                                                              int32_t* __restrict__ kstar_out) {
  constexpr int M = S * KVC_BIG_H;
  __shared__ SssShared sh;
  __shared__ double s_before;
  __shared__ int s_chunk;
  const int nwg = G.n * (G.hi - G.lo);
  const int L = D.L[G.seq[0]];
  const bool even = (L & 1) == 0;
  const int slot = even ? (int)blockIdx.x : 2 * (int)blockIdx.x;
  const int u = kvc_group_unit(G, D.upseq, slot);
  const int u2 = even ? u : kvc_group_unit(G, D.upseq, min(slot + 1, nwg - 1));
  const BigItem it = kvc_big_item(base, Np, M, L, slot);
  const int nb = L / 2 + 1, per = (nb + KVC_BIG_CH - 1) / KVC_BIG_CH;
  const int t = threadIdx.x;
  int ks[2] = {L / 2, L / 2};
  for (int part = 0; part < (even ? 1 : 2); ++part) {
    const float2* F = part ? it.Fb2 : it.Fb;
    // the chunk in which the cumulative energy reaches the target
    if (t == 0) {
      double total = 0.0;
      for (int c = 0; c < KVC_BIG_CH; ++c) total += it.sums[2 * c + part];
      const double target = (double)D.rho * total;
      double cum = 0.0;
      int cc = -1;
      for (int c = 0; c < KVC_BIG_CH && cc < 0; ++c) {
        if (cum + it.sums[2 * c + part] >= target) cc = c;
        else cum += it.sums[2 * c + part];
      }
      s_chunk = cc;
      s_before = cum;
      // (the chunk's last bin, should the bin-by-bin sums fall short of the
      // chunk's total by rounding)
      sh.kstar = cc >= 0 ? min(nb, cc * per + per) - 1 : L / 2;
      sh.sd[0] = target;
    }
    __syncthreads();
    const int cc = s_chunk;
    const double target = sh.sd[0], before0 = s_before;
    __syncthreads();
    if (cc >= 0) {
      // contiguous runs of the chunk's bins per thread, a block scan of
      // their energies, then each run walked in order
      const int c0 = min(nb, cc * per), c1 = min(nb, c0 + per);
      const int run = (c1 - c0 + SSS_T - 1) / SSS_T;
      const int r0 = min(c1, c0 + t * run), r1 = min(c1, r0 + run);
      double esum = 0.0;
      for (int k = r0; k < r1; ++k) esum += (double)F[k].x * F[k].x + (double)F[k].y * F[k].y;
      double tot;
      double e = before0 + block_scan<double>(esum, sh.sd, &tot);
      int cand = L;
      for (int k = r0; k < r1 && cand == L; ++k) {
        e += (double)F[k].x * F[k].x + (double)F[k].y * F[k].y;
        if (e >= target) cand = k;
      }
      if (cand < L) atomicMin(&sh.kstar, cand);
    }
    __syncthreads();
    ks[part] = sh.kstar;
    __syncthreads();
  }
  if (t == 0) {
    it.kst[0] = ks[0];
    it.kst[1] = even ? ks[0] : ks[1];
    if (mode & 4) {
      kstar_out[u] = ks[0];
      if (u2 != u) kstar_out[u2] = ks[1];
    }
  }
}

// The masked spectrum merged back and split: for the sub-sequence index j,
// values n = j + q H (q < S) of the sequence the inverse transforms,
// a_n = conj(z_n) conj(w_n) (z: the unit's complex sequence from its masked
// bins, or G1 + i G2 for a pair), then the radix-S split.  Grid (item,
// range of 1024 j).
template <int S>
__global__ __launch_bounds__(256) void kvc_big_merge_kernel(KvcDesc D, KvcSeqGroup G, int Np,
                                                            float2* __restrict__ base) {
  constexpr int M = S * KVC_BIG_H, H = KVC_BIG_H, JB = 4;
  constexpr int PER_WG = 256 * JB, WGS = H / PER_WG;
  const int L = D.L[G.seq[0]];
  const bool even = (L & 1) == 0;
  const int item = (int)blockIdx.x / WGS, jw = (int)blockIdx.x % WGS;
  const BigItem it = kvc_big_item(base, Np, M, L, even ? item : 2 * item);
  const float2* cw = base + kvc_big_scratch(Np, M).cw_off;
  const int kstar = it.kst[0], kstar2 = it.kst[1];
  auto Fm = [&](int kk, float2 v) { return kk <= kstar ? v : make_float2(0.f, 0.f); };
  auto Fm2 = [&](int kk, float2 v) { return kk <= kstar2 ? v : make_float2(0.f, 0.f); };
  float2 f1[JB][S], f2[JB][S], c[JB][S];
#pragma unroll
  for (int i = 0; i < JB; ++i) {
    const int j = jw * PER_WG + i * 256 + (int)threadIdx.x;
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const int n = min(j + q * H, Np - 1);   // (clamped: every load in bounds)
      // even: bins n and Np - n; odd: bin n or L - n of each unit
      const int i1 = even ? n : (n <= (L - 1) / 2 ? n : L - n);
      f1[i][q] = it.Fb[min(i1, kstar)];   // (masked below; the indices kept in bounds)
      f2[i][q] = even ? it.Fb[min(Np - n, kstar)] : it.Fb2[min(i1, kstar2)];
      c[i][q] = cw[n];
    }
  }
#pragma unroll
  for (int i = 0; i < JB; ++i) {
    const int j = jw * PER_WG + i * 256 + (int)threadIdx.x;
    float2 a[S];
#pragma unroll
    for (int q = 0; q < S; ++q) {
      const int n = j + q * H;
      float2 z;
      if (even) {
        const float2 Fk = Fm(n, f1[i][q]), Fr = Fm(Np - n, f2[i][q]);
        const float2 A = make_float2(0.5f * (Fk.x + Fr.x), 0.5f * (Fk.y - Fr.y));
        const float2 Dd = make_float2(0.5f * (Fk.x - Fr.x), 0.5f * (Fk.y + Fr.y));
        const float2 B = cmul(cispi(2.0f * (float)n / (float)L), Dd);
        z = make_float2(A.x - B.y, A.y + B.x);
      } else {
        // G1 + i G2, each unit's spectrum extended by conjugate symmetry
        const bool lo = n <= (L - 1) / 2;
        const float2 g1 = lo ? Fm(n, f1[i][q]) : conjf2(Fm(L - n, f1[i][q]));
        const float2 g2 = lo ? Fm2(n, f2[i][q]) : conjf2(Fm2(L - n, f2[i][q]));
        z = make_float2(g1.x - g2.y, g1.y + g2.x);
      }
      a[q] = n < Np ? cmul(conjf2(z), c[i][q]) : make_float2(0.f, 0.f);
    }
    kvc_big_split<S>(it.Y, j, M, [&](int n) { return a[(n - j) / H]; });
  }
}

// Per unit, after the second convolution: the low-pass row
// lp = conj(conj(w_m) conj(sum_r ...) / M) / Np, the blend with the raw row,
// and the selection on it.  mode without bit 0: selection on s_in as given.
// Odd L: the unit's low-pass row is the real (first unit of the pair) or
// imaginary (second) part of its pair's inverse.
template <int S, int VS>
__global__ __launch_bounds__(SSS_T) void kvc_big_finish_kernel(
    KvcDesc D, int mode, KvcSeqGroup G, int Np, const float* __restrict__ s_in,
    float* __restrict__ s_hat_out, const int32_t* __restrict__ budgets,
    const int64_t* __restrict__ offsets, int32_t* __restrict__ idx_out,
    float2* __restrict__ base) {
  constexpr int M = S * KVC_BIG_H, H = KVC_BIG_H, KB = kvc_big_batch<S>();
  constexpr int kStage = 32768;
  static_assert(2 * VS * SSS_T >= 32768, "selection layout covers the row");
  __shared__ int stage[kStage];
  __shared__ SssShared sh;
  const int u = kvc_group_unit(G, D.upseq, (int)blockIdx.x);
  const int seq = u / D.upseq, within = u - seq * D.upseq;
  const int L = D.L[seq];
  const int64_t row = D.srow_base[seq] + (int64_t)within * L;
  const float* srow = s_in + row;
  const bool even = (L & 1) == 0;
  const int t = threadIdx.x;
  float kr[VS], ki[VS];
  const float* src = srow;
  if (mode & 1) {
    const BigScratch bs = kvc_big_scratch(Np, M);
    const float2* cw = base + bs.cw_off;
    const int b = (int)blockIdx.x, second = even ? 0 : (b & 1);
    const float2* Y = base + bs.rows_off + (size_t)(b - second) * bs.ustride;
    // (the unit's own slot past its M transform values: free here, and never
    // the pair's transform values, which are in the first unit's slot below M)
    float* hs = reinterpret_cast<float*>(base + bs.rows_off + (size_t)b * bs.ustride + M);
    float* hrow = (mode & 4) ? s_hat_out + row : nullptr;
    const float invM = 1.0f / (float)M, invNp = 1.0f / (float)Np;
    const float a = D.alpha, oma = 1.0f - D.alpha;
    const int ex = even ? 0 : kvc_big_exp(base + bs.rows_off + (size_t)b * bs.ustride, Np, M);
    for (int m0 = t; m0 < Np; m0 += KB * SSS_T) {
      float2 e[KB][S], c[KB], sv[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const int m = min(m0 + i * SSS_T, Np - 1);
#pragma unroll
        for (int r = 0; r < S; ++r) e[i][r] = Y[(size_t)r * H + (m & (H - 1))];
        c[i] = cw[m];
        sv[i] = even ? make_float2(srow[2 * m], srow[2 * m + 1]) : make_float2(srow[m], 0.f);
      }
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const int m = m0 + i * SSS_T;
        if (m >= Np) continue;
        float2 q = e[i][0];
#pragma unroll
        for (int r = 1; r < S; ++r) {
          const float2 v = cmul(e[i][r], kvc_twiddle(r * m, M));
          q = make_float2(q.x + v.x, q.y + v.y);
        }
        const float2 x = cmul(c[i], make_float2(q.x * invM, -q.y * invM));
        const float lre = x.x * invNp, lim = -x.y * invNp;
        if (even) {
          const float h0 = oma * sv[i].x + a * lre, h1 = oma * sv[i].y + a * lim;
          hs[2 * m] = h0;
          hs[2 * m + 1] = h1;
          if (hrow) {
            hrow[2 * m] = h0;
            hrow[2 * m + 1] = h1;
          }
        } else {
          const float h = oma * sv[i].x + a * ldexpf(second ? lim : lre, ex);
          hs[m] = h;
          if (hrow) hrow[m] = h;
        }
      }
    }
    if (!(mode & 2)) return;
    __syncthreads();
    src = hs;
  }
#pragma unroll
  for (int s = 0; s < VS; ++s) {
    const int p = 2 * VS * t + 2 * s;
    kr[s] = p < L ? src[p] : 0.f;
    ki[s] = p + 1 < L ? src[p + 1] : 0.f;
  }
  __syncthreads();
  select_unit<VS>(D, u, L, kr, ki, budgets, offsets, idx_out, sh, stage, kStage, t, true);
}

static int kvc_bluestein_logm(int L) {
  const int Np = (L & 1) ? L : L / 2;
  int logm = 0;
  while ((1 << logm) < 2 * Np - 1) ++logm;
  return logm;
}

// Scratch for lengths that are not powers of two (BluesteinScratch, or
// BigScratch from M = 32768 on).
size_t kvc_sss_scratch_bytes(int L, int units) {
  if ((L & (L - 1)) == 0) return 0;
  const int Np = (L & 1) ? L : L / 2;
  const int logm = kvc_bluestein_logm(L);
  if (logm >= KVC_BIG_LOGH) {
    const BigScratch b = kvc_big_scratch(Np, 1 << logm);
    return sizeof(float2) * (b.rows_off + b.ustride * (size_t)units);
  }
  const BluesteinScratch b = kvc_bluestein_scratch(Np, 1 << logm);
  return b.rows_off + b.bytes_per_unit * (size_t)units;
}

template <int S>
static hipError_t launch_big(const KvcDesc& D, const KvcSeqGroup& g, int nwg, int mode, int Np,
                             const float* s_in, float* s_hat_out, int32_t* kstar_out,
                             const int32_t* budgets, const int64_t* offsets, int32_t* idx_out,
                             float2* base, hipStream_t st) {
  constexpr int M = S * KVC_BIG_H;
  if (nwg > 65535) return hipErrorInvalidConfiguration;  // (grid y of the split)
  if (mode & 1) {
    hipLaunchKernelGGL(kvc_big_chirp_split_kernel<S>, dim3(KVC_BIG_H / 256), dim3(256), 0, st,
                       Np, base);
    hipLaunchKernelGGL(kvc_big_chirp_fft_kernel<S>, dim3(S), dim3(SSS_T), 0, st, base);
    const bool paired = (D.L[g.seq[0]] & 1) != 0;
    const int items = kvc_big_items(nwg, paired);
    if (paired)
      hipLaunchKernelGGL(kvc_big_scale_kernel, dim3(nwg), dim3(SSS_T), 0, st, D, g, Np, M,
                         s_in, base);
    hipLaunchKernelGGL((kvc_big_conv_kernel<S, true>), dim3(items * S), dim3(SSS_T), 0, st, D, g,
                       Np, s_in, base);
    hipLaunchKernelGGL(kvc_big_bins_kernel<S>, dim3(items * KVC_BIG_CH), dim3(256), 0, st, D, g,
                       Np, base);
    hipLaunchKernelGGL(kvc_big_kstar_kernel<S>, dim3(items), dim3(SSS_T), 0, st, D, mode, g, Np,
                       base, kstar_out);
    hipLaunchKernelGGL(kvc_big_merge_kernel<S>, dim3(items * (KVC_BIG_H / 1024)), dim3(256), 0,
                       st, D, g, Np, base);
    hipLaunchKernelGGL((kvc_big_conv_kernel<S, false>), dim3(items * S), dim3(SSS_T), 0, st, D,
                       g, Np, s_in, base);
  }
  if (D.L[g.seq[0]] > 32768)
    hipLaunchKernelGGL((kvc_big_finish_kernel<S, 32>), dim3(nwg), dim3(SSS_T), 0, st, D, mode, g,
                       Np, s_in, s_hat_out, budgets, offsets, idx_out, base);
  else
    hipLaunchKernelGGL((kvc_big_finish_kernel<S, 16>), dim3(nwg), dim3(SSS_T), 0, st, D, mode, g,
                       Np, s_in, s_hat_out, budgets, offsets, idx_out, base);
  return hipGetLastError();
}

// Units [u0, u1) must lie in one sequence.
hipError_t kvc_launch_sss_select(const KvcDesc& D, const KvcSeqGroup& g, int mode,
                                 const float* s_in, float* s_hat_out, int32_t* kstar_out,
                                 const int32_t* budgets, const int64_t* offsets, int32_t* idx_out,
                                 void* scratch, hipStream_t st) {
  const int nwg = g.n * (g.hi - g.lo);
  if (nwg <= 0) return hipSuccess;
  const int L = D.L[g.seq[0]];
  if ((L & (L - 1)) != 0) {
    if (!scratch && (mode & 1)) return hipErrorInvalidValue;
    const int Np = (L & 1) ? L : L / 2;
    const int logm = kvc_bluestein_logm(L);
    if (logm >= KVC_BIG_LOGH) {
      float2* base = (float2*)scratch;
      switch (logm) {
        case KVC_BIG_LOGH:
          return launch_big<1>(D, g, nwg, mode, Np, s_in, s_hat_out, kstar_out, budgets, offsets,
                               idx_out, base, st);
        case KVC_BIG_LOGH + 1:
          return launch_big<2>(D, g, nwg, mode, Np, s_in, s_hat_out, kstar_out, budgets, offsets,
                               idx_out, base, st);
        case KVC_BIG_LOGH + 2:
          return launch_big<4>(D, g, nwg, mode, Np, s_in, s_hat_out, kstar_out, budgets, offsets,
                               idx_out, base, st);
        default: return hipErrorInvalidValue;
      }
    }
    const BluesteinScratch b = kvc_bluestein_scratch(Np, 1 << logm);
    char* base = (char*)scratch;
    float2* bhat = scratch ? (float2*)base : nullptr;
    float2* cw = scratch ? (float2*)(base + b.chirp_off) : nullptr;
    float2* rows = scratch ? (float2*)(base + b.rows_off) : nullptr;
    void (*chirp)(int, float2*, float2*) = nullptr;
    void (*kern)(KvcDesc, int, KvcSeqGroup, const float*, float*, int32_t*, const int32_t*,
                 const int64_t*, int32_t*, float2*, const float2*, const float2*) = nullptr;
    switch (logm) {
#define KVC_GEN(LM) case LM: chirp = kvc_sss_chirp_kernel<LM>; kern = kvc_sss_general_kernel<LM>; break;
      KVC_GEN(7) KVC_GEN(8) KVC_GEN(9) KVC_GEN(10) KVC_GEN(11) KVC_GEN(12) KVC_GEN(13)
      KVC_GEN(14)
#undef KVC_GEN
      default: return hipErrorInvalidValue;
    }
    if (mode & 1) hipLaunchKernelGGL(chirp, dim3(1), dim3(SSS_T), 0, st, Np, bhat, cw);
    hipLaunchKernelGGL(kern, dim3(nwg), dim3(SSS_T), 0, st, D, mode, g, s_in, s_hat_out,
                       kstar_out, budgets, offsets, idx_out, rows, (const float2*)bhat,
                       (const float2*)cw);
    return hipGetLastError();
  }
  void (*kern)(KvcDesc, int, KvcSeqGroup, const float*, float*, int32_t*, const int32_t*,
               const int64_t*, int32_t*) = nullptr;
  switch (L) {
    case 64: kern = kvc_sss_select_kernel<5>; break;
    case 128: kern = kvc_sss_select_kernel<6>; break;
    case 256: kern = kvc_sss_select_kernel<7>; break;
    case 512: kern = kvc_sss_select_kernel<8>; break;
    case 1024: kern = kvc_sss_select_kernel<9>; break;
    case 2048: kern = kvc_sss_select_kernel<10>; break;
    case 4096: kern = kvc_sss_select_kernel<11>; break;
    case 8192: kern = kvc_sss_select_kernel<12>; break;
    case 16384: kern = kvc_sss_select_kernel<13>; break;
    case 32768: kern = kvc_sss_select_kernel<14>; break;
    case 65536: kern = kvc_sss_select_kernel<15>; break;
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(kern, dim3(nwg), dim3(SSS_T), 0, st, D, mode, g, s_in, s_hat_out,
                     kstar_out, budgets, offsets, idx_out);
  return hipGetLastError();
}
