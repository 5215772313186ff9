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

__device__ __forceinline__ int phys(int a) { return a; }

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
    for (int s = 0; s < V; ++s) lds[phys(widx(s))] = re[s];
    if (x.xw >= 0) lds[phys(x.xw)] = x.wre;
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) re[s] = lds[phys(ridx(s))];
    if (x.xr >= 0) x.rre = lds[phys(x.xr)];
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) lds[phys(widx(s))] = im[s];
    if (x.xw >= 0) lds[phys(x.xw)] = x.wim;
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) im[s] = lds[phys(ridx(s))];
    if (x.xr >= 0) x.rim = lds[phys(x.xr)];
  }
  __syncthreads();
}

// Same exchange with real and imaginary parts moved together (when the LDS
// buffer holds N complex values): two barriers instead of four.
template <int V, class WF, class RF>
__device__ __forceinline__ void exchange2(float (&re)[V], float (&im)[V], float2* lds, bool act,
                                          WF widx, RF ridx, Extra& x) {
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) lds[widx(s)] = make_float2(re[s], im[s]);
    if (x.xw >= 0) lds[x.xw] = make_float2(x.wre, x.wim);
  }
  __syncthreads();
  if (act) {
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const float2 v = lds[ridx(s)];
      re[s] = v.x;
      im[s] = v.y;
    }
    if (x.xr >= 0) {
      const float2 v = lds[x.xr];
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
  static constexpr int kFloats = kPair ? 2 * N : N;
};

template <int N, int V, class WF, class RF>
__device__ __forceinline__ void xchg(float (&re)[V], float (&im)[V], float* lds, bool act, WF widx,
                                     RF ridx, Extra& x) {
  if constexpr (Xbuf<N>::kPair)
    exchange2<V>(re, im, reinterpret_cast<float2*>(lds), act, widx, ridx, x);
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
template <int N, int V, int Ns, int RM = 32, class RF>
__device__ __forceinline__ void fft_stages(float (&re)[V], float (&im)[V], float* lds, int t,
                                           bool act, RF ridx_final, Extra& xf) {
  constexpr int T = N / V;
  constexpr int R = fft_radix(N, V, Ns, RM);
  constexpr int Nn = Ns * R;
  if (act) fft_pass<V, R, T, Ns>(re, im, t);
  auto wf = [&](int s) { return out_index<R, T, Ns>(s, t); };
  if constexpr (Nn >= N) {
    xchg<N, V>(re, im, lds, act, wf, ridx_final, xf);
  } else {
    constexpr int R2 = fft_radix(N, V, Nn, RM);
    Extra none{-1, -1, 0.f, 0.f, 0.f, 0.f};
    xchg<N, V>(re, im, lds, act, wf, [&](int s) { return in_index<R2, T, N>(s, t); }, none);
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

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // -0 and +0 are equal
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct SssShared {
  double sd[SSS_WAVES];
  int si[SSS_WAVES];
  int s3[2][3][SSS_WAVES];
  int kstar;
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
  const int hv = V / 2;
  // z_m = s_{2m} + i s_{2m+1}, in the order of the first radix-V pass.
  if (act) {
    const float2* z = reinterpret_cast<const float2*>(srow);
#pragma unroll
    for (int s = 0; s < V; ++s) {
      const float2 v = z[in_index<V, T, N>(s, t)];
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
  fft_stages<N, V, 1>(re, im, lds, t, act, pair_idx, xf);

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
  // Natural bin order: lower chunks (t ascending), bin N/2, upper chunks
  // (t descending).  Prefix energies from two block scans.
  double lo_tot, hi_tot;
  const double lo_before = block_scan<double>(lo_sum, sh.sd, &lo_tot);
  const double hi_incl = block_scan<double>(hi_sum, sh.sd, &hi_tot) + hi_sum;
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
  xchg<N, V>(re, im, lds, act, pair_idx, [&](int s) { return in_index<V, T, N>(s, t); }, xi);

  // Inverse FFT as conj(FFT(conj(x))) / N, ending in natural chunks
  // (slot s holds index tV + s).
#pragma unroll
  for (int s = 0; s < V; ++s) im[s] = -im[s];
  Extra none{-1, -1, 0.f, 0.f, 0.f, 0.f};
  fft_stages<N, V, 1>(re, im, lds, t, act, [&](int s) { return t * V + s; }, none);

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
  const int w = D.window;
  const int ncand = L - w;
  const int b = budgets[u];
  const int k = b - w;
  const int64_t off = offsets[u];
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
  // per bit (the reduction slots alternate between bits).  Per bit, the
  // keys still equal to T's prefix with that bit set are `hit`: they stay
  // equal if T takes the bit, else they are above T from then on.
  if (k > 0 && k < ncand) {
    int acnt = 0;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
      uint32_t hit[NG];
      int cnt = acnt;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        hit[g] = match[g] & P[g][bit];
        cnt += __popc(hit[g]);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
      if ((threadIdx.x & 63) == 0) sh.s3[bit & 1][0][threadIdx.x >> 6] = cnt;
      __syncthreads();
      int tot = 0;
#pragma unroll
      for (int i = 0; i < SSS_WAVES; ++i) tot += sh.s3[bit & 1][0][i];
      if (tot >= k) {
#pragma unroll
        for (int g = 0; g < NG; ++g) match[g] = hit[g];
      } else {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          above[g] |= hit[g];
          acnt += __popc(hit[g]);
          match[g] &= ~P[g][bit];
        }
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
  const int eq_before = block_scan<int>(neq, sh.si, &eq_total);
  block_scan<int>(ngt, sh.si, &gt_total);
  (void)eq_total;
  const bool take_all = k >= ncand;
  const bool take_none = k <= 0;
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
      else if (take_all) sel = true;
      else if (take_none) sel = false;
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
  const int base = block_scan<int>(nsel, sh.si, &nsel_total);
  if (b <= kStage) {
    // Compact into LDS, then one coalesced copy of the b positions.
    if (act) {
      int o = 0;
#pragma unroll
      for (int s = 0; s < 2 * V; ++s) {
        const bool sel = (s < 32) ? ((selmask_lo >> s) & 1u) : ((selmask_hi >> (s - 32)) & 1u);
        if (sel && base + o < b) stage[base + (o++)] = p0 + s;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < b; i += SSS_T) idx_out[off + i] = stage[i];
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
  __shared__ __attribute__((aligned(16))) float lds[Xbuf<N>::kFloats];
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
                   Xbuf<N>::kFloats, t, act);
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
// (m < 16384, so m^2 fits 32 bits).
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

static int kvc_bluestein_logm(int L) {
  const int Np = (L & 1) ? L : L / 2;
  int logm = 0;
  while ((1 << logm) < 2 * Np - 1) ++logm;
  return logm;
}

// Scratch for lengths that are not powers of two (see BluesteinScratch).
size_t kvc_sss_scratch_bytes(int L, int units) {
  if ((L & (L - 1)) == 0) return 0;
  const int Np = (L & 1) ? L : L / 2;
  const BluesteinScratch b = kvc_bluestein_scratch(Np, 1 << kvc_bluestein_logm(L));
  return b.rows_off + b.bytes_per_unit * (size_t)units;
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
      KVC_GEN(14) KVC_GEN(15)
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
