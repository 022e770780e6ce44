// gmm_topm.hip -- soft multi-assignment: for every row, the components of
// largest responsibility (Flash-GMM, Section 4 and Conclusion: vectors near a
// cluster boundary are stored in every list whose final responsibility passes
// a threshold).  Rank 1 is always kept; ranks 2..m are kept while
// r >= threshold; ties go to the lower component index.
//
// The decisions (order, threshold) are taken on float64 scores:
//   1. the float32 MFMA logits of the fused E-step give every score s~ with an
//      error bound E (per component from the prologue: err.x |x| + err.y |x|^2,
//      plus the float32 rounding of s~ itself), so s~ - E <= s <= s~ + E; each
//      row's Mt = max (s~ - E) is a lower bound of its true best score
//      (exchanged across the waves of the workgroup);
//   2. every component whose s~ + E reaches Mt - 32 (log2 units) is a
//      candidate and is rescored exactly, in float64, by direct differences:
//      every component within 32 of the true best is among them; the others
//      carry responsibilities below 2^-32 and enter the log-sum-exp only as
//      float32 terms;
//   3. per row the candidates are sorted (score descending, index ascending),
//      and LSE, responsibilities and the kept ranks follow in float64.
// A row with more than CAP candidates is rescored over all K components by
// one wave (the workgroup's waves take such rows in turn).
//
// Top-k mode (the approx_top_k training mode of the GMMXX README: a row keeps
// its k best log-scores and normalises over them): the candidate threshold is
// instead a lower bound of the row's k-th best true score -- the k-th largest
// of the per-lane maxima of s~ - E over the row's components (k different
// components reach it) -- so every component of the true top k is a
// candidate; the m = k best after rescoring are kept, with responsibilities
// and log-sum-exp over those k only.
#include "gmm_device.h"
#include "gmm_internal.h"

#include <math.h>

namespace gmm {

template <int COV, int DP, int KW>
__global__ void __launch_bounds__(512) topm_kernel(TopmArgs A) {
  constexpr int T = kTopmRows;
  constexpr int CAP = kTopmCap;
  constexpr int F = feat_F(COV, DP);
  constexpr int FS = feat_stride(F);
  constexpr int NT = KW / 16;
  constexpr int KQ = F / 16;
  constexpr int NQ = quad_count(DP);
  constexpr bool QUAD = (COV == FULL || COV == TIED);
  constexpr float DELTA = 32.f;
  constexpr double LN2 = 0.69314718055994530942;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nthr = blockDim.x;
  const int NW = A.NW, KP = A.KP, K = A.K;
  const int b = blockIdx.x / A.Gb;
  const int g = blockIdx.x % A.Gb;
  const int64_t N = A.N;
  const int D = (int)A.D;
  const int m = A.m;

  extern __shared__ float lds[];
  float* Wl = lds;                                          // KP*F, fragment order
  float* phi = Wl + (size_t)KP * F;                         // T*FS
  float* raw = phi + T * FS;                                // T*DP
  double* xsq = reinterpret_cast<double*>(raw + T * DP);    // T
  double* rednc = xsq + T;                                  // NW*T: per-wave sum of non-candidate terms
  double* cl = rednc + NW * T;                              // T*CAP candidate scores
  float* redm = reinterpret_cast<float*>(cl + T * CAP);     // NW*T per-wave row max
  int* ck = reinterpret_cast<int*>(redm + NW * T);          // T*CAP candidate indices
  int* cnt = ck + T * CAP;                                  // T
  int* qtab = cnt + T;                                      // F
  float* xnq = reinterpret_cast<float*>(qtab + F);          // T*2: |x|, |x|^2 of each row
  float* kth = xnq + 2 * T;                                 // T: top-k candidate threshold of each row
  float* lsc = reinterpret_cast<float*>(cl);                // top-k: T*16*NW per-lane maxima (before cl is used)
  const bool topk = A.topk != 0;

  {
    const float4* src = reinterpret_cast<const float4*>(A.W + (size_t)b * KP * F);
    float4* dst = reinterpret_cast<float4*>(Wl);
    for (int i = threadIdx.x; i < KP * F / 4; i += nthr) dst[i] = src[i];
  }
  if constexpr (QUAD) {
    for (int f = threadIdx.x; f < F; f += nthr)
      qtab[f] = f < DP ? ((f << 16) | 0xFFFF) : (f - DP < NQ ? quad_pair<DP>(f - DP) : -1);
  }
  double creg[NT], areg[NT];
  float ex[NT], ey[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int k = wv * KW + nt * 16 + (lane & 15);
    creg[nt] = A.c[(size_t)b * KP + k];
    areg[nt] = (COV == SPH) ? A.a[(size_t)b * KP + k] : 0.0;
    const float2 e = A.err[(size_t)b * KP + k];
    ex[nt] = e.x;
    ey[nt] = e.y;
  }
  const int64_t xoff = (int64_t)b * A.stride_b;  // first element of problem b (elements of the row type)

  // rows of the next tile are fetched into registers while this tile computes,
  // when a tile is at most PF elements per thread (uniform across the block)
  constexpr int PF = 4;
  const bool pre = T * DP <= PF * nthr;
  float pv[PF];
  auto fetch_rows = [&](int64_t tile) {
    const int64_t r0 = tile * T;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int j = threadIdx.x + i * nthr;
      float v = 0.f;
      if (j < T * DP) {
        const int r = j / DP, d = j % DP;
        if (r0 + r < N && d < D) v = x_value(A.x, A.xtype, xoff + (r0 + r) * A.ld_x + d);
      }
      pv[i] = v;
    }
  };
  if (pre && g < A.ntiles) fetch_rows(g);

  for (int64_t t = g; t < A.ntiles; t += A.Gb) {
    const int64_t row0 = t * T;
    __syncthreads();  // previous tile fully consumed
    if (pre) {
      // the prefetched rows, with their direct features
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        const int j = threadIdx.x + i * nthr;
        if (j < T * DP) {
          const int r = j / DP, d = j % DP;
          raw[j] = pv[i];
          phi[r * FS + d] = pv[i];
          if constexpr (COV == DIAG) phi[r * FS + DP + d] = pv[i] * pv[i];
        }
      }
      if (t + A.Gb < A.ntiles) fetch_rows(t + A.Gb);
    } else {
      for (int j = threadIdx.x; j < T * DP; j += nthr) {
        const int r = j / DP, d = j % DP;
        const int64_t row = row0 + r;
        raw[j] = (row < N && d < D) ? x_value(A.x, A.xtype, xoff + row * A.ld_x + d) : 0.f;
      }
    }
    for (int p = threadIdx.x; p < T; p += nthr) cnt[p] = 0;
    __syncthreads();  // the row norms below read whole rows
    if (!pre) {
      for (int j = threadIdx.x; j < T * DP; j += nthr) {
        const int r = j / DP, d = j % DP;
        const float v = raw[j];
        phi[r * FS + d] = v;
        if constexpr (COV == DIAG) phi[r * FS + DP + d] = v * v;
      }
    }
    for (int r = threadIdx.x; r < T; r += nthr) {
      double s = 0.0;
      for (int d = 0; d < D; ++d) s += (double)raw[r * DP + d] * (double)raw[r * DP + d];
      xsq[r] = s;
      xnq[2 * r] = (float)sqrt(s) * (1.f + 0x1p-20f);
      xnq[2 * r + 1] = (float)s * (1.f + 0x1p-20f);
    }
    if constexpr (QUAD) {
      constexpr int NQP = F - DP;
      for (int j = threadIdx.x; j < T * NQP; j += nthr) {
        const int r = j / NQP, qi = j % NQP;
        const int de = qtab[DP + qi];
        float v = 0.f;
        if (de >= 0) {
          const int d = de >> 16, e = de & 0xFFFF;
          v = raw[r * DP + d] * raw[r * DP + e];
        }
        phi[r * FS + DP + qi] = v;
      }
    }
    __syncthreads();

    // ---- approximate logits (log2 units), as in the fused E-step
    floatx4 acc[NT];
    double lg[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v) lg[nt][v] = creg[nt];
    const float* Wwave = Wl + (size_t)wv * NT * KQ * 256;
    for (int kq = 0; kq < KQ; ++kq) {
      if (kq % 2 == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      floatx4 bw[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bw[nt] = *reinterpret_cast<const floatx4*>(Wwave + ((nt * KQ + kq) * 64 + lane) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float av = phi[(lane & 15) * FS + (kq * 4 + j) * 4 + (lane >> 4)];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bw[nt][j], acc[nt], 0, 0, 0);
      }
      if (kq % 2 == 1 || kq == KQ - 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) lg[nt][v] += (double)acc[nt][v];
      }
    }
    if constexpr (COV == SPH) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const double xs = xsq[4 * (lane >> 4) + v];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) lg[nt][v] += areg[nt] * xs;
      }
    }
    // ---- error bounds: lo <= true score <= hi; the row maximum of lo
    float lo[NT][4], hi[NT][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = 4 * (lane >> 4) + v;
      const float xn = xnq[2 * p], xq = xnq[2 * p + 1];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float lv = (float)lg[nt][v];
        const float e = lv > -INFINITY ? fmaf(ex[nt], xn, ey[nt] * xq) + 0x1p-22f * fabsf(lv) : 0.f;
        lo[nt][v] = lv - e;
        hi[nt][v] = lv + e;
      }
    }
    float mw[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float mx = lo[0][v];
#pragma unroll
      for (int nt = 1; nt < NT; ++nt) mx = fmaxf(mx, lo[nt][v]);
      if (topk) lsc[(4 * (lane >> 4) + v) * (16 * NW) + wv * 16 + (lane & 15)] = mx;
      mw[v] = row16_max(mx);
    }
    if ((lane & 15) == 0)
      *reinterpret_cast<floatx4*>(&redm[wv * T + 4 * (lane >> 4)]) = floatx4{mw[0], mw[1], mw[2], mw[3]};
    __syncthreads();
    float Mt[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = 4 * (lane >> 4) + v;
      float mx = -INFINITY;
      for (int w2 = 0; w2 < NW; ++w2) mx = fmaxf(mx, redm[w2 * T + p]);
      Mt[v] = mx;
    }
    if (topk) {
      // per row (a wave each, in turn): the m-th largest of the 16 NW lane
      // maxima of lo -- m different components reach it, so the row's m-th
      // best true score is at least that
      for (int p = wv; p < T; p += NW) {
        const int nv = 16 * NW;
        float a0 = lane < nv ? lsc[p * nv + lane] : -INFINITY;
        float a1 = lane + 64 < nv ? lsc[p * nv + lane + 64] : -INFINITY;
        float mx = -INFINITY;
        for (int j = 0; j < m; ++j) {
          mx = (float)wave_max((double)fmaxf(a0, a1));
          const uint64_t b0 = __builtin_amdgcn_ballot_w64(a0 == mx);
          if (b0) {
            if (lane == (int)__builtin_ctzll(b0)) a0 = -INFINITY;
          } else {
            const uint64_t b1 = __builtin_amdgcn_ballot_w64(a1 == mx);
            if (b1 && lane == (int)__builtin_ctzll(b1)) a1 = -INFINITY;
          }
        }
        if (lane == 0) kth[p] = mx;
      }
      __syncthreads();
    }
    // ---- candidates: first counted (each takes a slot), the rest summed as
    // float32 terms; then, in rows whose candidates fit the list, rescored
    // exactly (a row past CAP is rescored over all K below instead)
    int slotv[NT][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = 4 * (lane >> 4) + v;
      const bool valid = row0 + p < N;
      const float thc = topk ? kth[p] : Mt[v] - DELTA;
      float nc = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float lv = (float)lg[nt][v];
        const int k = wv * KW + nt * 16 + (lane & 15);
        slotv[nt][v] = -1;
        if (valid && k < K && hi[nt][v] > -INFINITY && hi[nt][v] >= thc) {
          slotv[nt][v] = atomicAdd(&cnt[p], 1);
        } else if (!topk && valid && lv > -INFINITY) {
          nc += __builtin_amdgcn_exp2f(lv - Mt[v]);
        }
      }
      nc = row16_sum(nc);
      if ((lane & 15) == 0) rednc[wv * T + p] = (double)nc;
    }
    __syncthreads();  // every row's candidate count is final
    if constexpr (COV == SPH || COV == DIAG) {
      // the candidates' components into the lists; then their float64 scores
      // by direct differences: a wave per row in turn, its four 16-lane groups
      // four candidates at a time, lane li taking features li, li + 16, ...
      // (coalesced reads of the means), summed by a 16-lane DPP tree
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int p = 4 * (lane >> 4) + v;
        const bool fits = cnt[p] <= CAP;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          if (slotv[nt][v] >= 0 && fits) ck[p * CAP + slotv[nt][v]] = wv * KW + nt * 16 + (lane & 15);
      }
      __syncthreads();
      constexpr double kLog2e = 1.4426950408889634074;
      const int grp = lane >> 4, li = lane & 15;
      for (int p = wv; p < T; p += NW) {
        const int n = cnt[p];
        if (row0 + p >= N || n > CAP) continue;  // uniform across the wave
        for (int c0i = 0; c0i < n; c0i += 4) {
          const int c = c0i + grp;
          const int k = ck[p * CAP + (c < n ? c : n - 1)];
          const float* mu = A.mu + ((size_t)b * A.K + k) * D;
          const double* P = A.prec + ((size_t)b * A.KP + k) * (size_t)A.prec_stride;
          double q = 0.0;
          for (int d = li; d < D; d += 16) {
            const double t = (double)raw[p * DP + d] - (double)mu[d];
            q += (COV == DIAG ? P[d] : 1.0) * t * t;
          }
          q = row16_sum_f64(q);
          if constexpr (COV == SPH) q *= P[0];
          if (li == 0 && c < n) cl[p * CAP + c] = A.c0[(size_t)b * A.KP + k] - 0.5 * kLog2e * q;
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int p = 4 * (lane >> 4) + v;
        const bool fits = cnt[p] <= CAP;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int slot = slotv[nt][v];
          if (slot >= 0 && fits) {
            const int k = wv * KW + nt * 16 + (lane & 15);
            cl[p * CAP + slot] = exact_score<COV, DP, false>(A, b, k, D, raw + p * DP);
            ck[p * CAP + slot] = k;
          }
        }
      }
    }
    __syncthreads();

    // ---- per row: sort the candidates, LSE in float64, kept ranks
    for (int p = threadIdx.x; p < T; p += nthr) {
      const int64_t row = row0 + p;
      const int n = cnt[p];
      if (row >= N || n > CAP) continue;
      double* L = cl + p * CAP;
      int* Kx = ck + p * CAP;
      for (int i = 1; i < n; ++i) {  // insertion sort: score descending, index ascending
        const double li = L[i];
        const int ki = Kx[i];
        int j = i - 1;
        while (j >= 0 && before(li, ki, L[j], Kx[j])) {
          L[j + 1] = L[j];
          Kx[j + 1] = Kx[j];
          --j;
        }
        L[j + 1] = li;
        Kx[j + 1] = ki;
      }
      const double M = n > 0 ? L[0] : -INFINITY;
      double lse;
      int c = 0;
      if (topk) {
        // the m best, normalised over themselves
        const int kept = min(m, n);
        double S = 0.0;
        for (int j = 0; j < kept; ++j) S += exp2(L[j] - M);
        lse = M + log2(S);
        for (int j = 0; j < m; ++j) {
          A.idx[((size_t)b * N + row) * m + j] = j < kept ? Kx[j] : -1;
          A.resp[((size_t)b * N + row) * m + j] = j < kept ? (float)exp2(L[j] - lse) : 0.f;
        }
        c = kept;
      } else {
        float mt = -INFINITY;
        double ncs = 0.0;
        for (int w2 = 0; w2 < NW; ++w2) mt = fmaxf(mt, redm[w2 * T + p]);
        for (int w2 = 0; w2 < NW; ++w2) ncs += rednc[w2 * T + p];
        double S = 0.0;
        for (int j = 0; j < n; ++j) S += exp2(L[j] - M);
        S += ncs * exp2((double)mt - M);
        lse = M + log2(S);
        for (int j = 0; j < m; ++j) {
          int kk = -1;
          float rr = 0.f;
          if (j < n) {
            const double r = exp2(L[j] - lse);
            if ((j == 0 || r >= (double)A.thr) && c == j) {
              kk = Kx[j];
              rr = (float)r;
              ++c;
            }
          }
          A.idx[((size_t)b * N + row) * m + j] = kk;
          A.resp[((size_t)b * N + row) * m + j] = rr;
        }
      }
      if (A.count) A.count[(size_t)b * N + row] = c;
      if (A.logp) A.logp[(size_t)b * N + row] = (float)(lse * LN2);
    }
    __syncthreads();

    // ---- rows with more than CAP candidates: all K components, one wave per
    // row (row p to wave p mod NW); no barrier inside, every wave reaches the
    // next tile's
    {
      for (int p = wv; p < T; p += NW) {
        const int64_t row = row0 + p;
        if (row >= N || cnt[p] <= CAP) continue;  // uniform across the wave
        constexpr int PER = (kTopmMaxK + 63) / 64;
        double ls[PER];
        double mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int k = lane + 64 * i;
          ls[i] = k < K ? exact_score<COV, DP, false>(A, b, k, D, raw + p * DP) : -INFINITY;
          mx = fmax(mx, ls[i]);
        }
        const double M = wave_max(mx);
        double lse = 0.0;
        if (!topk) {
          double s = 0.0;
#pragma unroll
          for (int i = 0; i < PER; ++i) s += ls[i] > -INFINITY ? exp2(ls[i] - M) : 0.0;
          lse = M + log2(wave_sum(s));
        }
        // the m best (score, index), one per round; lane j keeps round j's
        double rl = -INFINITY;
        int rk = 0x7fffffff;
        for (int j = 0; j < m; ++j) {
          double bl = -INFINITY;
          int bk = 0x7fffffff;
#pragma unroll
          for (int i = 0; i < PER; ++i) {
            const int k = lane + 64 * i;
            if (k < K && before(ls[i], k, bl, bk)) { bl = ls[i]; bk = k; }
          }
          wave_best(bl, bk);
#pragma unroll
          for (int i = 0; i < PER; ++i)
            if (lane + 64 * i == bk) ls[i] = -INFINITY;  // taken
          if (lane == j) {
            rl = bl;
            rk = bk;
          }
        }
        // top-k: the log-sum-exp of the kept ones (round 0 holds the maximum)
        if (topk) lse = M + log2(wave_sum((lane < m && rk < K) ? exp2(rl - M) : 0.0));
        // the kept ranks are a prefix: top-k every one found; top-m rank 1, then
        // the ranks while r >= threshold
        const double r = rk < K ? exp2(rl - lse) : 0.0;
        const bool ok = lane < m && rk < K && (topk || lane == 0 || r >= (double)A.thr);
        const int c = (int)__builtin_ctzll(~__builtin_amdgcn_ballot_w64(ok));
        if (lane < m) {
          A.idx[((size_t)b * N + row) * m + lane] = lane < c ? rk : -1;
          A.resp[((size_t)b * N + row) * m + lane] = lane < c ? (float)r : 0.f;
        }
        if (lane == 0) {
          if (A.count) A.count[(size_t)b * N + row] = c;
          if (A.logp) A.logp[(size_t)b * N + row] = (float)(lse * LN2);
        }
      }
    }
  }
}

template <int COV, int DP, int KW>
static hipError_t launch_topm_one(const Plan& p, const TopmArgs& a, hipStream_t s) {
  auto kern = topm_kernel<COV, DP, KW>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.B * p.Gb)), dim3((unsigned)(64 * p.NW)), p.lds, s, a);
  return hipGetLastError();
}

#define GMM_TOPM_KW(COV, DP)                                      \
  switch (p.KW) {                                                 \
    case 16: return launch_topm_one<COV, DP, 16>(p, a, s);        \
    case 32: return launch_topm_one<COV, DP, 32>(p, a, s);        \
    default: return hipErrorInvalidValue;                         \
  }

template <int COV>
static hipError_t launch_topm_cov(const Plan& p, const TopmArgs& a, hipStream_t s) {
  if constexpr (COV == SPH || COV == DIAG) {
    switch (p.DP) {
      case 16: GMM_TOPM_KW(COV, 16)
      case 32: GMM_TOPM_KW(COV, 32)
      case 64: GMM_TOPM_KW(COV, 64)
      case 128: GMM_TOPM_KW(COV, 128)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (p.DP) {
      case 8: GMM_TOPM_KW(COV, 8)
      case 16: GMM_TOPM_KW(COV, 16)
      default: return hipErrorInvalidValue;
    }
  }
}

// ---------------------------------------------------------------- exact top-m
// Spherical and diagonal problems with more components than the tiled kernel
// holds (K > kTopmMaxK, float32-path rows): every score of a row exactly, in
// float64 by direct differences, c0_k - 1/2 log2(e) sum_d P_kd (x_d - mu_kd)^2
// (the oracle's own form), with a running log-sum-exp and the best m kept in
// registers (score descending, index ascending: the components arrive in
// increasing index, and an equal score never passes an earlier one).  One row
// per thread, its values in registers (float64); the components stream through
// LDS in tiles (means, precisions and constants as float64).
// The kept ranks follow the rule of topm_kernel.  At DP = 128 a row takes two
// lanes, each holding half its values (one row's 128 in registers spill): their
// partial sums meet by one exchange, and both lanes, with the same score, keep
// the same list.  grid: B * ceil(N / rows per block).
constexpr int kExactTile = 32;  // components per LDS tile (16 at DP = 128: static LDS stays under 64 KiB)
constexpr int kExactMaxM = 16;  // the widest m the API accepts

template <int DP>
constexpr int exact_split() { return DP >= 128 ? 2 : 1; }

template <int COV, int DP>
__global__ void __launch_bounds__(256) topm_exact_kernel(TopmArgs A) {
  constexpr double kLog2e = 1.4426950408889634074;
  constexpr double LN2 = 0.69314718055994530942;
  constexpr int PS = (COV == DIAG) ? DP : 1;  // precision values per component
  constexpr int SPLIT = exact_split<DP>();    // lanes per row
  constexpr int DH = DP / SPLIT;              // values per lane
  constexpr int RPB = 256 / SPLIT;            // rows per block
  constexpr int TILE = DP >= 128 ? kExactTile / 2 : kExactTile;
  __shared__ double smu[TILE * DP];
  __shared__ double sp[TILE * PS];
  __shared__ double sc0[TILE];
  const int nrb = (int)((A.N + RPB - 1) / RPB);
  const int b = blockIdx.x / nrb;
  const int half = SPLIT == 2 ? (threadIdx.x & 1) : 0;
  const int64_t row = (int64_t)(blockIdx.x % nrb) * RPB + threadIdx.x / SPLIT;
  const bool live = row < A.N;
  const int D = (int)A.D, K = A.K, m = A.m;
  const int64_t rc = live ? row : A.N - 1;
  const int d0 = half * DH;
  double x[DH];
#pragma unroll
  for (int d = 0; d < DH; ++d)
    x[d] = d0 + d < D ? (double)x_value(A.x, A.xtype, (int64_t)b * A.stride_b + rc * A.ld_x + d0 + d) : 0.0;
  double L[kExactMaxM];
  int Kx[kExactMaxM];
#pragma unroll
  for (int j = 0; j < kExactMaxM; ++j) {
    L[j] = -INFINITY;
    Kx[j] = 0x7fffffff;
  }
  double worst = -INFINITY;  // the m-th best so far
  int worstk = 0x7fffffff;
  double M = -INFINITY, S = 0.0;  // running maximum and sum of 2^(score - M)
  for (int k0 = 0; k0 < K; k0 += TILE) {
    const int nk = min(TILE, K - k0);
    __syncthreads();  // the previous tile is consumed
    for (int i = threadIdx.x; i < nk * DP; i += 256) {
      const int kk = i / DP, d = i % DP;
      smu[i] = d < D ? (double)A.mu[((size_t)b * K + k0 + kk) * D + d] : 0.0;
    }
    for (int i = threadIdx.x; i < nk * PS; i += 256) {
      const int kk = i / PS, d = i % PS;
      sp[i] = (COV == SPH || d < D) ? A.prec[((size_t)b * A.KP + k0 + kk) * (size_t)A.prec_stride + d] : 0.0;
    }
    for (int i = threadIdx.x; i < nk; i += 256) sc0[i] = A.c0[(size_t)b * A.KP + k0 + i];
    __syncthreads();
    for (int kk = 0; kk < nk; ++kk) {
      double q = 0.0;
#pragma unroll
      for (int d = 0; d < DH; ++d) {
        const double t = x[d] - smu[kk * DP + d0 + d];
        q = COV == DIAG ? fma(sp[kk * PS + d0 + d] * t, t, q) : fma(t, t, q);
      }
      if constexpr (SPLIT == 2) q += __shfl_xor(q, 1);  // the row's other half (a + b == b + a)
      if constexpr (COV == SPH) q *= sp[kk];
      const double sc = sc0[kk] - 0.5 * kLog2e * q;
      const int k = k0 + kk;
      if (!(sc > -INFINITY)) continue;  // a component without weight: no mass, never ranked
      if (sc > M) {
        S = S * exp2(M - sc) + 1.0;
        M = sc;
      } else {
        S += exp2(sc - M);
      }
      if (before(sc, k, worst, worstk)) {
        // insert into the kept list (fixed slots, so no register is indexed
        // at run time): the new entry sinks past every better one
        double cl = sc;
        int ck = k;
#pragma unroll
        for (int j = 0; j < kExactMaxM; ++j) {
          if (j < m && before(cl, ck, L[j], Kx[j])) {
            const double tl = L[j];
            const int tk = Kx[j];
            L[j] = cl;
            Kx[j] = ck;
            cl = tl;
            ck = tk;
          }
        }
#pragma unroll
        for (int j = 0; j < kExactMaxM; ++j)
          if (j == m - 1) {
            worst = L[j];
            worstk = Kx[j];
          }
      }
    }
  }
  if (!live || half != 0) return;
  const size_t o = ((size_t)b * A.N + row) * m;
  double lse;
  int c = 0;
  if (A.topk) {
    // the m best, normalised over themselves
    double St = 0.0;
#pragma unroll
    for (int j = 0; j < kExactMaxM; ++j)
      if (j < m && Kx[j] < K) St += exp2(L[j] - L[0]);
    lse = L[0] + log2(St);
  } else {
    lse = M + log2(S);
  }
#pragma unroll
  for (int j = 0; j < kExactMaxM; ++j) {
    if (j >= m) break;
    int kk = -1;
    float rr = 0.f;
    if (Kx[j] < K) {
      const double r = exp2(L[j] - lse);
      if ((A.topk || j == 0 || r >= (double)A.thr) && c == j) {
        kk = Kx[j];
        rr = (float)r;
        ++c;
      }
    }
    A.idx[o + j] = kk;
    A.resp[o + j] = rr;
  }
  if (A.count) A.count[(size_t)b * A.N + row] = c;
  if (A.logp) A.logp[(size_t)b * A.N + row] = (float)(lse * LN2);
}

template <int COV>
static hipError_t launch_topm_exact_cov(const Plan& p, const TopmArgs& a, hipStream_t s) {
  constexpr int RPB16 = 256 / exact_split<16>(), RPB128 = 256 / exact_split<128>();
  static_assert(RPB16 == 256 && RPB128 == 128, "rows per block");
  const int rpb = p.DP >= 128 ? RPB128 : RPB16;
  const unsigned grid = (unsigned)(p.B * ((p.N + rpb - 1) / rpb));
  switch (p.DP) {
    case 16: hipLaunchKernelGGL((topm_exact_kernel<COV, 16>), dim3(grid), dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((topm_exact_kernel<COV, 32>), dim3(grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((topm_exact_kernel<COV, 64>), dim3(grid), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((topm_exact_kernel<COV, 128>), dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topm_exact(const Plan& p, const TopmArgs& a, hipStream_t s) {
  if (p.cov == SPH) return launch_topm_exact_cov<SPH>(p, a, s);
  if (p.cov == DIAG) return launch_topm_exact_cov<DIAG>(p, a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_topm(const Plan& p, const TopmArgs& a, hipStream_t s) {
  switch (p.cov) {
    case SPH: return launch_topm_cov<SPH>(p, a, s);
    case DIAG: return launch_topm_cov<DIAG>(p, a, s);
    case FULL: return launch_topm_cov<FULL>(p, a, s);
    case TIED: return launch_topm_cov<TIED>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmm
