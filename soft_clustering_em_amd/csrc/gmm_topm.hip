// gmm_topm.hip -- soft multi-assignment: for every row, the components of
// largest responsibility (Flash-GMM, Section 4 and Conclusion: vectors near a
// cluster boundary are stored in every list whose final responsibility passes
// a threshold).  Rank 1 is always kept; ranks 2..m are kept while
// r >= threshold; ties go to the lower component index.
//
// The decisions (order, threshold) are taken on float64 scores:
//   1. the float32 MFMA logits of the fused E-step give each row an
//      approximate maximum Mt (exchanged across the waves of the workgroup);
//   2. every component whose approximate score is within 32 (log2 units) of
//      Mt is a candidate and is rescored exactly, in float64, by direct
//      differences; the others carry responsibilities below 2^-32 and enter
//      the log-sum-exp only as float32 terms;
//   3. per row the candidates are sorted (score descending, index ascending),
//      and LSE, responsibilities and the kept ranks follow in float64.
// A row with more than CAP candidates is rescored over all K components by
// one wave (the workgroup's waves take such rows in turn).
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
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int k = wv * KW + nt * 16 + (lane & 15);
    creg[nt] = A.c[(size_t)b * KP + k];
    areg[nt] = (COV == SPH) ? A.a[(size_t)b * KP + k] : 0.0;
  }
  const float* xb = reinterpret_cast<const float*>(A.x) + (size_t)b * A.stride_b;

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
        if (r0 + r < N && d < D) v = xb[(r0 + r) * A.ld_x + d];
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
        raw[j] = (row < N && d < D) ? xb[row * A.ld_x + d] : 0.f;
      }
    }
    for (int p = threadIdx.x; p < T; p += nthr) cnt[p] = 0;
    // diagonal features are complete when prefetched; the rest need the whole tile
    if (!pre || COV != DIAG) __syncthreads();
    if (!pre) {
      for (int j = threadIdx.x; j < T * DP; j += nthr) {
        const int r = j / DP, d = j % DP;
        const float v = raw[j];
        phi[r * FS + d] = v;
        if constexpr (COV == DIAG) phi[r * FS + DP + d] = v * v;
      }
    }
    if constexpr (COV == SPH) {
      for (int r = threadIdx.x; r < T; r += nthr) {
        double s = 0.0;
        for (int d = 0; d < D; ++d) s += (double)raw[r * DP + d] * (double)raw[r * DP + d];
        xsq[r] = s;
      }
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
    // ---- approximate row maximum over all components
    float mw[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float mx = (float)lg[0][v];
#pragma unroll
      for (int nt = 1; nt < NT; ++nt) mx = fmaxf(mx, (float)lg[nt][v]);
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
    // ---- candidates: first counted (each takes a slot), the rest summed as
    // float32 terms; then, in rows whose candidates fit the list, rescored
    // exactly (a row past CAP is rescored over all K below instead)
    int slotv[NT][4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int p = 4 * (lane >> 4) + v;
      const bool valid = row0 + p < N;
      float nc = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float lv = (float)lg[nt][v];
        slotv[nt][v] = -1;
        if (valid && lv >= Mt[v] - DELTA) {
          slotv[nt][v] = atomicAdd(&cnt[p], 1);
        } else if (valid && lv > -INFINITY) {
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
      float mt = -INFINITY;
      double ncs = 0.0;
      for (int w2 = 0; w2 < NW; ++w2) mt = fmaxf(mt, redm[w2 * T + p]);
      for (int w2 = 0; w2 < NW; ++w2) ncs += rednc[w2 * T + p];
      const double M = L[0];
      double S = 0.0;
      for (int j = 0; j < n; ++j) S += exp2(L[j] - M);
      S += ncs * exp2((double)mt - M);
      const double lse = M + log2(S);
      int c = 0;
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
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < PER; ++i) s += ls[i] > -INFINITY ? exp2(ls[i] - M) : 0.0;
        const double lse = M + log2(wave_sum(s));
        int c = 0;
        for (int j = 0; j < m; ++j) {
          // best remaining (score, index) over the wave
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
          const double r = exp2(bl - lse);
          const bool keep = bk < K && (j == 0 || r >= (double)A.thr) && c == j;
          if (lane == 0) {
            A.idx[((size_t)b * N + row) * m + j] = keep ? bk : -1;
            A.resp[((size_t)b * N + row) * m + j] = keep ? (float)r : 0.f;
          }
          if (keep) ++c;
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
