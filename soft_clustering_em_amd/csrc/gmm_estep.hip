// gmm_estep.hip -- the fused E-step + sufficient-statistics kernel.
//
// What it computes ("Flash-GMM: A Memory-Efficient Kernel for Scalable Soft
// Clustering", Section 2 and Section 3): for every row x_i of a tile, the
// log-scores l_ik = log pi_k + log N(x_i | theta_k) of all K components, the
// row log-sum-exp, the responsibilities r_ik = exp(l_ik - LSE_i), and their
// responsibility-weighted sums N_k, sum r x, sum r x x (in the feature basis),
// plus sum_i LSE_i.  The N x K matrix of responsibilities lives only in
// registers; what reaches memory is one O(K D) partial per workgroup.
//
// How it is laid out on gfx950 (CDNA4):
//   * Every log-score is linear in a feature vector phi(x) (x, x^2, or the
//     products x_d x_e) plus a per-component constant, so the logits of a
//     tile are one dense contraction
//     phi(X) (T x F) * W (F x K) and the statistics are another,
//     phi(X)^T (F x T) * R (T x K).  The logits run on v_mfma_f32_16x16x4_f32;
//     the statistics on v_mfma_f64_16x16x4_f64 with features rebuilt in
//     float64 (x, x*x and x_d*x_e are exact there), so raw moments are summed
//     without the cancellation that turning them into variances would expose:
//     a component that has collapsed onto a few rows has a variance many
//     orders below mu^2, and only float64 sums keep it.
//   * The logit accumulator's register layout (lane l holds component l%16 of
//     rows 4(l/16)+v) is exactly the B-operand layout the statistics MFMA needs
//     for R, so responsibilities go from the exponential straight into the
//     second contraction without an LDS transpose.
//   * The float32 logit contraction is flushed into float64 every 32
//     features, and the per-component constant (and the spherical |x|^2 term)
//     is added in float64: the terms of the expanded quadratic form are far
//     larger than their sum, and a float32 accumulator alone would lose the
//     absolute accuracy that the responsibilities of distant rows need.
//   * Components are split across the waves of a workgroup (KW per wave); a
//     row's max and sum over its own KW components is a 16-lane DPP all-reduce
//     plus an in-register fold, and the per-wave partials meet in LDS.
//   * The tile of features is staged once in LDS and read by both
//     contractions; the next tile's rows are loaded into registers while the
//     current tile computes.
//   * N_k (and, for spherical components, sum r |x|^2) accumulate on the VALU
//     in float64; the workgroup partial is written in float64.
//   * Workgroups stride over tiles (tile t -> workgroup t mod Gb), and each
//     writes its own partial slot: no atomics, fixed reduction order.
#include "gmm_internal.h"

#include <math.h>

namespace gmm {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

// 16-lane all-reduce with DPP (quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror,
// row_mirror); every lane of a 16-lane row ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_mov<0xB1>(v);
  v = v + dpp_mov<0x4E>(v);
  v = v + dpp_mov<0x141>(v);
  v = v + dpp_mov<0x140>(v);
  return v;
}


template <int COV, int DP, int KW, int T>
__global__ void __launch_bounds__(512) estep_kernel(EStepArgs A) {
  constexpr int F = feat_F(COV, DP);
  constexpr int G = feat_G(COV, DP);
  constexpr int FS = feat_stride(F > G ? F : G);
  constexpr int NT = KW / 16;   // 16-component column tiles per wave
  constexpr int RB = T / 16;    // 16-row blocks per tile
  constexpr int GM = G / 16;    // 16-row statistic tiles
  constexpr int KQ = F / 16;    // groups of 4 MFMA k-steps
  constexpr int NQ = quad_count(DP);
  constexpr bool QUAD = (COV == FULL || COV == TIED);
  constexpr float LN2 = 0.693147180559945309f;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nthr = blockDim.x;
  const int NW = A.NW, KP = A.KP;
  const int b = blockIdx.x / A.Gb;
  const int g = blockIdx.x % A.Gb;
  const int64_t N = A.N;
  const int D = (int)A.D;

  extern __shared__ float lds[];
  float* Wl = lds;                          // KP*F, fragment order
  float* phi = Wl + (size_t)KP * F;         // T*FS features
  double* xsq = reinterpret_cast<double*>(phi + T * FS);  // T (spherical), float64
  float* redm = reinterpret_cast<float*>(xsq + T);         // NW*T
  float* reds = redm + NW * T;              // NW*T

  // ---- stage this problem's logit weights in LDS (linear copy, 16 B per lane)
  {
    const floatx4* src = reinterpret_cast<const floatx4*>(A.W + (size_t)b * KP * F);
    floatx4* dst = reinterpret_cast<floatx4*>(Wl);
    const int n4 = KP * F / 4;
    for (int i = threadIdx.x; i < n4; i += nthr) dst[i] = src[i];
  }
  double creg[NT], areg[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int k = wv * KW + nt * 16 + (lane & 15);
    creg[nt] = A.c[(size_t)b * KP + k];
    areg[nt] = (COV == SPH) ? A.a[(size_t)b * KP + k] : 0.0;
  }

  doublex4 sacc[GM][NT];
  double nk[NT], qs[NT];
#pragma unroll
  for (int mt = 0; mt < GM; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = doublex4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) nk[nt] = qs[nt] = 0.0;
  double ll = 0.0;
  // statistic feature held by this lane in row tile mt: f = 16 mt + lane%16;
  // for the product features its two factors (d, e); -1 marks padding
  int fd[GM], fe[GM];
#pragma unroll
  for (int mt = 0; mt < GM; ++mt) {
    const int f = mt * 16 + (lane & 15);
    fd[mt] = f;
    fe[mt] = -1;
    if constexpr (COV == DIAG) {
      if (f >= DP) { fd[mt] = f - DP; fe[mt] = f - DP; }
    } else if constexpr (QUAD) {
      if (f >= DP) {
        int q = f - DP, d = 0, base = 0;
        if (q < NQ) {
          while (q >= base + (DP - d)) { base += DP - d; ++d; }
          fd[mt] = d;
          fe[mt] = d + (q - base);
        } else {
          fd[mt] = -1;
        }
      }
    }
  }

  // ---- register prefetch of one tile of rows (x part only)
  // Each thread owns rows/columns of the tile in 4-element chunks:
  // chunk j -> row j / (DP/4), columns 4*(j % (DP/4)) .. +3.
  constexpr int CPR = DP / 4;                  // chunks per row
  constexpr int NCH = T * CPR;                 // chunks per tile
  // chunks per thread held in registers between tiles (at most four, i.e. 16
  // registers); a tile with more chunks than that is loaded directly instead
  constexpr int MAXC = (NCH + 63) / 64 < 4 ? (NCH + 63) / 64 : 4;
  const bool prefetch = NCH <= MAXC * nthr;
  floatx4 pre[MAXC];
  const float* xb = reinterpret_cast<const float*>(A.x) + (size_t)b * A.stride_b;

  auto load_chunk = [&](int64_t row0, int j) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (j < NCH) {
      const int r = j / CPR, c4 = (j % CPR) * 4;
      const int64_t row = row0 + r;
      if (row < N) {
        const float* src = xb + row * A.ld_x + c4;
        if (A.vec4 && c4 + 4 <= D) {
          v = *reinterpret_cast<const floatx4*>(src);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (c4 + e < D) ? src[e] : 0.f;
        }
      }
    }
    return v;
  };
  auto load_tile = [&](int64_t tile) {
#pragma unroll
    for (int q = 0; q < MAXC; ++q) pre[q] = load_chunk(tile * T, threadIdx.x + q * nthr);
  };
  auto store_chunk = [&](int j, floatx4 v) {
    const int r = j / CPR, c4 = (j % CPR) * 4;
    *reinterpret_cast<float2*>(&phi[r * FS + c4]) = float2{v[0], v[1]};
    *reinterpret_cast<float2*>(&phi[r * FS + c4 + 2]) = float2{v[2], v[3]};
    if constexpr (COV == DIAG) {
      *reinterpret_cast<float2*>(&phi[r * FS + DP + c4]) = float2{v[0] * v[0], v[1] * v[1]};
      *reinterpret_cast<float2*>(&phi[r * FS + DP + c4 + 2]) = float2{v[2] * v[2], v[3] * v[3]};
    }
  };

  int64_t t = g;
  if (prefetch && t < A.ntiles) load_tile(t);
  for (; t < A.ntiles; t += A.Gb) {
    const int64_t row0 = t * T;
    __syncthreads();  // every wave is done reading the previous tile's features
    // ---- features: x part (and x^2 for diag), from the prefetch registers
    if (prefetch) {
#pragma unroll
      for (int q = 0; q < MAXC; ++q) {
        const int j = threadIdx.x + q * nthr;
        if (j < NCH) store_chunk(j, pre[q]);
      }
    } else {
      for (int j = threadIdx.x; j < NCH; j += nthr) store_chunk(j, load_chunk(row0, j));
    }
    if constexpr (COV == SPH || QUAD) {
      __syncthreads();
      if constexpr (COV == SPH) {
        for (int r = threadIdx.x; r < T; r += nthr) {
          double s = 0.0;
#pragma unroll 8
          for (int d = 0; d < DP; ++d) s += (double)phi[r * FS + d] * (double)phi[r * FS + d];
          xsq[r] = s;
        }
      } else {
        // products x_d x_e, d <= e, upper triangle in row-major order, then zero padding
        constexpr int NQP = F - DP;
        for (int j = threadIdx.x; j < T * NQP; j += nthr) {
          const int r = j / NQP, qi = j % NQP;
          float v = 0.f;
          if (qi < NQ) {
            // invert qi -> (d, e): row d holds DP - d entries
            int d = 0, base = 0;
            while (qi >= base + (DP - d)) { base += DP - d; ++d; }
            const int e = d + (qi - base);
            v = phi[r * FS + d] * phi[r * FS + e];
          }
          phi[r * FS + DP + qi] = v;
        }
      }
    }
    __syncthreads();  // features of this tile are visible
    if (prefetch && t + A.Gb < A.ntiles) load_tile(t + A.Gb);  // in flight during the compute below

    // ---- logits (log2 units): lg[rb][nt] = c + phi(X) W, float32 MFMA partial
    // sums over 32 features flushed into float64
    floatx4 acc[RB][NT];
    double lg[RB][NT][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) lg[rb][nt][v] = creg[nt];
    const float* Wwave = Wl + (size_t)wv * NT * KQ * 256;
#pragma unroll 2
    for (int kq = 0; kq < KQ; ++kq) {
      if (kq % 2 == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[rb][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      floatx4 bw[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bw[nt] = *reinterpret_cast<const floatx4*>(Wwave + ((nt * KQ + kq) * 64 + lane) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ks = kq * 4 + j;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float av = phi[(rb * 16 + (lane & 15)) * FS + ks * 4 + (lane >> 4)];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[rb][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bw[nt][j], acc[rb][nt], 0, 0, 0);
        }
      }
      if (kq % 2 == 1 || kq == KQ - 1) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) lg[rb][nt][v] += (double)acc[rb][nt][v];
      }
    }
    if constexpr (COV == SPH) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const double xs = xsq[rb * 16 + 4 * (lane >> 4) + v];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) lg[rb][nt][v] += areg[nt] * xs;
        }
    }

    // ---- row max over all components (a float32 shift; any value near the max will do)
    float mrow[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float m = (float)lg[rb][0][v];
#pragma unroll
        for (int nt = 1; nt < NT; ++nt) m = fmaxf(m, (float)lg[rb][nt][v]);
        mrow[rb][v] = row16_max(m);
      }
    if (NW > 1) {
      if ((lane & 15) == 0)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int v = 0; v < 4; ++v) redm[wv * T + rb * 16 + 4 * (lane >> 4) + v] = mrow[rb][v];
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int p = rb * 16 + 4 * (lane >> 4) + v;
          float m = redm[p];
          for (int w2 = 1; w2 < NW; ++w2) m = fmaxf(m, redm[w2 * T + p]);
          mrow[rb][v] = m;
        }
    }
    // ---- exponentials and row sums
    float srow[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float s = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float e = __builtin_amdgcn_exp2f((float)(lg[rb][nt][v] - (double)mrow[rb][v]));
          acc[rb][nt][v] = e;
          s += e;
        }
        srow[rb][v] = row16_sum(s);
      }
    if (NW > 1) {
      if ((lane & 15) == 0)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int v = 0; v < 4; ++v) reds[wv * T + rb * 16 + 4 * (lane >> 4) + v] = srow[rb][v];
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int p = rb * 16 + 4 * (lane >> 4) + v;
          float s = 0.f;
          for (int w2 = 0; w2 < NW; ++w2) s += reds[w2 * T + p];
          srow[rb][v] = s;
        }
    }
    // ---- responsibilities (rows past N get weight 0) and the log-likelihood
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int p = rb * 16 + 4 * (lane >> 4) + v;
        const bool valid = row0 + p < N;
        const float inv = valid ? 1.0f / srow[rb][v] : 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rb][nt][v] *= inv;
        if (wv == 0 && (lane & 15) == 0 && valid)
          ll += ((double)mrow[rb][v] + (double)__builtin_amdgcn_logf(srow[rb][v])) * (double)LN2;
      }

    // ---- statistics: sacc[mt][nt] += phi(X)^T R in float64; N_k (and sum r |x|^2) on the VALU
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int prow = rb * 16 + 4 * (lane >> 4) + s;
        double bop[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) bop[nt] = (double)acc[rb][nt][s];
#pragma unroll
        for (int mt = 0; mt < GM; ++mt) {
          double av;
          if constexpr (COV == SPH) {
            av = (double)phi[prow * FS + fd[mt]];
          } else {
            if (fe[mt] < 0) {
              av = fd[mt] >= 0 ? (double)phi[prow * FS + fd[mt]] : 0.0;
            } else {
              av = (double)phi[prow * FS + fd[mt]] * (double)phi[prow * FS + fe[mt]];
            }
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            sacc[mt][nt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bop[nt], sacc[mt][nt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) nk[nt] += (double)acc[rb][nt][v];
      if constexpr (COV == SPH) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const double xs = xsq[rb * 16 + 4 * (lane >> 4) + v];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) qs[nt] += (double)acc[rb][nt][v] * xs;
        }
      }
    }
  }

  // ---- epilogue: this workgroup's float64 partial
  const size_t bg = (size_t)b * A.Gb + g;
  double* part = A.part + bg * (size_t)KP * (2 + G);
  constexpr int PR = 2 + G;
#pragma unroll
  for (int mt = 0; mt < GM; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int k = wv * KW + nt * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // float64 MFMA output layout: lane l holds rows l/16 + 4 v of column l%16
        const int row = mt * 16 + (lane >> 4) + 4 * v;
        part[(size_t)k * PR + 2 + row] = sacc[mt][nt][v];
      }
    }
  // N_k and sum r|x|^2: the four lanes l, l+16, l+32, l+48 hold the same component
  __syncthreads();
  double* red64 = reinterpret_cast<double*>(lds);  // reuse the weight tile: KP*F floats >= 8*KP+4 doubles
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int k = wv * KW + nt * 16 + (lane & 15);
    red64[(k * 4 + (lane >> 4)) * 2 + 0] = nk[nt];
    red64[(k * 4 + (lane >> 4)) * 2 + 1] = qs[nt];
  }
  if (wv == 0 && (lane & 15) == 0) {
    // row log-likelihoods: lanes 0, 16, 32, 48 of wave 0 hold them
    red64[(size_t)KP * 8 + (lane >> 4)] = ll;
  }
  __syncthreads();
  for (int k = threadIdx.x; k < KP; k += nthr) {
    double s0 = 0.0, s1 = 0.0;
    for (int q = 0; q < 4; ++q) {
      s0 += red64[(k * 4 + q) * 2 + 0];
      s1 += red64[(k * 4 + q) * 2 + 1];
    }
    part[(size_t)k * PR + 0] = s0;
    part[(size_t)k * PR + 1] = s1;
  }
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int q = 0; q < 4; ++q) s += red64[(size_t)KP * 8 + q];
    A.llpart[bg] = s;
  }
}

// ------------------------------------------------------------------ dispatch
template <int COV, int DP, int KW, int T>
static hipError_t launch_one(const Plan& p, const EStepArgs& a, hipStream_t s) {
  auto kern = estep_kernel<COV, DP, KW, T>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytes);
    attr_set = true;
  }
  dim3 grid((unsigned)(p.B * p.Gb)), block((unsigned)(64 * p.NW));
  hipLaunchKernelGGL(kern, grid, block, p.lds, s, a);
  return hipGetLastError();
}

#define GMM_T_SWITCH(COV, DP, KW)                               \
  switch (p.T) {                                                \
    case 16: return launch_one<COV, DP, KW, 16>(p, a, s);       \
    case 32: return launch_one<COV, DP, KW, 32>(p, a, s);       \
    case 64: return launch_one<COV, DP, KW, 64>(p, a, s);       \
    default: return hipErrorInvalidValue;                       \
  }
#define GMM_KW_SWITCH(COV, DP)                                  \
  switch (p.KW) {                                               \
    case 16: GMM_T_SWITCH(COV, DP, 16)                          \
    case 32: GMM_T_SWITCH(COV, DP, 32)                          \
    default: return hipErrorInvalidValue;                       \
  }

template <int COV>
static hipError_t launch_cov(const Plan& p, const EStepArgs& a, hipStream_t s) {
  if constexpr (COV == SPH || COV == DIAG) {
    switch (p.DP) {
      case 16: GMM_KW_SWITCH(COV, 16)
      case 32: GMM_KW_SWITCH(COV, 32)
      case 64: GMM_KW_SWITCH(COV, 64)
      case 128: GMM_KW_SWITCH(COV, 128)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (p.DP) {
      case 8: GMM_KW_SWITCH(COV, 8)
      case 16: GMM_KW_SWITCH(COV, 16)
      default: return hipErrorInvalidValue;
    }
  }
}

hipError_t launch_estep(const Plan& p, const EStepArgs& a, hipStream_t s) {
  switch (p.cov) {
    case SPH: return launch_cov<SPH>(p, a, s);
    case DIAG: return launch_cov<DIAG>(p, a, s);
    case FULL: return launch_cov<FULL>(p, a, s);
    case TIED: return launch_cov<TIED>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

// Variants the planner may choose: the instantiated ones whose register
// allocation fits without spilling (checked with -Rpass-analysis=kernel-resource-usage).
bool estep_variant_exists(int cov, int dp, int kw, int t) {
  if (kw != 16 && kw != 32) return false;
  if (t != 16 && t != 32 && t != 64) return false;
  if (cov == SPH) {
    if (dp == 16) return true;
    if (dp == 32 || dp == 64) return !(kw == 32 && t == 64);
    if (dp == 128) return kw == 16 ? t <= 32 : t == 16;
    return false;
  }
  if (cov == DIAG) {
    if (dp == 16 || dp == 32) return !(kw == 32 && t == 64);
    if (dp == 64) return kw == 16 || t == 16;
    if (dp == 128) return kw == 16 && t == 16;
    return false;
  }
  if (cov == FULL || cov == TIED) {
    if (dp == 8) return t <= 32;
    if (dp == 16) return kw == 16 && t == 16;
    return false;
  }
  return false;
}

}  // namespace gmm
