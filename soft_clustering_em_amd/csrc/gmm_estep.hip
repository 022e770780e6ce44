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
//     tile are one dense contraction phi(X) (T x F) * W (F x K) and the
//     statistics are another, phi(X)^T (F x T) * R (T x K).  The logits run on
//     v_mfma_f32_16x16x4_f32; the statistics on v_mfma_f64_16x16x4_f64 with
//     features rebuilt in float64 (x, x*x and x_d*x_e are exact there), so
//     raw moments are summed without the cancellation that turning them into
//     variances would expose: a component that has collapsed onto a few rows
//     has a variance many orders below mu^2, and only float64 sums keep it.
//   * The float32 logit contraction is flushed into float64 every 32
//     features, and the per-component constant (and the spherical |x|^2 term)
//     is added in float64: the terms of the expanded quadratic form are far
//     larger than their sum.  Components whose precision times squared scale
//     is too large even for that ("sharp" ones, e.g. collapsed onto a row)
//     are flagged by the prologue; for them every log-score that comes within
//     60 (log2 units) of its row's maximum is recomputed in float64 from
//     direct differences, -1/2 (x - mu)^T P (x - mu) -- the scores further
//     down carry responsibilities below 2^-60 whatever their rounding.
//   * The logit accumulator's register layout (lane l holds component l%16 of
//     rows 4(l/16)+v) is exactly the B-operand layout the statistics MFMA
//     needs for R, so responsibilities go from the exponential straight into
//     the second contraction without an LDS transpose.
//   * Components are split across the waves of a workgroup (KW per wave).  A
//     wave reduces its own components (in-register fold + 16-lane DPP
//     all-reduce) to a per-row (max, sum of exp) pair; the pairs of all waves
//     meet in LDS once per tile and are combined in wave order.
//   * Rows arrive with global_load_lds_dwordx4 straight into a double-buffered
//     LDS tile while the previous tile computes; features are built from it
//     into a padded LDS tile read by both contractions.
//   * Workgroups stride over tiles (tile t -> workgroup t mod Gb), and each
//     writes its own partial slot: no atomics, fixed reduction order.
#include "gmm_device.h"
#include "gmm_internal.h"

#include <math.h>

namespace gmm {

// BM (components in blocks, see launch_estep_blocked): 0 = the whole step in
// one launch; 1 = per (row, block) the maximum and the sum of 2^(l - max) over
// the block's components, nothing else; 2 = responsibilities against the row's
// maximum and log2 sum over every block (lrow), statistics added to the
// problem's partials at the block's components.
template <int COV, int DP, int KW, int T, int BM = 0>
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
  constexpr double LN2 = 0.69314718055994530942;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int nthr = blockDim.x;
  const int NW = A.NW, KP = A.KP;
  const int b = blockIdx.x / A.Gb;  // (problem, block) when blocked
  const int g = blockIdx.x % A.Gb;
  const int bp = BM ? b / A.nblk : b;  // the problem
  const int jb = BM ? b % A.nblk : 0;  // its component block
  // this launch's first component in the (B, KPT) arrays
  const size_t kbase = BM ? (size_t)bp * A.KPT + (size_t)jb * KP : (size_t)b * KP;
  const int64_t N = A.N;
  const int D = (int)A.D;

  extern __shared__ float lds[];
  float* Wl = lds;                                             // KP*F, fragment order
  float* phi = Wl + (size_t)KP * F;                            // T*FS features
  float* raw0 = phi + T * FS;                                  // 2 (direct) or 1 x T*DP raw rows
  double* xsq = reinterpret_cast<double*>(raw0 + (A.direct ? 2 : 1) * T * DP);  // T (spherical), float64
  float* red = reinterpret_cast<float*>(xsq + T);              // NW*T*2: per-wave (max, sum)
  int* qtab = reinterpret_cast<int*>(red + 2 * NW * T);        // F: (d, e) of product features

  // ---- stage this problem's logit weights in LDS (linear copy, 16 B per lane)
  {
    const floatx4* src = reinterpret_cast<const floatx4*>(A.W + kbase * F);
    floatx4* dst = reinterpret_cast<floatx4*>(Wl);
    const int n4 = KP * F / 4;
    for (int i = threadIdx.x; i < n4; i += nthr) dst[i] = src[i];
  }
  if constexpr (QUAD) {
    for (int f = threadIdx.x; f < F; f += nthr)
      qtab[f] = f < DP ? ((f << 16) | 0xFFFF) : (f - DP < NQ ? quad_pair<DP>(f - DP) : -1);
  }
  double creg[NT], areg[NT];
  bool sharp[NT];
  bool any_sharp = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int k = wv * KW + nt * 16 + (lane & 15);
    creg[nt] = A.c[kbase + k];
    areg[nt] = (COV == SPH) ? A.a[kbase + k] : 0.0;
    sharp[nt] = A.sharp[kbase + k] != 0;
    // one decision per wave: does any of its components need the exact path
    any_sharp = any_sharp || (__builtin_amdgcn_ballot_w64(sharp[nt]) != 0);
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
  // statistic feature held by this lane in row tile mt: f = 16 mt + lane%16,
  // as (fd, fe): fe < 0 -> x_fd (or 0 when fd < 0); else x_fd * x_fe
  // (spherical and diagonal: x_f, or x_{f-DP}^2 in the diagonal's second
  // half, which starts at a 16-row tile boundary -- known per tile at compile time)
  int fd[QUAD ? GM : 1], fe[QUAD ? GM : 1];
  if constexpr (QUAD) {
#pragma unroll
    for (int mt = 0; mt < GM; ++mt) {
      const int f = mt * 16 + (lane & 15);
      fd[mt] = f;
      fe[mt] = -1;
      if (f >= DP) {
        if (f - DP < NQ) {
          const int de = quad_pair<DP>(f - DP);
          fd[mt] = de >> 16;
          fe[mt] = de & 0xFFFF;
        } else {
          fd[mt] = -1;
        }
      }
    }
  }

  // ---- rows: a tile of T rows x D floats.  Direct path: the rows of a tile
  // are contiguous and 16-byte aligned, so they are copied into LDS with
  // global_load_lds_dwordx4 (one 16-byte chunk per lane, lanes in order).
  const float* xb = reinterpret_cast<const float*>(A.x) + (size_t)bp * A.stride_b;
  const int rawstride = A.direct ? D : DP;  // floats per row in the raw LDS tile
  auto issue_tile = [&](int64_t tile, float* rawbuf) {
    const int64_t row0 = tile * T;
    const int64_t nrows = (N - row0) < T ? (N - row0) : T;
    const int nch = (int)(nrows * D / 4);  // valid 16-byte chunks of this tile
    for (int c0 = wv * 64; c0 < nch; c0 += nthr) {
      const int c = c0 + lane;
      if (c < nch)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(xb + row0 * D + (int64_t)c * 4),
            (__attribute__((address_space(3))) void*)(rawbuf + c0 * 4), 16, 0, 0);
    }
  };
  // element-wise staging (any row stride, any row type: 16-bit rows decoded
  // exactly to float32 here)
  auto load_tile_sync = [&](int64_t tile, float* rawbuf) {
    const int64_t row0 = tile * T;
    for (int j = threadIdx.x; j < T * DP; j += nthr) {
      const int r = j / DP, d = j % DP;
      const int64_t row = row0 + r;
      rawbuf[j] = (row < N && d < D) ? x_value(A.x, A.xtype, (int64_t)bp * A.stride_b + row * A.ld_x + d) : 0.f;
    }
  };

  int64_t t = g;
  int cur = 0;
  if (A.direct && t < A.ntiles) issue_tile(t, raw0);
  for (; t < A.ntiles; t += A.Gb, cur ^= 1) {
    const int64_t row0 = t * T;
    float* raw = A.direct ? raw0 + cur * T * DP : raw0;
    if (A.direct) wait_vmem();
    __syncthreads();  // rows of this tile have landed; every wave is done with the previous tile
    if (!A.direct) {
      load_tile_sync(t, raw);
      __syncthreads();
    }
    // ---- features of this tile (rows past N are zero)
    for (int j = threadIdx.x; j < T * (DP / 4); j += nthr) {
      const int r = j / (DP / 4), c4 = (j % (DP / 4)) * 4;
      floatx4 v = {0.f, 0.f, 0.f, 0.f};
      if (row0 + r < N) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (c4 + e < D) ? raw[r * rawstride + c4 + e] : 0.f;
      }
      *reinterpret_cast<float2*>(&phi[r * FS + c4]) = float2{v[0], v[1]};
      *reinterpret_cast<float2*>(&phi[r * FS + c4 + 2]) = float2{v[2], v[3]};
      if constexpr (COV == DIAG) {
        *reinterpret_cast<float2*>(&phi[r * FS + DP + c4]) = float2{v[0] * v[0], v[1] * v[1]};
        *reinterpret_cast<float2*>(&phi[r * FS + DP + c4 + 2]) = float2{v[2] * v[2], v[3] * v[3]};
      }
    }
    if constexpr (COV == SPH) {
      for (int r = threadIdx.x; r < T; r += nthr) {
        double s = 0.0;
        if (row0 + r < N)
          for (int d = 0; d < D; ++d) {
            const double x = (double)raw[r * rawstride + d];
            s += x * x;
          }
        xsq[r] = s;
      }
    }
    if constexpr (QUAD) {
      // product features: a thread takes one feature (d, e) for all T rows,
      // so the table lookup and its checks happen once per feature and the
      // rows run with compile-time offsets
      constexpr int NQP = F - DP;
      const int nvalid = (int)((N - row0) < T ? (N - row0) : T);
      for (int qi = threadIdx.x; qi < NQP; qi += nthr) {
        const int de = qtab[DP + qi];
        const int d = de >> 16, e = de & 0xFFFF;
        const bool ok = de >= 0 && d < D && e < D;
        const int dd = ok ? d : 0, ee = ok ? e : 0;
#pragma unroll
        for (int r = 0; r < T; ++r) {
          const float v = raw[r * rawstride + dd] * raw[r * rawstride + ee];
          phi[r * FS + DP + qi] = (ok && r < nvalid) ? v : 0.f;
        }
      }
    }
    // the next tile's rows into the other raw buffer, in flight during the compute below
    if (A.direct && t + A.Gb < A.ntiles) issue_tile(t + A.Gb, raw0 + (cur ^ 1) * T * DP);
    __syncthreads();  // features visible

    // ---- logits (log2 units): lg[rb][nt] = c + phi(X) W; float32 MFMA partial
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

    // ---- sharp components: every score that may come within 60 (log2 units)
    // of its row's top, again exactly.  Full and tied (a D x D product per
    // score): each lane lists its own (row block, component tile, row) items
    // and the wave loops only as often as its busiest lane needs, not once per
    // row position with any such lane.  Spherical and diagonal (D terms per
    // score): inline below, per row position.
    if (QUAD && any_sharp) {
      uint32_t todo = 0;  // bit (rb NT + nt) 4 + v
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float m = (float)lg[rb][0][v];
#pragma unroll
          for (int nt = 1; nt < NT; ++nt) m = fmaxf(m, (float)lg[rb][nt][v]);
          m = row16_max(m);
          const int p = rb * 16 + 4 * (lane >> 4) + v;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            if (sharp[nt] && (float)lg[rb][nt][v] >= m - 60.f && row0 + p < N) todo |= 1u << ((rb * NT + nt) * 4 + v);
        }
      static_assert(RB * NT * 4 <= 32, "one bit per item");
      while (__builtin_amdgcn_ballot_w64(todo != 0) != 0) {
        if (todo != 0) {
          const int bit = __builtin_ctz(todo);
          todo &= todo - 1;
          const int v = bit & 3, nt = (bit >> 2) % NT, rb = (bit >> 2) / NT;
          const int p = rb * 16 + 4 * (lane >> 4) + v;
          const int k = wv * KW + nt * 16 + (lane & 15);
          const double e = exact_score<COV, DP>(A, bp, jb * KP + k, D, phi + p * FS, BM ? A.KPT : 0);
#pragma unroll
          for (int rb2 = 0; rb2 < RB; ++rb2)
#pragma unroll
            for (int nt2 = 0; nt2 < NT; ++nt2)
#pragma unroll
              for (int v2 = 0; v2 < 4; ++v2)
                if ((rb2 * NT + nt2) * 4 + v2 == bit) lg[rb2][nt2][v2] = e;
        }
      }
    }

    // ---- per-wave row max and sum of exponentials over this wave's components
    float mrow[RB][4], srow[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float m = (float)lg[rb][0][v];
#pragma unroll
        for (int nt = 1; nt < NT; ++nt) m = fmaxf(m, (float)lg[rb][nt][v]);
        m = row16_max(m);
        if (!QUAD && any_sharp) {
          const int p = rb * 16 + 4 * (lane >> 4) + v;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if (sharp[nt] && (float)lg[rb][nt][v] >= m - 60.f && row0 + p < N) {
              const int k = wv * KW + nt * 16 + (lane & 15);
              lg[rb][nt][v] = exact_score<COV, DP>(A, bp, jb * KP + k, D, phi + p * FS, BM ? A.KPT : 0);
            }
          }
          m = (float)lg[rb][0][v];
#pragma unroll
          for (int nt = 1; nt < NT; ++nt) m = fmaxf(m, (float)lg[rb][nt][v]);
          m = row16_max(m);
        }
        if (m == -INFINITY) m = 0.f;  // no live component in this wave: every exp below is 0
        float s = 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float e = __builtin_amdgcn_exp2f((float)(lg[rb][nt][v] - (double)m));
          acc[rb][nt][v] = e;
          s += e;
        }
        mrow[rb][v] = m;
        srow[rb][v] = row16_sum(s);
      }
    // ---- combine the waves: M = max_w m_w, S = sum_w s_w 2^(m_w - M).
    // Each 16-lane group holds rows 4g..4g+3 of a row block; lane j of the
    // group takes row v = j/4 and waves q, q+4 (q = j%4), then the quad
    // (lanes 4v..4v+3) reduces with DPP and its first lane's result is
    // broadcast to the group with ds_swizzle.  Waves enter in a fixed order.
    float scale[RB][4];
    if constexpr (BM == 2) {
      // r = 2^(l - m_own) 2^(m_own - M - log2 S), M and log2 S of the row over every block
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int p = rb * 16 + 4 * (lane >> 4) + v;
          const bool valid = row0 + p < N;
          const float2 lr = A.lrow[(size_t)bp * A.ldl + (valid ? row0 + p : 0)];
          // the exponent is <= 0 (the wave's maximum is at most the row's, log2 S >= 0)
          // except for a wave with no live component, whose maximum was set to
          // 0 and whose terms are all 0: the clamp keeps its scale finite
          scale[rb][v] = valid ? __builtin_amdgcn_exp2f(fminf((mrow[rb][v] - lr.x) - lr.y, 0.f)) : 0.f;
        }
    } else if (NW > 1) {
      float* redm = red;            // [NW][T]
      float* reds = red + NW * T;   // [NW][T]
      if ((lane & 15) == 0)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int p = rb * 16 + 4 * (lane >> 4);
          *reinterpret_cast<floatx4*>(&redm[wv * T + p]) = floatx4{mrow[rb][0], mrow[rb][1], mrow[rb][2], mrow[rb][3]};
          *reinterpret_cast<floatx4*>(&reds[wv * T + p]) = floatx4{srow[rb][0], srow[rb][1], srow[rb][2], srow[rb][3]};
        }
      __syncthreads();
      const int j = lane & 15, vq = j >> 2, q = j & 3;
      const int w0 = q < NW ? q : NW - 1, w1 = q + 4 < NW ? q + 4 : NW - 1;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int p = rb * 16 + 4 * (lane >> 4) + vq;
        const float m0 = redm[w0 * T + p], s0 = reds[w0 * T + p];
        const float m1 = redm[w1 * T + p], s1 = reds[w1 * T + p];
        const bool ok0 = q < NW && s0 > 0.f, ok1 = q + 4 < NW && s1 > 0.f;
        float M = fmaxf(ok0 ? m0 : -INFINITY, ok1 ? m1 : -INFINITY);
        M = fmaxf(M, dpp_mov<0xB1>(M));
        M = fmaxf(M, dpp_mov<0x4E>(M));
        float S = (ok0 ? s0 * __builtin_amdgcn_exp2f(m0 - M) : 0.f) + (ok1 ? s1 * __builtin_amdgcn_exp2f(m1 - M) : 0.f);
        S = S + dpp_mov<0xB1>(S);
        S = S + dpp_mov<0x4E>(S);
        // this wave's share of row v: 2^(m_own - M) / S
        const float mown = vq == 0 ? mrow[rb][0] : vq == 1 ? mrow[rb][1] : vq == 2 ? mrow[rb][2] : mrow[rb][3];
        const bool valid = row0 + p < N && S > 0.f;
        // mown <= M except for a wave with no live component (mown set to 0,
        // every term 0), where 2^(0 - M) would overflow to +inf for a row
        // whose best score lies below -128 and 0 * inf give NaN: clamped
        const float sc = valid ? __builtin_amdgcn_exp2f(fminf(mown - M, 0.f)) / S : 0.f;
        if constexpr (BM == 1) {
          if (wv == 0 && q == 0 && row0 + p < N) A.pb[((size_t)bp * A.ldl + row0 + p) * A.nblk + jb] = float2{M, S};
        } else {
          if (wv == 0 && q == 0 && valid) ll += ((double)M + (double)__builtin_amdgcn_logf(S)) * LN2;
        }
        // broadcast lane 4v of the 16-lane group: and_mask 0x10, or_mask 4v
        scale[rb][0] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(sc), 0x10 | (0 << 5)));
        scale[rb][1] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(sc), 0x10 | (4 << 5)));
        scale[rb][2] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(sc), 0x10 | (8 << 5)));
        scale[rb][3] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(sc), 0x10 | (12 << 5)));
      }
    } else {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int p = rb * 16 + 4 * (lane >> 4) + v;
          const bool valid = row0 + p < N;
          scale[rb][v] = valid ? 1.0f / srow[rb][v] : 0.f;
          if constexpr (BM == 1) {
            if ((lane & 15) == 0 && valid)
              A.pb[((size_t)bp * A.ldl + row0 + p) * A.nblk + jb] = float2{mrow[rb][v], srow[rb][v]};
          } else {
            if ((lane & 15) == 0 && valid)
              ll += ((double)mrow[rb][v] + (double)__builtin_amdgcn_logf(srow[rb][v])) * LN2;
          }
        }
    }
    if constexpr (BM == 1) continue;  // the (max, sum) pass ends here
    // ---- responsibilities (rows past N get weight 0)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[rb][nt][v] *= scale[rb][v];

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
          if constexpr (QUAD) {
            if (fe[mt] < 0) {
              av = fd[mt] >= 0 ? (double)phi[prow * FS + fd[mt]] : 0.0;
            } else {
              av = (double)phi[prow * FS + fd[mt]] * (double)phi[prow * FS + fe[mt]];
            }
          } else if (COV == DIAG && mt * 16 >= DP) {
            const double xv = (double)phi[prow * FS + mt * 16 - DP + (lane & 15)];
            av = xv * xv;
          } else {
            av = (double)phi[prow * FS + mt * 16 + (lane & 15)];
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

  if constexpr (BM == 1) return;
  // ---- epilogue: this workgroup's float64 partial (blocked: the block's
  // components of the problem's partial, added to it after the first chunk)
  const size_t bg = (size_t)bp * A.Gb + g;
  constexpr int PR = 2 + G;
  double* part = BM ? A.part + (bg * (size_t)A.KPT + (size_t)jb * KP) * PR : A.part + bg * (size_t)KP * PR;
  const bool addp = BM == 2 && A.accumulate;
#pragma unroll
  for (int mt = 0; mt < GM; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int k = wv * KW + nt * 16 + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // float64 MFMA output layout: lane l holds rows l/16 + 4 v of column l%16
        const int row = mt * 16 + (lane >> 4) + 4 * v;
        double* dst = &part[(size_t)k * PR + 2 + row];
        *dst = addp ? *dst + sacc[mt][nt][v] : sacc[mt][nt][v];
      }
    }
  // N_k and sum r|x|^2: the four lanes l, l+16, l+32, l+48 hold the same component
  __syncthreads();
  double* red64 = reinterpret_cast<double*>(lds);  // reuse the weight tile (8*KP + 64 doubles fit in it)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int k = wv * KW + nt * 16 + (lane & 15);
    red64[(k * 4 + (lane >> 4)) * 2 + 0] = nk[nt];
    red64[(k * 4 + (lane >> 4)) * 2 + 1] = qs[nt];
  }
  if (wv == 0) red64[(size_t)KP * 8 + lane] = ll;  // row log-likelihoods, held by lanes of wave 0
  __syncthreads();
  for (int k = threadIdx.x; k < KP; k += nthr) {
    double s0 = 0.0, s1 = 0.0;
    for (int q = 0; q < 4; ++q) {
      s0 += red64[(k * 4 + q) * 2 + 0];
      s1 += red64[(k * 4 + q) * 2 + 1];
    }
    part[(size_t)k * PR + 0] = addp ? part[(size_t)k * PR + 0] + s0 : s0;
    part[(size_t)k * PR + 1] = addp ? part[(size_t)k * PR + 1] + s1 : s1;
  }
  if (BM == 0 && threadIdx.x == 0) {
    double s = 0.0;
    for (int q = 0; q < 64; ++q) s += red64[(size_t)KP * 8 + q];
    A.llpart[bg] = s;
  }
}

// Variants the planner may choose: the instantiated ones whose register
// allocation fits without spilling (checked with -Rpass-analysis=kernel-resource-usage).
static constexpr bool variant_ok(int cov, int dp, int kw, int t) {
  if (kw != 16 && kw != 32) return false;
  if (t != 16 && t != 32 && t != 64) return false;
  if (cov == SPH) {
    if (dp == 16 || dp == 32) return !(kw == 32 && t == 64);
    if (dp == 64) return kw == 16 || t <= 32;
    if (dp == 128) return kw == 16 ? t <= 32 : t == 16;
    return false;
  }
  if (cov == DIAG) {
    if (dp == 16 || dp == 32) return kw == 16 || t <= 32;
    if (dp == 64) return kw == 16 ? t <= 32 : t == 16;
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

// ------------------------------------------------------------------ dispatch
template <int COV, int DP, int KW, int T, int BM = 0>
static hipError_t launch_one(const Plan& p, const EStepArgs& a, hipStream_t s) {
  if constexpr (!variant_ok(COV, DP, KW, T) || (BM != 0 && COV != SPH && COV != DIAG)) {
    return hipErrorInvalidValue;  // never planned: not instantiated
  } else {
    auto kern = estep_kernel<COV, DP, KW, T, BM>;
    static bool attr_set = false;
    if (!attr_set) {
      (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
      attr_set = true;
    }
    // blocked: one workgroup row group per (problem, block)
    dim3 grid((unsigned)(p.B * (BM ? p.nblk : 1) * p.Gb)), block((unsigned)(64 * p.NW));
    hipLaunchKernelGGL(kern, grid, block, p.lds, s, a);
    return hipGetLastError();
  }
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

bool estep_variant_exists(int cov, int dp, int kw, int t) { return variant_ok(cov, dp, kw, t); }

// ------------------------------------------------------------ blocked components
// When a problem has more components than one workgroup holds, they go in
// nblk blocks of p.NW * p.KW, each (problem, block) a problem index of the
// launch with the rows shared (Flash-GMM Section 3's tiling, the row's
// normaliser taken over every block): the (max, sum) pass, the row combine,
// then the statistics pass, whose partials land at the block's components.
#define GMM_T_SWITCH_B(COV, DP, KW, BM)                         \
  switch (p.T) {                                                \
    case 16: return launch_one<COV, DP, KW, 16, BM>(p, a, s);   \
    case 32: return launch_one<COV, DP, KW, 32, BM>(p, a, s);   \
    case 64: return launch_one<COV, DP, KW, 64, BM>(p, a, s);   \
    default: return hipErrorInvalidValue;                       \
  }
#define GMM_KW_SWITCH_B(COV, DP, BM)                            \
  switch (p.KW) {                                               \
    case 16: GMM_T_SWITCH_B(COV, DP, 16, BM)                    \
    case 32: GMM_T_SWITCH_B(COV, DP, 32, BM)                    \
    default: return hipErrorInvalidValue;                       \
  }

template <int COV, int BM>
static hipError_t launch_blocked_cov(const Plan& p, const EStepArgs& a, hipStream_t s) {
  switch (p.DP) {
    case 16: GMM_KW_SWITCH_B(COV, 16, BM)
    case 32: GMM_KW_SWITCH_B(COV, 32, BM)
    case 64: GMM_KW_SWITCH_B(COV, 64, BM)
    case 128: GMM_KW_SWITCH_B(COV, 128, BM)
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_estep_blocked(const Plan& p, const EStepArgs& a, int mode, hipStream_t s) {
  if (p.cov == SPH) return mode == 1 ? launch_blocked_cov<SPH, 1>(p, a, s) : launch_blocked_cov<SPH, 2>(p, a, s);
  if (p.cov == DIAG) return mode == 1 ? launch_blocked_cov<DIAG, 1>(p, a, s) : launch_blocked_cov<DIAG, 2>(p, a, s);
  return hipErrorInvalidValue;
}

// The row combine: per row the maximum M over its blocks and
// S = sum_j S_j 2^(M_j - M) in float64, kept as (M, log2 S); the row's
// log-likelihood (M + log2 S) ln 2 summed per workgroup in thread order into
// its partial (added to it after the first chunk).  A row whose blocks all
// have S_j = 0 (no live component) gets (0, +inf): responsibilities 0, and no
// log-likelihood, as in the one-launch step.  grid: B * Gb blocks of 256.
__global__ void __launch_bounds__(256) block_combine_kernel(int64_t N, int nblk, int64_t ldl, int Gb,
                                                            const float2* __restrict__ pb, float2* __restrict__ lrow,
                                                            double* __restrict__ llpart, int accumulate) {
  constexpr double LN2 = 0.69314718055994530942;
  __shared__ double red[256];
  const int b = blockIdx.x / Gb, g = blockIdx.x % Gb;
  double ll = 0.0;
  for (int64_t row = (int64_t)g * 256 + threadIdx.x; row < N; row += (int64_t)Gb * 256) {
    const float2* P = pb + ((size_t)b * ldl + row) * nblk;
    float M = -INFINITY;
    for (int j = 0; j < nblk; ++j)
      if (P[j].y > 0.f) M = fmaxf(M, P[j].x);
    double S = 0.0;
    for (int j = 0; j < nblk; ++j)
      if (P[j].y > 0.f) S += (double)P[j].y * exp2((double)P[j].x - (double)M);
    float2 out = float2{0.f, INFINITY};
    if (S > 0.0) {
      const double l2 = log2(S);
      out = float2{M, (float)l2};
      ll += ((double)M + l2) * LN2;
    }
    lrow[(size_t)b * ldl + row] = out;
  }
  red[threadIdx.x] = ll;
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
    for (int i = 0; i < 256; ++i) sum += red[i];
    llpart[blockIdx.x] = (accumulate ? llpart[blockIdx.x] : 0.0) + sum;
  }
}

hipError_t launch_block_combine(int64_t B, int64_t N, int nblk, int64_t ldl, int Gb, const float2* pb, float2* lrow,
                                double* llpart, int accumulate, hipStream_t s) {
  hipLaunchKernelGGL(block_combine_kernel, dim3((unsigned)(B * Gb)), dim3(256), 0, s, N, nblk, ldl, Gb, pb, lrow,
                     llpart, accumulate);
  return hipGetLastError();
}

}  // namespace gmm
