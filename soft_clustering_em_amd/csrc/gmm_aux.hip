// gmm_aux.hip -- the small kernels around the fused E-step:
//   prologue : theta -> logit weights W (fragment order) and constants c
//   reduce   : fixed-order float64 sum of the workgroup partials, converted to
//              statistics centred at the input means
//   mstep    : the M-step on O(K D) data
//
// The log-score of component k (Flash-GMM, Section 2: the unnormalised score
// pi_k N(x | mu_k, Sigma_k), taken in log space) is written as a linear
// function of a feature vector phi(x) plus a constant:
//   log pi_k N(x|mu_k,Sigma_k) = log pi_k - 1/2 (D log 2pi + log det Sigma_k
//                                 + mu^T P mu) + x^T P mu - 1/2 x^T P x,
// with P = Sigma_k^{-1}.  The prologue evaluates the weights of that linear
// form in float64 and stores them (times log2 e) as float32.
#include "gmm_internal.h"

#include <math.h>

#include <algorithm>

namespace gmm {

static constexpr double kLog2e = 1.4426950408889634074;
// A component is "sharp" when the terms of its expanded log-score reach
// lambda_max * (|mu|^2 + tr Sigma) > kSharp: float32 products and partial sums
// of that size no longer give the log-score to the accuracy the
// responsibilities need, and the fused kernel evaluates it in float64.
static constexpr double kSharp = 1.0e4;
static constexpr double kLog2Pi = 1.8378770664093454836;
// Error coefficient of the approximate (float32-MFMA) log-score: its float32
// products and partial sums over each group of 32 features (then added in
// float64) carry at most about 34 roundings of 2^-24 of the sum of the
// absolute terms; 2^-18 (64 roundings) leaves a margin.  The sum of absolute
// terms is bounded per component by L1 |x| + Q |x|^2 (L1 = |linear weights|,
// Q bounds the quadratic ones), see prologue_kernel.
static constexpr double kScoreErr = 0x1p-18;

__device__ __forceinline__ size_t wfrag_index(int k, int f, int KW, int F) {
  const int w = k / KW, kk = k % KW, nt = kk / 16, col = kk % 16;
  const int ks = f / 4, kq = ks / 4, j = ks % 4, lane = (f % 4) * 16 + col;
  const int NT = KW / 16, KQ = F / 16;
  return ((((size_t)(w * NT + nt) * KQ + kq) * 64 + lane) * 4 + j);
}

// row-major upper-triangle index of (d, e), d <= e, in a DP x DP matrix
__device__ __forceinline__ int quad_index(int d, int e, int DP) { return d * DP - d * (d - 1) / 2 + (e - d); }

// Cholesky A = L L^T in place by the threads of a block.  A (row-major, row
// stride ld, float64, in LDS) holds a D x D (D <= 16) symmetric matrix on entry and L
// in its lower triangle on return (the upper triangle keeps its entries).
// Right-looking: for column j the pivot l_jj = sqrt(a_jj), the column below
// it divided by l_jj, then the trailing lower triangle updated by
// a_ik -= l_ij l_kj (j < k <= i), so every entry subtracts its products in the
// order p = 0, 1, ...  Returns whether A is positive definite (the same on
// every thread).  Every thread of the block calls it (it holds barriers).
__device__ bool chol_block(int D, double* A, int ld) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  for (int j = 0; j < D; ++j) {
    __syncthreads();
    // a_jj is not written again once column j has been formed
    const double piv = A[j * ld + j];
    if (!(piv > 0.0)) return false;  // every thread read the same value
    const double l = sqrt(piv);
    for (int i = j + 1 + tid; i < D; i += nthr) A[i * ld + j] /= l;
    __syncthreads();
    // trailing entries (i, k), j < k <= i < D, on a 16-wide grid of threads
    for (int t = tid; t < (D - 1 - j) * 16; t += nthr) {
      const int i = j + 1 + (t >> 4), k = j + 1 + (t & 15);
      if (k <= i) A[i * ld + k] -= A[i * ld + j] * A[k * ld + j];
    }
  }
  __syncthreads();
  for (int d = tid; d < D; d += nthr) A[d * ld + d] = sqrt(A[d * ld + d]);
  __syncthreads();
  return true;
}

// fixed-order (butterfly) sum over the 64 lanes of a wave
__device__ __forceinline__ double wave_sum64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ double wave_max64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}

// ------------------------------------------------------------------ prologue
// Component (b, k) by the threads of one block (any multiple of 64; every
// thread calls it, it holds barriers).  Its sums run on the first wave in a
// fixed lane order, so the values do not depend on the block size: the
// prologue kernel (64 threads) and the reduction's M-step blocks (which form
// the next iteration's prologue in gmm_fit) write the same bits.
__device__ __forceinline__ void prologue_component(int cov, int D, int K, int KP, int DP, int F, int KW, int b, int k,
                                   const float* __restrict__ w, const float* __restrict__ mu,
                                   const float* __restrict__ cv, float2* __restrict__ err, float* __restrict__ W,
                                   double* __restrict__ prec, int prec_stride, double* __restrict__ c0,
                                   double* __restrict__ c, double* __restrict__ a, int32_t* __restrict__ flag,
                                   int32_t* __restrict__ sharp) {
  const int tid = threadIdx.x;
  const bool w0 = tid < 64;  // the reductions run on the block's first wave
  float* Wb = W + (size_t)b * KP * F;
  double* precb = prec + ((size_t)b * KP + k) * prec_stride;
  __shared__ double sm_mu[128];
  __shared__ double sm_v[128];                // diag precisions / P mu
  __shared__ double sm_S[16 * 16], sm_L[16 * 16], sm_Li[16 * 16], sm_P[16 * 16];
  __shared__ double sm_c;
  __shared__ int sm_ok;

  if (k >= K) {  // padding component: never responsible
    for (int f = tid; f < F; f += blockDim.x) Wb[wfrag_index(k, f, KW, F)] = 0.f;
    if (tid == 0) {
      if (err) err[(size_t)b * KP + k] = float2{0.f, 0.f};
      c[(size_t)b * KP + k] = -INFINITY;
      c0[(size_t)b * KP + k] = -INFINITY;
      a[(size_t)b * KP + k] = 0.0;
      flag[(size_t)b * KP + k] = 0;
      sharp[(size_t)b * KP + k] = 0;
    }
    return;
  }
  for (int d = tid; d < D; d += blockDim.x) sm_mu[d] = (double)mu[((size_t)b * K + k) * D + d];
  const double logpi = log((double)w[(size_t)b * K + k]);
  __syncthreads();

  if (cov == SPH || cov == DIAG) {
    // precisions lambda_d (spherical: one value)
    for (int d = tid; d < D; d += blockDim.x)
      sm_v[d] = (cov == SPH) ? 1.0 / (double)cv[(size_t)b * K + k] : 1.0 / (double)cv[((size_t)b * K + k) * D + d];
    __syncthreads();
    // per-dimension terms on the block's threads (one log per variance;
    // spherical: one log in all), then fixed-order wave sums
    double logdet = 0.0, quad = 0.0, scale = 0.0, lmax = 0.0, l1 = 0.0, bad = 0.0;
    for (int d = tid; w0 && d < D; d += 64) {
      const double v = (cov == SPH) ? (double)cv[(size_t)b * K + k] : (double)cv[((size_t)b * K + k) * D + d];
      if (!(v > 0.0) || isinf(v)) bad = 1.0;
      if (cov == DIAG) logdet += log(v);
      quad += sm_v[d] * sm_mu[d] * sm_mu[d];
      lmax = fmax(lmax, sm_v[d]);
      scale += sm_mu[d] * sm_mu[d] + v;
      l1 += (sm_v[d] * sm_mu[d]) * (sm_v[d] * sm_mu[d]);
    }
    if (w0) {
      logdet = wave_sum64(logdet);
      quad = wave_sum64(quad);
      scale = wave_sum64(scale);
      lmax = wave_max64(lmax);
      l1 = wave_sum64(l1);
      bad = wave_max64(bad);
    }
    if (tid == 0) {
      const bool ok = bad == 0.0;
      // spherical: the lambda |x|^2 term is added in float64, only x . (lambda mu)
      // runs in float32; diagonal: sum_d lambda_d x_d^2 / 2 <= lambda_max |x|^2 / 2
      if (err)
        err[(size_t)b * KP + k] = ok ? float2{(float)(kScoreErr * kLog2e * sqrt(l1)),
                                              (float)(cov == DIAG ? kScoreErr * kLog2e * 0.5 * lmax : 0.0)}
                                     : float2{0.f, 0.f};
      if (cov == SPH) logdet = D * log((double)cv[(size_t)b * K + k]);
      sm_ok = ok;
      sm_c = ok ? (logpi - 0.5 * (D * kLog2Pi + logdet + quad)) * kLog2e : -INFINITY;
      c0[(size_t)b * KP + k] = ok ? (logpi - 0.5 * (D * kLog2Pi + logdet)) * kLog2e : -INFINITY;
      sharp[(size_t)b * KP + k] = (ok && lmax * scale > kSharp) ? 1 : 0;
    }
    if (cov == SPH) {
      if (tid == 0) precb[0] = sm_v[0];
    } else {
      for (int d = tid; d < D; d += blockDim.x) precb[d] = sm_v[d];
    }
    __syncthreads();
    const bool ok = sm_ok;
    for (int f = tid; f < F; f += blockDim.x) {
      double val = 0.0;
      if (ok) {
        if (f < DP) {
          if (f < D) val = sm_v[f] * sm_mu[f] * kLog2e;
        } else if (cov == DIAG && f - DP < D) {
          val = -0.5 * sm_v[f - DP] * kLog2e;
        }
      }
      Wb[wfrag_index(k, f, KW, F)] = (float)val;
    }
    if (tid == 0) {
      c[(size_t)b * KP + k] = sm_c;
      a[(size_t)b * KP + k] = (cov == SPH && ok) ? -0.5 * sm_v[0] * kLog2e : 0.0;
      flag[(size_t)b * KP + k] = ok ? 0 : 4;
    }
    return;
  }

  // full / tied: P = Sigma^{-1} through the Cholesky factor Sigma = L L^T;
  // sm_L, sm_Li and sm_P are 16 x 16 with row stride 16
  const float* S = (cov == FULL) ? cv + ((size_t)b * K + k) * D * D : cv + (size_t)b * D * D;
  for (int i = tid; i < D * D; i += blockDim.x) {
    sm_S[i] = (double)S[i];
    sm_L[(i / D) * 16 + i % D] = (double)S[i];
  }
  const bool ok = chol_block(D, sm_L, 16);  // starts and ends with a barrier
  if (ok) {
    // column j of L^{-1} on lane j: forward substitution on e_j (its entries
    // above row j are zero, so the products over p < j add nothing); only the
    // lower triangle of sm_L is read
    if (tid < 16) {
      const int j = tid;
      double col[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        double t = (i == j) ? 1.0 : 0.0;
#pragma unroll
        for (int p = 0; p < i; ++p) t -= sm_L[i * 16 + p] * col[p];
        col[i] = (i < j) ? 0.0 : t / sm_L[i * 16 + i];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sm_Li[i * 16 + j] = col[i];
    }
    __syncthreads();
    // P = L^{-T} L^{-1}, four entries per thread
    for (int i = tid; i < 256; i += blockDim.x) {
      const int d = i / 16, e = i % 16;
      double s = 0.0;
      if (d < D && e < D)
        for (int p = 0; p < D; ++p) s += sm_Li[p * 16 + d] * sm_Li[p * 16 + e];
      sm_P[i] = s;
    }
    __syncthreads();
    // per-thread terms, then fixed-order wave sums: lambda_max(P) <=
    // ||P^2||_F^(1/2) = (sum_i lambda_i^4)^(1/4) (P symmetric positive
    // definite), an upper bound far tighter than tr P when the eigenvalues are
    // spread; sum over d <= e of |x_d x_e W_de| = |x|^T |P| |x| / 2 <=
    // ||P||_F |x|^2 / 2 bounds the quadratic terms
    double s4 = 0.0, pf = 0.0;
    for (int i = tid; w0 && i < 256; i += 64) {
      const int d = i / 16, e = i % 16;
      double s = 0.0;
      for (int p = 0; p < D; ++p) s += sm_P[d * 16 + p] * sm_P[p * 16 + e];
      s4 += s * s;
      pf += sm_P[i] * sm_P[i];
    }
    double logdet = 0.0, quad = 0.0, scale = 0.0, l1 = 0.0;
    if (tid < D) {
      const int d = tid;
      double v = 0.0;
      for (int e = 0; e < D; ++e) v += sm_P[d * 16 + e] * sm_mu[e];
      sm_v[d] = v;
      logdet = 2.0 * log(sm_L[d * 16 + d]);
      quad = sm_mu[d] * v;
      scale = sm_mu[d] * sm_mu[d] + sm_S[d * D + d];
      l1 = v * v;
    }
    if (w0) {
      s4 = wave_sum64(s4);
      pf = wave_sum64(pf);
      logdet = wave_sum64(logdet);
      quad = wave_sum64(quad);
      scale = wave_sum64(scale);
      l1 = wave_sum64(l1);
    }
    if (tid == 0) {
      const double lmax = sqrt(sqrt(s4));
      if (err)
        err[(size_t)b * KP + k] = float2{(float)(kScoreErr * kLog2e * sqrt(l1)), (float)(kScoreErr * kLog2e * 0.5 * sqrt(pf))};
      sm_c = (logpi - 0.5 * (D * kLog2Pi + logdet + quad)) * kLog2e;
      c0[(size_t)b * KP + k] = (logpi - 0.5 * (D * kLog2Pi + logdet)) * kLog2e;
      sharp[(size_t)b * KP + k] = lmax * scale > kSharp ? 1 : 0;
    }
    for (int i = tid; i < DP * DP; i += blockDim.x) {
      const int d = i / DP, e = i % DP;
      precb[i] = (d < D && e < D) ? sm_Li[d * 16 + e] : 0.0;
    }
  }
  __syncthreads();
  for (int f = tid; f < F; f += blockDim.x) {
    double val = 0.0;
    if (ok) {
      if (f < DP) {
        if (f < D) val = sm_v[f] * kLog2e;
      } else if (f - DP < quad_count(DP)) {
        // invert the upper-triangle index
        int q = f - DP, d = 0, base = 0;
        while (q >= base + (DP - d)) { base += DP - d; ++d; }
        const int e = d + (q - base);
        if (d < D && e < D) val = (d == e ? -0.5 : -1.0) * sm_P[d * 16 + e] * kLog2e;
      }
    }
    Wb[wfrag_index(k, f, KW, F)] = (float)val;
  }
  if (tid == 0) {
    c[(size_t)b * KP + k] = ok ? sm_c : -INFINITY;
    a[(size_t)b * KP + k] = 0.0;
    flag[(size_t)b * KP + k] = ok ? 0 : 4;
    if (!ok) {
      sharp[(size_t)b * KP + k] = 0;
      if (err) err[(size_t)b * KP + k] = float2{0.f, 0.f};
    }
  }
}

// grid: B*KP blocks of 64 threads; block (b, k).
__global__ void __launch_bounds__(64) prologue_kernel(int cov, int D, int K, int KP, int DP, int F, int KW,
                                                      const float* __restrict__ w, const float* __restrict__ mu,
                                                      const float* __restrict__ cv, float2* __restrict__ err,
                                                      float* __restrict__ W,
                                                      double* __restrict__ prec, int prec_stride,
                                                      double* __restrict__ c0, double* __restrict__ c,
                                                      double* __restrict__ a, int32_t* __restrict__ flag,
                                                      int32_t* __restrict__ sharp) {
  prologue_component(cov, D, K, KP, DP, F, KW, blockIdx.x / KP, blockIdx.x % KP, w, mu, cv, err, W, prec,
                     prec_stride, c0, c, a, flag, sharp);
}

hipError_t launch_prologue(const Plan& p, const float* w, const float* mu, const float* cv, float2* err, float* W,
                           double* prec, double* c0, double* c, double* a, int32_t* flag, int32_t* sharp,
                           hipStream_t s) {
  hipLaunchKernelGGL(prologue_kernel, dim3((unsigned)(p.B * p.KP)), dim3(64), 0, s, p.cov, (int)p.D, (int)p.K,
                     p.KP, p.DP, p.F, p.KW, w, mu, cv, err, W, prec, p.prec_stride, c0, c, a, flag, sharp);
  return hipGetLastError();
}

// mean log-likelihood of B problems over n_total rows (the streamed fit step,
// whose per-chunk reductions add into ll)
__global__ void mean_ll_kernel(int64_t B, const double* __restrict__ ll, int64_t n_total, double* __restrict__ mean_ll) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) mean_ll[b] = ll[b] / (double)n_total;
}

hipError_t launch_mean_ll(int64_t B, const double* ll, int64_t n_total, double* mean_ll, hipStream_t s) {
  hipLaunchKernelGGL(mean_ll_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, B, ll, n_total, mean_ll);
  return hipGetLastError();
}

__device__ __forceinline__ void mstep_component(int cov, int D, int b, int K, int k, const double* __restrict__ nk,
                                const double* __restrict__ sx, const double* __restrict__ sxx, int64_t n_total,
                                float* w, float* mu, float* cv, double reg, const int32_t* in_flag,
                                int in_flag_stride, int32_t* comp_status, double* sm_delta, double* sm_S,
                                double* sm_L);

// ------------------------------------------------------------------ reduce
// grid: B*K + B blocks.  Block (b, k) sums the Gb partials of component k in
// workgroup order (float64) into raw[b][k][:], and (non-tied) writes the
// statistics centred at the input means.  Blocks B*K + b sum the
// log-likelihood partials.  Tied covariance is centred by centre_tied_kernel.
__global__ void __launch_bounds__(1024) reduce_kernel(int cov, int D, int K, int KP, int DP, int PR, int Gb, int llG,
                                                     int64_t N, const double* __restrict__ part,
                                                     const double* __restrict__ llpart,
                                                     const float* __restrict__ mu, double* __restrict__ raw,
                                                     double* nk, double* sx, double* sxx, double* ll,
                                                     double* mean_ll, int accumulate, int B, MstepFuse M) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  extern __shared__ double sm[];
  __shared__ double sm_S[16 * 16], sm_L[16 * 16];
  // fixed-order sum of n values v(g), g = 0..n-1, split into nseg contiguous
  // segments (segment q: thread-local sum, sixteen loads in flight), the
  // segment sums then added in segment order
  auto seg_sum = [&](const double* src, size_t stride, int n, int nseg, int q) {
    const int g0 = (int)((int64_t)n * q / nseg), g1 = (int)((int64_t)n * (q + 1) / nseg);
    double s = 0.0;
    int g = g0;
    for (; g + 16 <= g1; g += 16) {
      double v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = src[(size_t)(g + u) * stride];
#pragma unroll
      for (int u = 0; u < 16; ++u) s += v[u];
    }
    for (; g < g1; ++g) s += src[(size_t)g * stride];
    return s;
  };
  if ((int64_t)blockIdx.x >= (int64_t)B * K) {
    const int b = blockIdx.x - B * K;
    // thread segments, summed per wave by a fixed butterfly, then the wave
    // sums in wave order
    const double v = wave_sum64(seg_sum(llpart + (size_t)b * llG, 1, llG, nthr, tid));
    if ((tid & 63) == 0) sm[tid >> 6] = v;
    __syncthreads();
    if (tid == 0) {
      double s = 0.0;
      for (int q = 0; q < nthr / 64; ++q) s += sm[q];
      ll[b] = accumulate ? ll[b] + s : s;
      if (mean_ll) mean_ll[b] = s / (double)N;
    }
    return;
  }
  const int b = blockIdx.x / K, k = blockIdx.x % K;
  double* r = sm;            // PR
  double* m = sm + PR;       // D
  double* segs = m + D;      // PR * nseg <= nthr
  const size_t stride = (size_t)KP * PR;
  // each statistic over the workgroups 0..Gb-1: in nseg segments when the
  // statistics are fewer than the threads
  const int nseg = std::max(1, nthr / PR);
  const double* src0 = part + ((size_t)b * Gb * KP + k) * PR;
  if (nseg == 1) {
    for (int j = tid; j < PR; j += nthr) r[j] = seg_sum(src0 + j, stride, Gb, 1, 0);
  } else {
    // neighbouring threads take neighbouring statistics of one segment, so
    // their loads coalesce
    if (tid < PR * nseg) segs[(tid % PR) * nseg + tid / PR] = seg_sum(src0 + tid % PR, stride, Gb, nseg, tid / PR);
    __syncthreads();
    for (int j = tid; j < PR; j += nthr) {
      double s = 0.0;
      for (int q = 0; q < nseg; ++q) s += segs[j * nseg + q];
      r[j] = s;
    }
  }
  for (int j = tid; j < PR; j += nthr) raw[((size_t)b * KP + k) * PR + j] = r[j];
  for (int d = tid; d < D; d += blockDim.x) m[d] = (double)mu[((size_t)b * K + k) * D + d];
  __syncthreads();
  if (cov == TIED) return;
  const double n = r[0];
  const size_t bk = (size_t)b * K + k;
  if (tid == 0) nk[bk] = accumulate ? nk[bk] + n : n;
  for (int d = tid; d < D; d += blockDim.x) {
    const double v = r[2 + d];
    sx[bk * D + d] = accumulate ? sx[bk * D + d] + v : v;
  }
  if (cov == SPH) {
    if (tid == 0) {
      double dot = 0.0, mm = 0.0;
      for (int d = 0; d < D; ++d) {
        dot += m[d] * r[2 + d];
        mm += m[d] * m[d];
      }
      const double v = r[1] - 2.0 * dot + mm * n;
      sxx[bk] = accumulate ? sxx[bk] + v : v;
    }
  } else if (cov == DIAG) {
    for (int d = tid; d < D; d += blockDim.x) {
      const double v = r[2 + DP + d] - 2.0 * m[d] * r[2 + d] + m[d] * m[d] * n;
      sxx[bk * D + d] = accumulate ? sxx[bk * D + d] + v : v;
    }
  } else {  // FULL
    for (int i = tid; i < D * D; i += blockDim.x) {
      const int d = i / D, e = i % D;
      const int q = d <= e ? quad_index(d, e, DP) : quad_index(e, d, DP);
      const double v = r[2 + DP + q] - m[d] * r[2 + e] - r[2 + d] * m[e] + m[d] * m[e] * n;
      sxx[bk * D * D + i] = accumulate ? sxx[bk * D * D + i] + v : v;
    }
  }
  if (M.w) {
    // the M-step of this component, from the statistics this block just wrote
    // (the block's own global writes are visible to it after the barrier); it
    // reads and then replaces this component's mean only
    __syncthreads();
    mstep_component(cov, D, b, K, k, nk, sx, sxx, M.n_total, M.w, M.mu, M.cv, M.reg, M.in_flag, M.in_flag_stride,
                    M.comp_status, m, sm_S, sm_L);
    if (M.next.W) {
      // the next iteration's prologue of this component, from the parameters
      // just written (visible to the block after the barrier)
      __syncthreads();
      const PrologueOut& P = M.next;
      prologue_component(cov, D, K, P.KP, P.DP, P.F, P.KW, b, k, M.w, M.mu, M.cv, nullptr, P.W, P.prec,
                         P.prec_stride, P.c0, P.c, P.a, P.flag, P.sharp);
    }
  }
}

// Tied: sxx = sum_k sum_i r_ik (x_i - mu_k)(x_i - mu_k)^T from the raw sums.
// grid: B blocks.
__global__ void __launch_bounds__(256) centre_tied_kernel(int D, int K, int KP, int DP, int PR,
                                                          const double* __restrict__ raw,
                                                          const float* __restrict__ mu, double* nk, double* sx,
                                                          double* sxx, int accumulate) {
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int k = tid; k < K; k += blockDim.x) {
    const size_t bk = (size_t)b * K + k;
    const double v = raw[((size_t)b * KP + k) * PR];
    nk[bk] = accumulate ? nk[bk] + v : v;
  }
  for (int i = tid; i < K * D; i += blockDim.x) {
    const int k = i / D, d = i % D;
    const double v = raw[((size_t)b * KP + k) * PR + 2 + d];
    sx[(size_t)b * K * D + i] = accumulate ? sx[(size_t)b * K * D + i] + v : v;
  }
  for (int i = tid; i < D * D; i += blockDim.x) {
    const int d = i / D, e = i % D;
    const int q = d <= e ? quad_index(d, e, DP) : quad_index(e, d, DP);
    double s = 0.0;
    for (int k = 0; k < K; ++k) {
      const double* r = raw + ((size_t)b * KP + k) * PR;
      const double md = (double)mu[((size_t)b * K + k) * D + d];
      const double me = (double)mu[((size_t)b * K + k) * D + e];
      s += r[2 + DP + q] - md * r[2 + e] - r[2 + d] * me + md * me * r[0];
    }
    sxx[(size_t)b * D * D + i] = accumulate ? sxx[(size_t)b * D * D + i] + s : s;
  }
}

hipError_t launch_reduce_raw(const Plan& p, const double* part, const double* llpart, const float* mu,
                             double* raw, double* nk, double* sx, double* sxx, double* ll, double* mean_ll,
                             int accumulate, hipStream_t s, const MstepFuse* fuse) {
  // few components (fewer blocks than two per CU): enough threads that each
  // statistic is summed in segments of about 32 workgroup partials (the
  // loads in flight hide the memory latency), a multiple of the wave, 256 to
  // 1024; many components: 256, the blocks themselves fill the chip
  const int64_t want = (int64_t)p.PR * ((p.Gb + 31) / 32);
  const unsigned threads = p.B * p.K >= 512 ? 256u
                           : (unsigned)std::min<int64_t>(1024, std::max<int64_t>(256, (want + 63) / 64 * 64));
  const size_t lds = sizeof(double) * (size_t)(p.PR + p.D + threads);
  MstepFuse M{};
  if (fuse && p.cov != TIED && !accumulate) M = *fuse;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)(p.B * p.K + p.B)), dim3(threads), lds, s, p.cov, (int)p.D,
                     (int)p.K, p.KP, p.DP, p.PR, p.Gb, p.llG, p.N, part, llpart, mu, raw, nk, sx, sxx, ll, mean_ll,
                     accumulate, (int)p.B, M);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.cov != TIED) return e;
  hipLaunchKernelGGL(centre_tied_kernel, dim3((unsigned)p.B), dim3(256), 0, s, (int)p.D, (int)p.K, p.KP, p.DP,
                     p.PR, raw, mu, nk, sx, sxx, accumulate);
  return hipGetLastError();
}

// ------------------------------------------------------------------ M-step
// Flash-GMM Section 2, eqs. 1-3 (pi_k = N_k / n; mu'_k = sx_k / N_k; variance
// about the new mean, written through the centred statistics), diag / full
// forms as in "ML0094 GMM vs K-Means", Mathematical Formulation.  One
// component (b, k) by the threads of a block; sm_delta holds D doubles, sm_S
// and sm_L 16 x 16.
__device__ __forceinline__ void mstep_component(int cov, int D, int b, int K, int k, const double* __restrict__ nk,
                                const double* __restrict__ sx, const double* __restrict__ sxx, int64_t n_total,
                                float* w, float* mu, float* cv, double reg, const int32_t* in_flag,
                                int in_flag_stride, int32_t* comp_status, double* sm_delta, double* sm_S,
                                double* sm_L) {
  const int tid = threadIdx.x;
  const size_t bk = (size_t)b * K + k;
  const double n = nk[bk];
  const bool empty = !(n > 0.0);
  int32_t st = empty ? 1 : 0;
  if (in_flag) st |= in_flag[(size_t)b * in_flag_stride + k];
  if (tid == 0) w[bk] = (float)(n / (double)n_total);
  if (empty) {
    if (tid == 0 && comp_status) comp_status[bk] = st;
    return;  // mu_k and Sigma_k kept (uniform across the block)
  }
  for (int d = tid; d < D; d += blockDim.x) {
    const double m1 = sx[bk * D + d] / n;
    sm_delta[d] = m1 - (double)mu[bk * D + d];
  }
  __syncthreads();
  if (cov == SPH) {
    if (tid == 0) {
      double dd = 0.0;
      for (int d = 0; d < D; ++d) dd += sm_delta[d] * sm_delta[d];
      cv[bk] = (float)((sxx[bk] / n - dd) / (double)D + reg);
    }
  } else if (cov == DIAG) {
    for (int d = tid; d < D; d += blockDim.x)
      cv[bk * D + d] = (float)(sxx[bk * D + d] / n - sm_delta[d] * sm_delta[d] + reg);
  } else {  // FULL: check positive definiteness before committing
    for (int i = tid; i < D * D; i += blockDim.x) {
      const int d = i / D, e = i % D;
      sm_S[i] = sxx[bk * D * D + i] / n - sm_delta[d] * sm_delta[e] + (d == e ? reg : 0.0);
      sm_L[d * 16 + e] = sm_S[i];
    }
    if (!chol_block(D, sm_L, 16)) {
      if (tid == 0 && comp_status) comp_status[bk] = st | 2;
      return;  // previous mu_k and Sigma_k kept (uniform across the block)
    }
    for (int i = tid; i < D * D; i += blockDim.x) cv[bk * D * D + i] = (float)sm_S[i];
  }
  __syncthreads();
  for (int d = tid; d < D; d += blockDim.x) mu[bk * D + d] = (float)(sx[bk * D + d] / n);
  if (tid == 0 && comp_status) comp_status[bk] = st;
}

// grid: B*K blocks of 64 threads (spherical, diag, full).
__global__ void __launch_bounds__(64) mstep_kernel(int cov, int D, int K, const double* __restrict__ nk,
                                                   const double* __restrict__ sx, const double* __restrict__ sxx,
                                                   int64_t n_total, float* w, float* mu, float* cv, double reg,
                                                   const int32_t* in_flag, int in_flag_stride,
                                                   int32_t* comp_status) {
  __shared__ double sm_delta[128];
  __shared__ double sm_S[16 * 16], sm_L[16 * 16];
  mstep_component(cov, D, blockIdx.x / K, K, blockIdx.x % K, nk, sx, sxx, n_total, w, mu, cv, reg, in_flag,
                  in_flag_stride, comp_status, sm_delta, sm_S, sm_L);
}

// Tied: one block per problem.
__global__ void __launch_bounds__(256) mstep_tied_kernel(int D, int K, const double* __restrict__ nk,
                                                         const double* __restrict__ sx,
                                                         const double* __restrict__ sxx, int64_t n_total, float* w,
                                                         float* mu, float* cv, double reg, const int32_t* in_flag,
                                                         int in_flag_stride, int32_t* comp_status) {
  const int b = blockIdx.x, tid = threadIdx.x;
  __shared__ double sm_S[16 * 16], sm_L[16 * 16];
  extern __shared__ double sm_delta[];  // K*D
  for (int i = tid; i < K * D; i += blockDim.x) {
    const int k = i / D;
    const double n = nk[(size_t)b * K + k];
    sm_delta[i] = n > 0.0 ? sx[(size_t)b * K * D + i] / n - (double)mu[(size_t)b * K * D + i] : 0.0;
  }
  __syncthreads();
  for (int i = tid; i < D * D; i += blockDim.x) {
    const int d = i / D, e = i % D;
    double s = sxx[(size_t)b * D * D + i];
    for (int k = 0; k < K; ++k) s -= nk[(size_t)b * K + k] * sm_delta[k * D + d] * sm_delta[k * D + e];
    sm_S[i] = s / (double)n_total + (d == e ? reg : 0.0);
    sm_L[d * 16 + e] = sm_S[i];
  }
  const bool pd = chol_block(D, sm_L, 16);
  if (pd)
    for (int i = tid; i < D * D; i += blockDim.x) cv[(size_t)b * D * D + i] = (float)sm_S[i];
  for (int k = tid; k < K; k += blockDim.x) {
    const size_t bk = (size_t)b * K + k;
    const double n = nk[bk];
    w[bk] = (float)(n / (double)n_total);
    int32_t st = (n > 0.0 ? 0 : 1) | (pd ? 0 : 2);
    if (in_flag) st |= in_flag[(size_t)b * in_flag_stride + k];
    if (comp_status) comp_status[bk] = st;
  }
  __syncthreads();
  if (pd)
    for (int i = tid; i < K * D; i += blockDim.x) {
      const int k = i / D;
      const double n = nk[(size_t)b * K + k];
      if (n > 0.0) mu[(size_t)b * K * D + i] = (float)(sx[(size_t)b * K * D + i] / n);
    }
}

hipError_t launch_mstep_strided(int cov, int64_t B, int64_t D, int64_t K, const double* nk, const double* sx,
                                const double* sxx, int64_t n_total, float* w, float* mu, float* cv, double reg,
                                const int32_t* in_flag, int in_flag_stride, int32_t* comp_status, hipStream_t s) {
  if (cov == TIED) {
    hipLaunchKernelGGL(mstep_tied_kernel, dim3((unsigned)B), dim3(256), sizeof(double) * (size_t)(K * D), s,
                       (int)D, (int)K, nk, sx, sxx, n_total, w, mu, cv, reg, in_flag, in_flag_stride, comp_status);
  } else {
    hipLaunchKernelGGL(mstep_kernel, dim3((unsigned)(B * K)), dim3(64), 0, s, cov, (int)D, (int)K, nk, sx, sxx,
                       n_total, w, mu, cv, reg, in_flag, in_flag_stride, comp_status);
  }
  return hipGetLastError();
}

}  // namespace gmm
