// gmm_topk.hip -- approximate top-k EM: the statistics of a step in which
// each row keeps only its k best components.
//
// What it computes (the approx_top_k training mode of the GMMXX README: each
// E-step keeps the top k component log-scores of a row and normalises over
// that subset; Flash-GMM Section 2 for the statistics and the M-step):
//   r'_ik = r_ik / sum_{j in top_k(i)} r_ij   for k in top_k(i), else 0,
//   N_k = sum_i r'_ik,  S1_k = sum_i r'_ik x_i,
//   S2_k = sum_i r'_ik (x_i - mu_k)^2 (per dimension; summed for spherical),
//   LL = sum_i log sum_{j in top_k(i)} pi_j N(x_i | theta_j).
//
// The kept set: the k best components among those with r_ik >= 2^-20 (the
// best one always) -- smaller responsibilities are below the float32
// resolution of the row's sum, and every component above that floor lies in
// the band of scores the top-m pass rescores exactly.
//
// How: the library's top-m pass with m = k and threshold 2^-20 gives each row
// that set in float64 order (ties to the lower index) with r_ik and log p(x_i);
// topk_rows_kernel forms each row's 1 / sum r over the kept set
// and its log-sum-exp over it; the posting-list kernels group the entries by
// component in increasing row order; topk_stats_kernel sums each component's
// entries in that fixed order in float64, one workgroup per (problem,
// component); topk_ll_kernel adds the rows' log-sum-exps in row order.
#include "gmm_internal.h"

#include <hip/hip_runtime.h>

#include <math.h>

namespace gmm {

namespace {

// per row: rinv = 1 / sum of the kept responsibilities, llrow = log p(x) + log of that sum
__global__ void __launch_bounds__(256) topk_rows_kernel(int64_t rows, int m, const float* __restrict__ resp,
                                                        const float* __restrict__ logp, double* __restrict__ rinv,
                                                        double* __restrict__ llrow) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows) return;
  double s = 0.0;
  for (int j = 0; j < m; ++j) s += (double)resp[i * m + j];
  rinv[i] = s > 0.0 ? 1.0 / s : 0.0;
  llrow[i] = (double)logp[i] + log(s);
}

struct TopkStatsArgs {
  const void* x;
  int bf16;
  int64_t N, ld_x, stride_b;
  int K, D, L, m, cov;
  const float* mu;        // (B, K, D) the means entering the step
  const int64_t* offsets; // (B, K+1)
  const int32_t* rows;    // (B, N m)
  const float* lresp;     // (B, N m)
  const double* rinv;     // (B, N)
  double *nk, *sx, *sxx;  // (B, K), (B, K, D), (B, K) or (B, K, D)
};

__device__ __forceinline__ double topk_load_x(const TopkStatsArgs& A, const char* xb, int64_t r, int d) {
  if (A.bf16) {
    const unsigned short h = reinterpret_cast<const unsigned short*>(xb)[r * A.ld_x + d];
    return (double)__uint_as_float((unsigned)h << 16);
  }
  return (double)reinterpret_cast<const float*>(xb)[r * A.ld_x + d];
}

// one workgroup per (problem, component): 256 threads in 256 / L row slots
// of L lanes (lane d: dimension d); slot g takes entries g, g + 256/L, ... of
// the component's list; the slots' float64 sums meet in LDS in slot order
__global__ void __launch_bounds__(256) topk_stats_kernel(TopkStatsArgs A) {
  __shared__ double s1[256], s2[256], sw[256];
  const int b = blockIdx.x / A.K, k = blockIdx.x % A.K;
  const int t = threadIdx.x, L = A.L, G = 256 / L;
  const int g = t / L, d = t % L;
  const bool on = d < A.D;
  const int64_t o0 = A.offsets[(size_t)b * (A.K + 1) + k], o1 = A.offsets[(size_t)b * (A.K + 1) + k + 1];
  const size_t nm = (size_t)A.N * A.m;
  const int32_t* rb = A.rows + (size_t)b * nm;
  const float* lr = A.lresp + (size_t)b * nm;
  const double* ri = A.rinv + (size_t)b * A.N;
  const char* xb = static_cast<const char*>(A.x) + (size_t)b * A.stride_b * (A.bf16 ? 2 : 4);
  const double c = on ? (double)A.mu[((size_t)b * A.K + k) * A.D + d] : 0.0;
  double a1 = 0.0, a2 = 0.0, aw = 0.0;
  for (int64_t e = o0 + g; e < o1; e += G) {
    const int64_t r = rb[e];
    const double wgt = (double)lr[e] * ri[r];
    const double v = on ? topk_load_x(A, xb, r, d) : 0.0;
    a1 += wgt * v;
    a2 += wgt * (v - c) * (v - c);
    aw += wgt;
  }
  s1[t] = a1;
  s2[t] = a2;
  sw[t] = aw;
  __syncthreads();
  if (t < L) {
    double t1 = 0.0, t2 = 0.0, tw = 0.0;
    for (int h = 0; h < G; ++h) {
      t1 += s1[h * L + t];
      t2 += s2[h * L + t];
      tw += sw[h * L + t];
    }
    if (on) {
      A.sx[((size_t)b * A.K + k) * A.D + d] = t1;
      if (A.cov == DIAG) A.sxx[((size_t)b * A.K + k) * A.D + d] = t2;
    }
    s2[t] = on ? t2 : 0.0;  // slot 0's entries were read above by this same thread
    if (t == 0) A.nk[(size_t)b * A.K + k] = tw;  // every lane of a slot carries the same weights
  }
  if (A.cov == SPH) {
    __syncthreads();
    if (t == 0) {
      double q = 0.0;
      for (int h = 0; h < L; ++h) q += s2[h];
      A.sxx[(size_t)b * A.K + k] = q;
    }
  }
}

// per problem: LL = sum of the rows' log-sum-exps in row order (per thread,
// then thread order); mean_ll = LL / N
__global__ void __launch_bounds__(256) topk_ll_kernel(int64_t N, const double* __restrict__ llrow,
                                                      double* __restrict__ ll, double* __restrict__ mean_ll) {
  __shared__ double red[256];
  const int b = blockIdx.x, t = threadIdx.x;
  const int64_t per = (N + 255) / 256, i0 = (int64_t)t * per, i1 = i0 + per < N ? i0 + per : N;
  double s = 0.0;
  for (int64_t i = i0; i < i1; ++i) s += llrow[(size_t)b * N + i];
  red[t] = s;
  __syncthreads();
  if (t == 0) {
    double q = 0.0;
    for (int i = 0; i < 256; ++i) q += red[i];
    ll[b] = q;
    if (mean_ll) mean_ll[b] = N > 0 ? q / (double)N : 0.0;
  }
}

}  // namespace

hipError_t launch_topk_stats(const void* x, int bf16, int64_t B, int64_t N, int64_t ld_x, int64_t stride_b, int K,
                             int D, int m, int cov, const float* resp, const float* logp, const float* mu,
                             const int64_t* offsets, const int32_t* rows, const float* lresp, double* rinv,
                             double* llrow, double* nk, double* sx, double* sxx, double* ll, double* mean_ll,
                             hipStream_t s) {
  const int64_t nrows = B * N;
  if (nrows > 0) {
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, s, nrows, m, resp, logp,
                       rinv, llrow);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  TopkStatsArgs A;
  A.x = x;
  A.bf16 = bf16;
  A.N = N;
  A.ld_x = ld_x;
  A.stride_b = stride_b;
  A.K = K;
  A.D = D;
  A.L = 1;
  while (A.L < D) A.L <<= 1;
  A.m = m;
  A.cov = cov;
  A.mu = mu;
  A.offsets = offsets;
  A.rows = rows;
  A.lresp = lresp;
  A.rinv = rinv;
  A.nk = nk;
  A.sx = sx;
  A.sxx = sxx;
  hipLaunchKernelGGL(topk_stats_kernel, dim3((unsigned)(B * K)), dim3(256), 0, s, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_ll_kernel, dim3((unsigned)B), dim3(256), 0, s, N, llrow, ll, mean_ll);
  return hipGetLastError();
}

}  // namespace gmm
