// gmm_fisher.hip -- Fisher vectors of sets of rows under one diagonal GMM.
//
// What it computes (Flash-GMM's closing discussion: the fused log-sum-exp
// followed by responsibility-weighted statistics is also the pattern of Fisher
// Vector encoding, Perronnin et al. 2010; the improved form of that work):
// for each set b of N rows, with r the responsibilities under the model
// (w, mu, sigma^2),
//   G_mu[k, d]  = (sum_i r_ik x_id - N_k mu_kd) / (sigma_kd N sqrt(w_k))
//   G_sig[k, d] = (sum_i r_ik (x_id - mu_kd)^2 / sigma_kd^2 - N_k) / (N sqrt(2 w_k))
// -- the gradients of the mean log-likelihood with respect to mu and sigma,
// scaled by the diagonal Fisher information -- laid out [G_mu, G_sig],
// k-major, then optionally a signed square root and L2 normalisation.
//
// How: the sums are exactly the per-problem statistics of the batched fused
// E-step (N_k, sum r x, and sum r (x - mu)^2 about the model's means), so the
// sets run as B problems of one batched E-step with the model replicated per
// problem; fisher_kernel then forms each set's vector from its float64
// statistics, one workgroup per set, with the L2 norm summed in a fixed order.
#include "gmm_internal.h"

#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>

namespace gmm {

namespace {

// the model (w (K), mu (K, D), var (K, D)) copied for each of B problems
__global__ void __launch_bounds__(256) fisher_replicate_kernel(int64_t B, int K, int D, const float* __restrict__ w,
                                                              const float* __restrict__ mu,
                                                              const float* __restrict__ var, float* __restrict__ wr,
                                                              float* __restrict__ mur, float* __restrict__ varr) {
  const int64_t KD = (int64_t)K * D, per = K + 2 * KD;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < B * per; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = i / per, j = i % per;
    if (j < K) wr[b * K + j] = w[j];
    else if (j < K + KD) mur[b * KD + (j - K)] = mu[j - K];
    else varr[b * KD + (j - K - KD)] = var[j - K - KD];
  }
}

// one workgroup (256 threads) per set: the 2 K D values, then the norm
__global__ void __launch_bounds__(256) fisher_kernel(int K, int D, int64_t N, uint32_t flags,
                                                     const float* __restrict__ w, const float* __restrict__ mu,
                                                     const float* __restrict__ var, const double* __restrict__ nk,
                                                     const double* __restrict__ sx, const double* __restrict__ sxx,
                                                     float* __restrict__ fv) {
  __shared__ double red[256];
  const int b = blockIdx.x, t = threadIdx.x;
  const int64_t KD = (int64_t)K * D;
  float* out = fv + (size_t)b * 2 * KD;
  const double* nkb = nk + (size_t)b * K;
  const double* sxb = sx + (size_t)b * KD;
  const double* sxxb = sxx + (size_t)b * KD;
  const bool power = (flags & 1u) != 0, l2 = (flags & 2u) != 0;
  double ss = 0.0;
  for (int64_t i = t; i < KD; i += blockDim.x) {
    const int k = (int)(i / D);
    const double wk = (double)w[k], m = (double)mu[i], v = (double)var[i];
    double gm = 0.0, gs = 0.0;
    if (N > 0 && wk > 0.0 && v > 0.0) {
      const double n = (double)N;
      gm = (sxb[i] - nkb[k] * m) / (sqrt(v) * n * sqrt(wk));
      gs = (sxxb[i] / v - nkb[k]) / (n * sqrt(2.0 * wk));
    }
    if (power) {
      gm = copysign(sqrt(fabs(gm)), gm);
      gs = copysign(sqrt(fabs(gs)), gs);
    }
    const float fm = (float)gm, fs = (float)gs;
    out[i] = fm;
    out[KD + i] = fs;
    ss += (double)fm * fm + (double)fs * fs;
  }
  if (!l2) return;
  red[t] = ss;
  __syncthreads();
  if (t == 0) {
    double s = 0.0;
    for (int i = 0; i < (int)blockDim.x; ++i) s += red[i];
    red[0] = s > 0.0 ? 1.0 / sqrt(s) : 0.0;
  }
  __syncthreads();
  const double scale = red[0];
  if (scale == 0.0) return;
  // each thread rescales the values it wrote
  for (int64_t i = t; i < KD; i += blockDim.x) {
    out[i] = (float)((double)out[i] * scale);
    out[KD + i] = (float)((double)out[KD + i] * scale);
  }
}

}  // namespace

hipError_t launch_fisher_replicate(int64_t B, int K, int D, const float* w, const float* mu, const float* var,
                                   float* wr, float* mur, float* varr, hipStream_t s) {
  const int64_t total = B * ((int64_t)K + 2 * (int64_t)K * D);
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(fisher_replicate_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s, B, K, D,
                     w, mu, var, wr, mur, varr);
  return hipGetLastError();
}

hipError_t launch_fisher(int64_t B, int K, int D, int64_t N, uint32_t flags, const float* w, const float* mu,
                         const float* var, const double* nk, const double* sx, const double* sxx, float* fv,
                         hipStream_t s) {
  hipLaunchKernelGGL(fisher_kernel, dim3((unsigned)B), dim3(256), 0, s, K, D, N, flags, w, mu, var, nk, sx, sxx, fv);
  return hipGetLastError();
}

}  // namespace gmm
