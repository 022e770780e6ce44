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
// With k >= K every component is kept: the exact EM step.
//
// How: the library's top-m pass in its top-k mode gives each row its k best
// components in float64 order (ties to the lower index), their
// responsibilities normalised over those k, and the log-sum-exp over them;
// topk_rows_kernel forms each row's 1 / sum r' (1 up to float32 rounding) and
// its log-likelihood term (summed per block of 256 rows in a fixed tree); the
// posting-list kernels group the entries by component in increasing row order;
// topk_stats_kernel splits each component's list into S contiguous parts, one
// workgroup per (problem, component, part), and sums a part's entries in list
// order in float64; topk_reduce_kernel adds the parts in part order and
// topk_ll_kernel the row blocks in block order.  Every sum has a fixed order:
// the step is bitwise reproducible.
#include "gmm_internal.h"

#include <hip/hip_runtime.h>

#include <math.h>

namespace gmm {

namespace {

constexpr int kRowsPerBlock = 256;

// per row: rinv = 1 / sum of the kept responsibilities (they were normalised
// over the kept set; this removes their float32 rounding from the weights);
// per block of 256 rows of one problem: the sum of the rows' log-sum-exp over
// their kept components, in a fixed tree
__global__ void __launch_bounds__(kRowsPerBlock) topk_rows_kernel(TopkStepArgs A, int64_t nblk) {
  __shared__ double red[kRowsPerBlock];
  const int64_t b = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t = threadIdx.x;
  const int64_t i = blk * kRowsPerBlock + t;
  double v = 0.0;
  if (i < A.N) {
    const int64_t gi = b * A.N + i;
    double s = 0.0;
    for (int j = 0; j < A.m; ++j) s += (double)A.resp[gi * A.m + j];
    A.rinv[gi] = s > 0.0 ? 1.0 / s : 0.0;
    v = (double)A.logp[gi];
  }
  red[t] = v;
  __syncthreads();
  for (int w = kRowsPerBlock / 2; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) A.llpart[b * nblk + blk] = red[0];
}

__device__ __forceinline__ double topk_load_x(const TopkStepArgs& A, const char* xb, int64_t r, int d) {
  if (A.xtype != 0) {
    const unsigned short h = reinterpret_cast<const unsigned short*>(xb)[r * A.ld_x + d];
    return A.xtype == 1 ? (double)__uint_as_float((unsigned)h << 16) : (double)__builtin_bit_cast(_Float16, h);
  }
  return (double)reinterpret_cast<const float*>(xb)[r * A.ld_x + d];
}

// one workgroup per (problem, component, part): 256 threads in 256 / L row
// slots of L lanes (lane d: dimension d); slot g takes entries g, g + 256/L,
// ... of the part, four in flight; the slots' float64 sums meet in LDS in slot
// order.  Partial layout per (b, k, s): [N_k, S1 (D), S2 per dimension (D)].
__global__ void __launch_bounds__(256) topk_stats_kernel(TopkStepArgs A, int L) {
  constexpr int U = 4;
  __shared__ double s1[256], s2[256], sw[256];
  const int S = A.S;
  const int s = blockIdx.x % S;
  const int k = (blockIdx.x / S) % A.K;
  const int64_t b = blockIdx.x / ((int64_t)S * A.K);
  const int t = threadIdx.x, G = 256 / L;
  const int g = t / L, d = t % L;
  const bool on = d < A.D;
  const int64_t o0 = A.offsets[b * (A.K + 1) + k], o1 = A.offsets[b * (A.K + 1) + k + 1];
  const int64_t len = o1 - o0;
  const int64_t p0 = o0 + len * s / S, p1 = o0 + len * (s + 1) / S;
  const size_t nm = (size_t)A.N * A.m;
  const int32_t* rb = A.rows + b * nm;
  const float* lr = A.lresp + b * nm;
  const double* ri = A.rinv + b * A.N;
  const char* xb = static_cast<const char*>(A.x) + b * A.stride_b * (A.xtype != 0 ? 2 : 4);
  const double c = on ? (double)A.mu[(b * A.K + k) * A.D + d] : 0.0;
  double a1 = 0.0, a2 = 0.0, aw = 0.0;
  for (int64_t e = p0 + g; e < p1; e += (int64_t)U * G) {
    int64_t r[U];
    float lw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t ee = e + (int64_t)u * G;
      r[u] = ee < p1 ? (int64_t)rb[ee] : -1;
      lw[u] = ee < p1 ? lr[ee] : 0.f;
    }
    double wgt[U], v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      wgt[u] = r[u] >= 0 ? (double)lw[u] * ri[r[u]] : 0.0;
      v[u] = (on && r[u] >= 0) ? topk_load_x(A, xb, r[u], d) : 0.0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a1 += wgt[u] * v[u];
      a2 += wgt[u] * (v[u] - c) * (v[u] - c);
      aw += wgt[u];
    }
  }
  s1[t] = a1;
  s2[t] = a2;
  sw[t] = aw;
  __syncthreads();
  if (t < L && on) {
    double t1 = 0.0, t2 = 0.0, tw = 0.0;
    for (int h = 0; h < G; ++h) {
      t1 += s1[h * L + t];
      t2 += s2[h * L + t];
      tw += sw[h * L + t];
    }
    double* part = A.part + ((b * A.K + k) * S + s) * (1 + 2 * (int64_t)A.D);
    part[1 + d] = t1;
    part[1 + A.D + d] = t2;
    if (t == 0) part[0] = tw;  // every lane of a slot carries the same weights
  }
}

// one workgroup per (problem, component): the parts added in part order;
// spherical S2 then summed over the dimensions in order
__global__ void __launch_bounds__(256) topk_reduce_kernel(TopkStepArgs A) {
  __shared__ double q2[256];
  const int64_t bk = blockIdx.x;
  const int t = threadIdx.x, S = A.S, D = A.D;
  const int64_t PR = 1 + 2 * (int64_t)D;
  const double* part = A.part + bk * S * PR;
  for (int cidx = t; cidx < PR; cidx += 256) {
    double v = 0.0;
    for (int s = 0; s < S; ++s) v += part[s * PR + cidx];
    if (cidx == 0) A.nk[bk] = v;
    else if (cidx <= D) A.sx[bk * D + cidx - 1] = v;
    else if (A.cov == DIAG) A.sxx[bk * D + cidx - 1 - D] = v;
    else q2[cidx - 1 - D] = v;  // D <= 256
  }
  if (A.cov == SPH) {
    __syncthreads();
    if (t == 0) {
      double q = 0.0;
      for (int d = 0; d < D; ++d) q += q2[d];
      A.sxx[bk] = q;
    }
  }
}

// per problem: LL = sum of the block sums (per thread in block order, then
// thread order); mean_ll = LL / N
__global__ void __launch_bounds__(256) topk_ll_kernel(TopkStepArgs A, int64_t nblk) {
  __shared__ double red[256];
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x;
  double s = 0.0;
  for (int64_t i = t; i < nblk; i += 256) s += A.llpart[b * nblk + i];
  red[t] = s;
  __syncthreads();
  if (t == 0) {
    double q = 0.0;
    for (int i = 0; i < 256; ++i) q += red[i];
    A.ll[b] = q;
    if (A.mean_ll) A.mean_ll[b] = A.N > 0 ? q / (double)A.N : 0.0;
  }
}

}  // namespace

hipError_t launch_topk_stats(const TopkStepArgs& A, hipStream_t s) {
  if (A.D > 256 || A.S < 1) return hipErrorInvalidValue;
  const int64_t nblk = (A.N + kRowsPerBlock - 1) / kRowsPerBlock;
  if (A.B * nblk > 0) {
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)(A.B * nblk)), dim3(kRowsPerBlock), 0, s, A, nblk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  int L = 1;
  while (L < A.D) L <<= 1;
  hipLaunchKernelGGL(topk_stats_kernel, dim3((unsigned)(A.B * A.K * A.S)), dim3(256), 0, s, A, L);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_reduce_kernel, dim3((unsigned)(A.B * A.K)), dim3(256), 0, s, A);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_ll_kernel, dim3((unsigned)A.B), dim3(256), 0, s, A, nblk);
  return hipGetLastError();
}

}  // namespace gmm
