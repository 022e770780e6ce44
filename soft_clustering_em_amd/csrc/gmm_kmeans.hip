// gmm_kmeans.hip -- one k-means (Lloyd) iteration: the hard-assignment limit
// of EM.
//
// What it computes ("ML0094 GMM vs K-Means": k-means gives each point to the
// centroid at the smallest distance, and is the limit of a GMM whose
// components share one spherical variance that goes to zero, where the
// posterior becomes an argmax; with 0/1 responsibilities the mean update is
// the mean of the cluster's points.  Flash-GMM, Section 4: k-means is the
// usual IVF coarse quantizer the GMM is a drop-in for):
//   labels_i  = argmin_k |x_i - c_k|^2  (ties to the lower k),
//   c'_k      = mean of the rows labelled k (a cluster with none keeps c_k),
//   inertia   = sum_i min_k |x_i - c_k|^2.
//
// How: with equal weights and one shared spherical variance, the component of
// largest responsibility is the nearest centroid for any value of that
// variance, so the labels come from the library's exact top-1 assignment
// (float32 / bf16 MFMA scores, a candidate band, float64 rescoring, ties to
// the lower index).  The variance only sets how wide the candidate band is in
// distance units; kmeans_params_kernel takes 2^-10 max_k |c_k|^2: then
// lambda (|c_k|^2 + D sigma^2) <= 2^10 + D, below the large-K path's sharp
// threshold for every D it takes, so no component needs the direct-difference
// rescoring there, and the candidate band is a few percent of the centroid
// scale.  The labels then go through the posting-list kernels (rows of each
// cluster in increasing order), and kmeans_update_kernel sums each cluster's
// rows in that fixed order in float64: no atomics, the same bits every run.
#include "gmm_internal.h"

#include <hip/hip_runtime.h>

#include <math.h>

namespace gmm {

namespace {

constexpr int kVarShift = 10;  // shared variance = 2^-kVarShift max_k |c_k|^2
static_assert((1 << kVarShift) + 128 < kLargeKSharp, "k-means components must stay below the sharp threshold");

// Per problem: w_k = 1/K and the shared variance 2^-kVarShift max(max_k |c_k|^2, 1e-20).
__global__ void __launch_bounds__(256) kmeans_params_kernel(int K, int D, const float* __restrict__ C,
                                                            float* __restrict__ w, float* __restrict__ cv) {
  __shared__ double red[256];
  const int b = blockIdx.x, t = threadIdx.x;
  const float* cb = C + (size_t)b * K * D;
  double mx = 0.0;
  for (int k = t; k < K; k += 256) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) {
      const double v = cb[(size_t)k * D + d];
      s += v * v;
    }
    mx = fmax(mx, s);
  }
  red[t] = mx;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (t < h) red[t] = fmax(red[t], red[t + h]);
    __syncthreads();
  }
  const float s2 = (float)ldexp(fmax(red[0], 1e-20), -kVarShift);
  const float wk = 1.0f / (float)K;
  for (int k = t; k < K; k += 256) {
    w[(size_t)b * K + k] = wk;
    cv[(size_t)b * K + k] = s2;
  }
}

struct UpdateArgs {
  const void* x;
  int xtype;                 // gmm_dtype of the rows
  int64_t N, ld_x, stride_b;
  int K, D, L;               // L: lanes per row (a power of two >= D, <= 256)
  const int64_t* offsets;    // (B, K+1)
  const int32_t* rows;       // (B, N)
  float* C;                  // (B, K, D) in/out
  int64_t* counts;           // (B, K) or null
  double* ip;                // (B, K): the cluster's share of the inertia
};

__device__ __forceinline__ double load_x(const UpdateArgs& A, const char* xb, int64_t r, int d) {
  if (A.xtype != 0) {
    const unsigned short h = reinterpret_cast<const unsigned short*>(xb)[r * A.ld_x + d];
    return A.xtype == 1 ? (double)__uint_as_float((unsigned)h << 16) : (double)__builtin_bit_cast(_Float16, h);
  }
  return (double)reinterpret_cast<const float*>(xb)[r * A.ld_x + d];
}

// One workgroup per (problem, cluster): 256 threads in 256 / L row slots of L
// lanes, lane d holding dimension d.  Slot g takes the cluster's rows
// g, g + 256/L, ... of its list; the slots' float64 sums then meet in LDS in
// slot order.
__global__ void __launch_bounds__(256) kmeans_update_kernel(UpdateArgs A) {
  __shared__ double ps[256], pq[256];
  const int b = blockIdx.x / A.K, k = blockIdx.x % A.K;
  const int t = threadIdx.x, L = A.L, G = 256 / L;
  const int g = t / L, d = t % L;
  const bool on = d < A.D;
  const int64_t o0 = A.offsets[(size_t)b * (A.K + 1) + k], o1 = A.offsets[(size_t)b * (A.K + 1) + k + 1];
  const int32_t* rb = A.rows + (size_t)b * A.N;
  const char* xb = static_cast<const char*>(A.x) + (size_t)b * A.stride_b * (A.xtype != 0 ? 2 : 4);
  float* cb = A.C + ((size_t)b * A.K + k) * A.D;
  const double c = on ? (double)cb[d] : 0.0;
  double s = 0.0, q = 0.0;
  int64_t j = o0 + g;
  constexpr int U = 4;  // independent row loads in flight per thread
  for (; j + (int64_t)(U - 1) * G < o1; j += (int64_t)U * G) {
    double v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = on ? load_x(A, xb, rb[j + (int64_t)u * G], d) : 0.0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s += v[u];
      q += (v[u] - c) * (v[u] - c);
    }
  }
  for (; j < o1; j += G) {
    const double v = on ? load_x(A, xb, rb[j], d) : 0.0;
    s += v;
    q += (v - c) * (v - c);
  }
  ps[t] = s;
  pq[t] = q;
  __syncthreads();
  const int64_t n = o1 - o0;
  if (t < L) {
    double ts = 0.0, tq = 0.0;
    for (int h = 0; h < G; ++h) {
      ts += ps[h * L + t];
      tq += pq[h * L + t];
    }
    if (on && n > 0) cb[d] = (float)(ts / (double)n);
    pq[t] = tq;  // slot 0's entries were read above by this same thread
  }
  __syncthreads();
  if (t == 0) {
    double tq = 0.0;
    for (int h = 0; h < L; ++h) tq += pq[h];
    A.ip[(size_t)b * A.K + k] = tq;
    if (A.counts) A.counts[(size_t)b * A.K + k] = n;
  }
}

// inertia[b] = sum_k ip[b][k] in component order
__global__ void __launch_bounds__(64) kmeans_inertia_kernel(int B, int K, const double* __restrict__ ip,
                                                           double* __restrict__ inertia) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= B) return;
  double s = 0.0;
  for (int k = 0; k < K; ++k) s += ip[(size_t)b * K + k];
  inertia[b] = s;
}

}  // namespace

hipError_t launch_kmeans_params(int64_t B, int K, int D, const float* C, float* w, float* cv, hipStream_t s) {
  hipLaunchKernelGGL(kmeans_params_kernel, dim3((unsigned)B), dim3(256), 0, s, K, D, C, w, cv);
  return hipGetLastError();
}

hipError_t launch_kmeans_update(const void* x, int xtype, int64_t B, int64_t N, int64_t ld_x, int64_t stride_b, int K,
                                int D, const int64_t* offsets, const int32_t* rows, float* C, int64_t* counts,
                                double* ip, double* inertia, hipStream_t s) {
  UpdateArgs A;
  A.x = x;
  A.xtype = xtype;
  A.N = N;
  A.ld_x = ld_x;
  A.stride_b = stride_b;
  A.K = K;
  A.D = D;
  A.L = 1;
  while (A.L < D) A.L <<= 1;
  A.offsets = offsets;
  A.rows = rows;
  A.C = C;
  A.counts = counts;
  A.ip = ip;
  hipLaunchKernelGGL(kmeans_update_kernel, dim3((unsigned)(B * K)), dim3(256), 0, s, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (inertia) {
    hipLaunchKernelGGL(kmeans_inertia_kernel, dim3((unsigned)((B + 63) / 64)), dim3(64), 0, s, (int)B, K, ip, inertia);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace gmm
