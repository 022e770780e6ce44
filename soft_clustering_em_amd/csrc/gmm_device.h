// gmm_device.h -- device helpers shared by the fused E-step kernel, the
// top-m kernels and the large-K kernels: 16-lane DPP reductions, wave-wide
// reductions and ranking order, the product-feature index map, and the
// float64 log-score by direct differences.
#pragma once

#include "gmm_internal.h"

#include <math.h>

namespace gmm {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

// Element idx of rows stored as xtype (a gmm_dtype: 0 float32, 1 bfloat16,
// 2 IEEE half), decoded exactly to float32.
__device__ __forceinline__ float x_value(const void* x, int xtype, int64_t idx) {
  if (xtype == 0) return reinterpret_cast<const float*>(x)[idx];
  const unsigned short h = reinterpret_cast<const unsigned short*>(x)[idx];
  if (xtype == 1) return __uint_as_float((unsigned)h << 16);
  return (float)__builtin_bit_cast(_Float16, h);
}

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

// all-reduce across the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32,
// l ^ 48) with the gfx950 row swaps: v_permlane16_swap exchanges rows 1 and 0
// and rows 3 and 2 between its two operands, v_permlane32_swap rows 2-3 and
// 0-1; given the same value twice, the two results hold the two halves.
__device__ __forceinline__ float rows4_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t rows4_or(uint32_t v) {
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = a[0] | a[1];
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return b[0] | b[1];
}

// all-reduce across the two 32-lane halves of a wave (lanes l, l ^ 32): given
// the same value twice, v_permlane32_swap returns the two halves
__device__ __forceinline__ float halves_max(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ uint32_t halves_or(uint32_t v) {
  auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return b[0] | b[1];
}
__device__ __forceinline__ double halves_sum_f64(double v) {
  const unsigned long long w = (unsigned long long)__double_as_longlong(v);
  auto lo = __builtin_amdgcn_permlane32_swap((unsigned)w, (unsigned)w, false, false);
  auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(w >> 32), (unsigned)(w >> 32), false, false);
  return __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0])) +
         __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
}

__device__ __forceinline__ double rows4_sum_f64(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  auto lo = __builtin_amdgcn_permlane16_swap((unsigned)u, (unsigned)u, false, false);
  auto hi = __builtin_amdgcn_permlane16_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
  v = __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0])) +
      __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
  const unsigned long long w = (unsigned long long)__double_as_longlong(v);
  auto lo2 = __builtin_amdgcn_permlane32_swap((unsigned)w, (unsigned)w, false, false);
  auto hi2 = __builtin_amdgcn_permlane32_swap((unsigned)(w >> 32), (unsigned)(w >> 32), false, false);
  return __longlong_as_double((long long)(((unsigned long long)hi2[0] << 32) | lo2[0])) +
         __longlong_as_double((long long)(((unsigned long long)hi2[1] << 32) | lo2[1]));
}

// 16-lane all-reduce of a double (the two halves moved by the DPP patterns of
// row16_sum)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffLL), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
__device__ __forceinline__ double row16_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return v;
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// product feature f >= DP of the quadratic feature map: (d, e) packed as d << 16 | e
template <int DP>
__device__ __forceinline__ int quad_pair(int q) {
  int d = 0, base = 0;
  while (q >= base + (DP - d)) { base += DP - d; ++d; }
  return (d << 16) | (d + (q - base));
}

// log2 of pi_k N(x | mu_k, Sigma_k) for one row x (float32 values in LDS,
// zero past D), by direct differences in float64:
// c0_k - 1/2 log2(e) (x - mu)^T P (x - mu).  prec holds 1/sigma^2
// (spherical: one value; diag: D values) or, for full/tied, the
// lower-triangular L^{-1} of Sigma = L L^T as DP x DP, zero past D.  UNROLL:
// that product runs fully unrolled over DP (the padding contributes 0), so
// its loads are issued together rather than one per loop trip -- for callers
// with the registers to spare.  kpt: components per problem in prec and c0
// when that differs from A.KP (components in blocks); 0 takes A.KP.
template <int COV, int DP, bool UNROLL = true, class Args>
__device__ __forceinline__ double exact_score(const Args& A, int b, int k, int D, const float* x, int kpt = 0) {
  constexpr double kLog2e = 1.4426950408889634074;
  const size_t KPx = kpt ? (size_t)kpt : (size_t)A.KP;  // components per problem in prec and c0
  const float* mu = A.mu + ((size_t)b * A.K + k) * D;
  const double* P = A.prec + ((size_t)b * KPx + k) * (size_t)A.prec_stride;
  double q = 0.0;
  // spherical and diagonal: eight trips per unrolled body so their loads are
  // in flight together; the sum keeps its order
  if constexpr (COV == SPH) {
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
      const double t = (double)x[d] - (double)mu[d];
      q += t * t;
    }
    q *= P[0];
  } else if constexpr (COV == DIAG) {
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
      const double t = (double)x[d] - (double)mu[d];
      q += P[d] * t * t;
    }
  } else if constexpr (!UNROLL) {
    for (int i = 0; i < D; ++i) {
      double z = 0.0;
      for (int j = 0; j <= i; ++j) z = fma(P[i * DP + j], (double)x[j] - (double)mu[j], z);
      q = fma(z, z, q);
    }
  } else {
    double t[DP];
#pragma unroll
    for (int j = 0; j < DP; ++j) t[j] = j < D ? (double)x[j] - (double)mu[j < D ? j : 0] : 0.0;
#pragma unroll
    for (int i = 0; i < DP; ++i) {
      double z = 0.0;
#pragma unroll
      for (int j = 0; j <= i; ++j) z = fma(P[i * DP + j], t[j], z);
      q = fma(z, z, q);
    }
  }
  return A.c0[(size_t)b * KPx + k] - 0.5 * kLog2e * q;
}

// ranking order of (log-score, component): higher score first, lower index on ties
__device__ __forceinline__ bool before(double la, int ka, double lb, int kb) {
  return la > lb || (la == lb && ka < kb);
}

// wave-wide (64-lane) reductions through ds_bpermute, fixed butterfly order
__device__ __forceinline__ double wave_max(double v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}
__device__ __forceinline__ void wave_best(double& l, int& k) {
  for (int off = 32; off >= 1; off >>= 1) {
    const double l2 = __shfl_xor(l, off);
    const int k2 = __shfl_xor(k, off);
    if (before(l2, k2, l, k)) { l = l2; k = k2; }
  }
}

}  // namespace gmm
