// gmm_kde.hip -- Gaussian kernel density estimate at query rows.
//
// What it computes (Flash-GMM's closing discussion names kernel density
// estimation beside Fisher vectors as the same fused log-sum-exp pattern):
// with M reference rows x_j and an isotropic bandwidth h, the estimate is the
// equal-weight mixture of spherical Gaussians N(x_j, h^2 I), so for a query y
//   log p(y) = LSE_j(-|y - x_j|^2 / (2 h^2)) - log M - (D / 2) log(2 pi h^2).
//
// How it is laid out on gfx950 (CDNA4): the reference set is a K = M mixture
// far wider than one workgroup's registers, so it streams past the queries as
// in a flash-attention forward pass:
//   * the references are centred at their mean (a translation leaves every
//     distance unchanged and keeps the expanded form below well conditioned)
//     and stored zero-padded to DP features and whole 64-row tiles, with their
//     scaled squared norms, by three small kernels;
//   * a workgroup holds 64 query rows in registers (four waves, one 16-row
//     block each, at most 128 registers so that four waves share a SIMD) and
//     walks every reference tile, double-buffered in LDS with one barrier per
//     tile;
//   * the cross terms y . x run on v_mfma_f32_16x16x4_f32; for the MFMA step
//     s, lane group g (lane / 16) supplies feature g DP/4 + s of its query row
//     and of its reference column, so a lane's features are contiguous and its
//     reference operands come from LDS as 16-byte reads;
//   * the log-scores, in log2 units, are l = -lam |y|^2 - lam |x|^2 + 2 lam y.x
//     with lam = log2(e) / (2 h^2); the row's own -lam |y|^2 is the same for
//     every reference, so the tiles carry l' = 2 lam y.x - lam |x|^2 and the
//     row term is added once, in float64, at the end;
//   * per row a reference maximum and per lane a running sum of
//     2^(l' - reference), combined across the row's 16 lanes at the end; the
//     reference moves (16-lane DPP maximum, rescaled sums) only when some score
//     of the wave's rows passes it by more than 8 log2 units, which after the
//     first tiles is rare;
//   * the terms that decide the sum are rescored exactly, as the fused E-step
//     rescores its sharp components: every reference whose score comes within
//     30 (log2 units) of the row's reference maximum is listed in LDS (up to 8
//     per row; when the reference moves, entries that fell below the band are
//     dropped); at the end each listed term's float32 value is taken out of the
//     sum and its float64 value from direct differences of the caller's rows
//     put in, the list read in increasing reference order.  A row with more
//     than 8 references within the band of its final maximum keeps its float32
//     sum (a broad bandwidth, where the float32 terms are accurate).
// Each query's sums run in one fixed order: the result is bitwise reproducible.
//
// Rounding: the float32 contraction's error on y.x is at most about
// DP eps |y - c| |x - c| (c the reference mean), so a float32 log-score is
// within about lam eps (2 DP |y - c| |x - c| + |y - c|^2 + |x - c|^2) log2
// units.  With the listed terms exact, what is left is that error on terms
// below 2^-30 of the largest, and the rounding of the sums.
#include "gmm_device.h"
#include "gmm_internal.h"

#include <math.h>

namespace gmm {

namespace {

constexpr int kKdeTile = 64;   // reference rows per LDS tile
constexpr int kKdeRB = 1;      // 16-row query blocks per wave
constexpr int kKdeWaves = 4;   // waves per workgroup, sharing each reference tile
constexpr int kKdeThreads = 64 * kKdeWaves;
constexpr int kKdeQ = kKdeWaves * 16 * kKdeRB;  // query rows per workgroup
constexpr float kKdeBand = 30.f;        // log2 units below the running maximum that are rescored
constexpr int kKdeCap = 8;              // rescored references per row
constexpr float kKdeSlack = 8.f;        // log2 units a score may pass a row's reference maximum before it moves

// c_d = mean of the references' feature d, summed in float64 in a fixed order
__global__ void __launch_bounds__(256) kde_centre_kernel(const float* __restrict__ x, int64_t M, int64_t ld, int D,
                                                         float* __restrict__ cen) {
  __shared__ double red[256];
  const int d = blockIdx.x, t = threadIdx.x;
  double s = 0.0;
  if (d < D)
    for (int64_t j = t; j < M; j += 256) s += (double)x[j * ld + d];
  red[t] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) cen[d] = d < D ? (float)(red[0] / (double)M) : 0.f;
}

// centred references, (Mp, DP) float32, zero past M rows and D features
__global__ void __launch_bounds__(256) kde_refs_kernel(const float* __restrict__ x, int64_t M, int64_t Mp, int64_t ld,
                                                       int D, int DP, const float* __restrict__ cen,
                                                       float* __restrict__ xc) {
  const int64_t n = Mp * DP;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t j = i / DP;
    const int d = (int)(i % DP);
    xc[i] = (j < M && d < D) ? x[j * ld + d] - cen[d] : 0.f;
  }
}

// bx_j = -lam |x_j - c|^2 from the stored centred row (float64 sum); -inf past M
__global__ void __launch_bounds__(256) kde_norms_kernel(const float* __restrict__ xc, int64_t M, int64_t Mp, int DP,
                                                        double lam, float* __restrict__ bx) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= Mp) return;
  if (j >= M) {
    bx[j] = -INFINITY;
    return;
  }
  double s = 0.0;
  for (int d = 0; d < DP; ++d) {
    const double v = (double)xc[j * DP + d];
    s += v * v;
  }
  bx[j] = (float)(-lam * s);
}

template <int DP>
__global__ void __launch_bounds__(kKdeThreads, DP >= 128 ? 2 : 4) kde_kernel(KdeArgs A) {
  constexpr int KS = DP / 4;    // MFMA steps; lane group g holds features g KS .. g KS + KS - 1
  constexpr int RS = DP + 4;    // LDS row stride in floats (16-byte aligned rows)
  constexpr int RB = kKdeRB;
  constexpr int NT = kKdeTile / 16;
  constexpr int NP = kKdeTile * DP / 4;                        // 16-byte pieces of a tile
  constexpr int PER = (NP + kKdeThreads - 1) / kKdeThreads;    // per thread
  constexpr double LN2 = 0.69314718055994530942;
  static_assert(KS % 4 == 0 && kKdeTile <= kKdeThreads, "tile shape");
  __shared__ float xs[2][kKdeTile * RS];
  __shared__ float bs[2][kKdeTile];
  __shared__ double ays[kKdeQ];
  __shared__ int cj[kKdeQ * kKdeCap];    // listed references per row
  __shared__ float cl[kKdeQ * kKdeCap];  // their float32 scores
  __shared__ int cn[kKdeQ];              // references that qualified (may exceed kKdeCap)

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t nqb = (A.N + kKdeQ - 1) / kKdeQ;
  const int64_t b = blockIdx.x / nqb, q0 = (blockIdx.x % nqb) * kKdeQ;
  const float* yb = A.y + b * A.stride_b;

  // ---- this wave's query rows, centred, as MFMA A operands; -lam |y - c|^2 per row
  float a[RB][KS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t row = q0 + 16 * RB * wv + 16 * rb + c16;
    const bool ok = row < A.N;
    double ss = 0.0;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int d = g * KS + s;
      const float v = (ok && d < A.D) ? yb[row * A.ld + d] - A.cen[d] : 0.f;
      a[rb][s] = v;
      ss += (double)v * (double)v;
    }
    // the row's four feature quarters sit in lanes c16, c16 + 16, + 32, + 48
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (g == 0) ays[16 * RB * wv + 16 * rb + c16] = -A.lam * ss;
  }

  // ---- reference tiles: fetched into registers one tile ahead, stored to the idle LDS buffer
  floatx4 pf[PER];
  float pb = 0.f;
  auto fetch = [&](int64_t t) {
    const floatx4* src = reinterpret_cast<const floatx4*>(A.xc + t * kKdeTile * DP);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (NP % kKdeThreads == 0 || threadIdx.x + kKdeThreads * i < NP) pf[i] = src[threadIdx.x + kKdeThreads * i];
    if (threadIdx.x < kKdeTile) pb = A.bx[t * kKdeTile + threadIdx.x];
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = (threadIdx.x + kKdeThreads * i) * 4;
      if (NP % kKdeThreads == 0 || e < 4 * NP) *reinterpret_cast<floatx4*>(&xs[buf][(e / DP) * RS + e % DP]) = pf[i];
    }
    if (threadIdx.x < kKdeTile) bs[buf][threadIdx.x] = pb;
  };
  for (int i = threadIdx.x; i < kKdeQ; i += kKdeThreads) cn[i] = 0;
  fetch(0);
  stash(0);
  __syncthreads();  // tile 0, the row norms and the list counts visible

  // epilogue layout of a 16x16 block: lane holds rows 4 g + v (v = 0..3) of
  // column c16.  The scores below leave out the row's own -lam |y - c|^2 (added
  // once at the end in float64); mx is the row's reference maximum, within
  // kKdeSlack below the largest score seen; lost: the largest score this lane
  // could not list (the row's list was full)
  float mx[RB][4], sm[RB][4], lost[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      mx[rb][v] = -INFINITY;
      sm[rb][v] = 0.f;
      lost[rb][v] = -INFINITY;
    }

  const int64_t ntiles = A.Mp / kKdeTile;
  for (int64_t t = 0; t < ntiles; ++t) {
    const int buf = (int)(t & 1);
    if (t + 1 < ntiles) fetch(t + 1);
    floatx4 acc[RB][NT];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rb][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    const float* xt = xs[buf];
#pragma unroll
    for (int q = 0; q < KS / 4; ++q) {
      floatx4 bw[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bw[nt] = *reinterpret_cast<const floatx4*>(&xt[(nt * 16 + c16) * RS + g * KS + 4 * q]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[rb][nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rb][4 * q + j], bw[nt][j], acc[rb][nt], 0, 0, 0);
    }
    float bxv[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bxv[nt] = bs[buf][nt * 16 + c16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float l[NT];
        float lm = -INFINITY;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          l[nt] = fmaf(A.s2, acc[rb][nt][v], bxv[nt]);
          lm = fmaxf(lm, l[nt]);
        }
        const int pr = 16 * RB * wv + 16 * rb + 4 * g + v;
        float mr = mx[rb][v];
        // the reference moves only when a score passes it by more than
        // kKdeSlack (a wave-uniform test over the wave's four rows at v; the
        // first tile always moves it, every tile holding a real reference)
        if (__builtin_amdgcn_ballot_w64(lm > mr + kKdeSlack) != 0) {
          const float mn = fmaxf(mr, row16_max(lm));
          sm[rb][v] *= __builtin_amdgcn_exp2f(mr - mn);
          // a row's list is touched only by its own 16 lanes of this wave,
          // whose LDS operations execute in program order
          if (mn > mr && c16 == 0) {  // drop the listed terms now below the band
            const int n = min(cn[pr], kKdeCap);
            int k = 0;
            for (int q = 0; q < n; ++q) {
              const float lq = cl[pr * kKdeCap + q];
              if (lq >= mn - kKdeBand) {
                cj[pr * kKdeCap + k] = cj[pr * kKdeCap + q];
                cl[pr * kKdeCap + k] = lq;
                ++k;
              }
            }
            cn[pr] = k;
          }
          mx[rb][v] = mr = mn;
        }
        float s = sm[rb][v];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s += __builtin_amdgcn_exp2f(l[nt] - mr);
        sm[rb][v] = s;
        // terms within the band of the reference (a superset of those within
        // the band of the true maximum): listed for the exact rescoring
        // (padding scores are -inf)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (l[nt] >= mr - kKdeBand) {
            const int slot = atomicAdd(&cn[pr], 1);
            if (slot < kKdeCap) {
              cj[pr * kKdeCap + slot] = (int)(t * kKdeTile + nt * 16 + c16);
              cl[pr * kKdeCap + slot] = l[nt];
            } else {
              lost[rb][v] = fmaxf(lost[rb][v], l[nt]);
            }
          }
        }
      }
    // the idle buffer was last read before the previous barrier
    if (t + 1 < ntiles) stash(buf ^ 1);
    __syncthreads();
  }

  // ---- per row: the 16 lanes' sums; the listed terms exchanged for float64
  // ones (row, count and list are uniform across the row's 16 lanes); log p
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float st = row16_sum(sm[rb][v]);
      const int pr = 16 * RB * wv + 16 * rb + 4 * g + v;
      const int64_t row = q0 + pr;
      const int cnt = min(cn[pr], kKdeCap);
      const double m = (double)mx[rb][v];
      const double mfull = m + ays[pr];  // the reference in the frame of the full scores
      // complete when every term that could not be listed fell below the band
      const bool complete = row16_max(lost[rb][v]) < mx[rb][v] - kKdeBand;
      double S = (double)st;
      if (row < A.N && complete) {
        const float* yr = yb + row * A.ld;
        double sub = 0.0, add = 0.0;
        int last = -1;
        for (int r = 0; r < cnt; ++r) {
          // the next listed reference in increasing order (the list's own order
          // follows the atomics)
          int jn = 0x7fffffff;
          float ln = 0.f;
          for (int q = 0; q < cnt; ++q) {
            const int jq = cj[pr * kKdeCap + q];
            if (jq > last && jq < jn) {
              jn = jq;
              ln = cl[pr * kKdeCap + q];
            }
          }
          last = jn;
          const float* xr = A.ref + (int64_t)jn * A.ld_ref;
          double d2 = 0.0;
          for (int d = c16; d < A.D; d += 16) {
            const double u = (double)yr[d] - (double)xr[d];
            d2 += u * u;
          }
          d2 = row16_sum_f64(d2);
          sub += exp2((double)ln - m);
          add += exp2(-A.lam_exact * d2 - mfull);
        }
        S = fmax(S - sub, 0.0) + add;
      }
      if (c16 == 0 && row < A.N) A.out[b * A.N + row] = (float)((mfull + log2(S)) * LN2 + A.cnst);
    }
}

template <int DP>
hipError_t launch_kde_dp(const KdeArgs& a, hipStream_t s) {
  const int64_t nqb = (a.N + kKdeQ - 1) / kKdeQ;
  hipLaunchKernelGGL(kde_kernel<DP>, dim3((unsigned)(a.B * nqb)), dim3(kKdeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int kde_query_rows() { return kKdeQ; }
int kde_tile_rows() { return kKdeTile; }

hipError_t launch_kde_prep(const float* x, int64_t M, int64_t ld, int D, int DP, int64_t Mp, double lam, float* cen,
                           float* xc, float* bx, hipStream_t s) {
  hipLaunchKernelGGL(kde_centre_kernel, dim3((unsigned)DP), dim3(256), 0, s, x, M, ld, D, cen);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = Mp * DP;
  const int64_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
  hipLaunchKernelGGL(kde_refs_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, M, Mp, ld, D, DP, cen, xc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kde_norms_kernel, dim3((unsigned)((Mp + 255) / 256)), dim3(256), 0, s, xc, M, Mp, DP, lam, bx);
  return hipGetLastError();
}

hipError_t launch_kde(const KdeArgs& a, int DP, hipStream_t s) {
  switch (DP) {
    case 16: return launch_kde_dp<16>(a, s);
    case 32: return launch_kde_dp<32>(a, s);
    case 64: return launch_kde_dp<64>(a, s);
    case 128: return launch_kde_dp<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmm
