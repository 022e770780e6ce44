/*
 * gmm_oracle.c -- plain float64 CPU implementation of one EM iteration for a
 * Gaussian mixture model, plus the soft multi-assignment read-out.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity oracle: it is called by
 * the test-suite, by the smoke check and by the benchmark's CPU-baseline leg,
 * never by the product path.  It shares no code, header, table or helper with
 * the HIP library; the two meet only at the seeded input generator.
 *
 * What it follows (all citations are to the public pages the method is
 * described on):
 *   - "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft Clustering",
 *     Section 2: the mixture density, the log-likelihood objective, the E-step
 *     score pi_k N(x_i | mu_k, Sigma_k), its normalisation into responsibilities
 *     r_ik computed in log space with log-sum-exp, and the M-step: effective
 *     counts N_k (eq. 1), mixture weights N_k / N, responsibility-weighted
 *     means (eq. 2) and the updated variance (eq. 3).  Isotropic components
 *     (Sigma_k = sigma_k^2 I) are the paper's own restriction (footnote 1).
 *   - "ML0094 GMM vs K-Means", Mathematical Formulation: the same updates with
 *     a responsibility-weighted covariance (diagonal / full elliptical
 *     components).
 *   - GMMXX README, "Covariance Coverage": the four covariance types and their
 *     parameter shapes (spherical (B,K), diag (B,K,D), tied (B,D,D),
 *     full (B,K,D,D)), batched (B,N,D) inputs.
 *   - Flash-GMM, Section 4 and Conclusion (multi-assignment): a vector is stored
 *     in every list whose final responsibility passes a threshold.
 *
 * Readings taken where the pages are silent (the equations did not survive
 * extraction):
 *   - the variance uses the NEW mean (eq. 3 follows the mean update); written
 *     here through the exact identity
 *        sum_i r (x - mu')^2 / N_k = S2c / N_k - (mu' - mu)^2,
 *     with S2c accumulated about the means entering the step; oracle_mstep_twopass
 *     computes the literal two-pass form as a cross-check;
 *   - spherical variance = mean over dimensions of the per-dimension variance;
 *   - a regulariser eps (reg_covar) is added to every variance / covariance
 *     diagonal after the update;
 *   - a component with N_k == 0 keeps mu_k and Sigma_k, gets pi_k = 0, flag 1;
 *     a full/tied covariance whose Cholesky factorisation fails keeps the old
 *     component, flag 2 (M-step) / the component is dropped from the E-step,
 *     flag 4 (input not positive definite);
 *   - top-m: sort by responsibility (ties to the lower index), always keep the
 *     first, keep ranks 2..m whose responsibility is >= threshold, pad with -1.
 *
 * Everything is float64.  Inputs X are decoded exactly from their storage type.
 * Rows are split over OpenMP threads in contiguous chunks; per-thread partial
 * sums are merged in thread-index order, so results are reproducible for a
 * fixed thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

enum { OC_SPHERICAL = 0, OC_DIAG = 1, OC_TIED = 2, OC_FULL = 3 };
enum { OX_F64 = 0, OX_F32 = 1, OX_BF16 = 2, OX_F16 = 3 };

static const double LOG_2PI = 1.8378770664093454835606594728112;

/* ---------- exact decoding of the stored input element ---------- */
static double half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1, ex = (h >> 10) & 0x1f, man = h & 0x3ff;
  double v;
  if (ex == 0) v = ldexp((double)man, -24);               /* subnormal */
  else if (ex == 31) v = man ? NAN : INFINITY;
  else v = ldexp((double)(man | 0x400), ex - 25);
  return sign ? -v : v;
}
static double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}
static double x_at(const void* X, int xtype, int64_t idx) {
  switch (xtype) {
    case OX_F64: return ((const double*)X)[idx];
    case OX_F32: return (double)((const float*)X)[idx];
    case OX_BF16: return bf16_to_double(((const uint16_t*)X)[idx]);
    default: return half_to_double(((const uint16_t*)X)[idx]);
  }
}

/* ---------- dense linear algebra, textbook forms ---------- */
/* Cholesky A = L L^T (row-major D x D, lower triangle of L written, upper
 * zeroed).  Returns 0 on success, -1 if A is not positive definite. */
static int cholesky(int D, const double* A, double* L) {
  memset(L, 0, sizeof(double) * (size_t)D * D);
  for (int j = 0; j < D; ++j) {
    double s = A[j * D + j];
    for (int p = 0; p < j; ++p) s -= L[j * D + p] * L[j * D + p];
    if (!(s > 0.0)) return -1;
    double ljj = sqrt(s);
    L[j * D + j] = ljj;
    for (int i = j + 1; i < D; ++i) {
      double t = A[i * D + j];
      for (int p = 0; p < j; ++p) t -= L[i * D + p] * L[j * D + p];
      L[i * D + j] = t / ljj;
    }
  }
  return 0;
}
/* Solve L z = v by forward substitution. */
static void forward_solve(int D, const double* L, const double* v, double* z) {
  for (int i = 0; i < D; ++i) {
    double t = v[i];
    for (int p = 0; p < i; ++p) t -= L[i * D + p] * z[p];
    z[i] = t / L[i * D + i];
  }
}

/* Per-component quantities derived from theta for the log-density:
 * log det Sigma_k and, for full/tied, the Cholesky factor of Sigma_k. */
typedef struct {
  int cov, D, K;
  const double* w;    /* (K) mixture weights pi_k */
  const double* mu;   /* (K,D) */
  const double* cv;   /* covariance parameters, shape by type */
  double* logdet;     /* (K) */
  double* chol;       /* full: (K,D,D); tied: (D,D); else unused */
  int* ok;            /* (K) 1 if the component is usable */
} comp_t;

static int comp_prepare(comp_t* c) {
  int D = c->D, K = c->K;
  if (c->cov == OC_TIED) {
    int bad = cholesky(D, c->cv, c->chol);
    double ld = 0;
    if (!bad) for (int d = 0; d < D; ++d) ld += 2.0 * log(c->chol[d * D + d]);
    for (int k = 0; k < K; ++k) { c->logdet[k] = ld; c->ok[k] = !bad; }
    return 0;
  }
  for (int k = 0; k < K; ++k) {
    double ld = 0;
    int ok = 1;
    if (c->cov == OC_SPHERICAL) {
      double v = c->cv[k];
      ok = v > 0;
      ld = D * log(v);
    } else if (c->cov == OC_DIAG) {
      for (int d = 0; d < D; ++d) {
        double v = c->cv[(size_t)k * D + d];
        if (!(v > 0)) ok = 0;
        ld += log(v);
      }
    } else {
      double* L = c->chol + (size_t)k * D * D;
      if (cholesky(D, c->cv + (size_t)k * D * D, L)) ok = 0;
      else for (int d = 0; d < D; ++d) ld += 2.0 * log(L[d * D + d]);
    }
    c->logdet[k] = ld;
    c->ok[k] = ok;
  }
  return 0;
}

/* log( pi_k N(x | mu_k, Sigma_k) ) by direct differences (the unnormalised
 * E-step score of Flash-GMM Section 2, in log space).  tmp: 2*D doubles. */
static double log_score(const comp_t* c, int k, const double* x, double* tmp) {
  int D = c->D;
  if (!c->ok[k]) return -INFINITY;
  const double* m = c->mu + (size_t)k * D;
  double q = 0;
  if (c->cov == OC_SPHERICAL) {
    for (int d = 0; d < D; ++d) { double t = x[d] - m[d]; q += t * t; }
    q /= c->cv[k];
  } else if (c->cov == OC_DIAG) {
    const double* v = c->cv + (size_t)k * D;
    for (int d = 0; d < D; ++d) { double t = x[d] - m[d]; q += t * t / v[d]; }
  } else {
    const double* L = (c->cov == OC_FULL) ? c->chol + (size_t)k * D * D : c->chol;
    double* diff = tmp;
    double* z = tmp + D;
    for (int d = 0; d < D; ++d) diff[d] = x[d] - m[d];
    forward_solve(D, L, diff, z);
    for (int d = 0; d < D; ++d) q += z[d] * z[d];
  }
  return log(c->w[k]) - 0.5 * (D * LOG_2PI + c->logdet[k] + q);
}

static int64_t sxx_len(int cov, int D, int K) {
  switch (cov) {
    case OC_SPHERICAL: return K;
    case OC_DIAG: return (int64_t)K * D;
    case OC_TIED: return (int64_t)D * D;
    default: return (int64_t)K * D * D;
  }
}

/* Responsibilities of one row: l[k] = log score, returns LSE, r[k] written. */
static double responsibilities(const comp_t* c, const double* x, double* l, double* r, double* tmp) {
  int K = c->K;
  double m = -INFINITY;
  for (int k = 0; k < K; ++k) { l[k] = log_score(c, k, x, tmp); if (l[k] > m) m = l[k]; }
  double s = 0;
  for (int k = 0; k < K; ++k) s += exp(l[k] - m);
  double lse = m + log(s);
  for (int k = 0; k < K; ++k) r[k] = exp(l[k] - lse);
  return lse;
}

/*
 * One E-step with sufficient statistics, for B independent problems.
 *   X      (B,N,D) storage xtype, contiguous
 *   w      (B,K), mu (B,K,D), cv (B, sxx_len) -- theta_t as float64
 * Outputs (float64):
 *   nk  (B,K)    N_k = sum_i r_ik                       (Flash-GMM eq. 1)
 *   sx  (B,K,D)  sum_i r_ik x_i                          (numerator of eq. 2)
 *   sxx (B,...)  sum_i r_ik (x_i - mu_k)^2 / (x_i - mu_k)(x_i - mu_k)^T,
 *                about the means entering the step; tied: summed over k
 *   ll  (B)      sum_i log p(x_i) = sum_i LSE_i          (log-likelihood)
 *   flags (B,K)  4 if the input covariance is not positive definite
 * Returns 0, or -1 on bad arguments.
 */
int oracle_estep(int cov, int B, int64_t N, int D, int K, const void* X, int xtype,
                 const double* w, const double* mu, const double* cv,
                 double* nk, double* sx, double* sxx, double* ll, int* flags, int nthreads) {
  if (B < 1 || N < 0 || D < 1 || K < 1 || cov < 0 || cov > 3) return -1;
  if (nthreads < 1) nthreads = omp_get_max_threads();
  int64_t L2 = sxx_len(cov, D, K);
  int64_t plen = K + (int64_t)K * D + L2 + 1; /* per-thread partial: nk, sx, sxx, ll */
  double* part = (double*)calloc((size_t)plen * nthreads, sizeof(double));
  double* logdet = (double*)malloc(sizeof(double) * K);
  double* chol = (double*)malloc(sizeof(double) * (size_t)(cov == OC_FULL ? K : 1) * D * D);
  int* ok = (int*)malloc(sizeof(int) * K);
  if (!part || !logdet || !chol || !ok) { free(part); free(logdet); free(chol); free(ok); return -1; }

  for (int b = 0; b < B; ++b) {
    /* the covariance parameters of one problem have the same length as its sxx */
    comp_t c = {cov, D, K, w + (size_t)b * K, mu + (size_t)b * K * D, cv + (size_t)b * L2, logdet, chol, ok};
    comp_prepare(&c);
    memset(part, 0, sizeof(double) * (size_t)plen * nthreads);
    const void* Xb = X;
    int64_t xoff = (int64_t)b * N * D;

#pragma omp parallel num_threads(nthreads)
    {
      int t = omp_get_thread_num(), nt = omp_get_num_threads();
      int64_t lo = N * t / nt, hi = N * (t + 1) / nt;
      double* p = part + (size_t)plen * t;
      double *pnk = p, *psx = p + K, *psxx = p + K + (int64_t)K * D, *pll = p + plen - 1;
      double* x = (double*)malloc(sizeof(double) * D);
      double* l = (double*)malloc(sizeof(double) * K);
      double* r = (double*)malloc(sizeof(double) * K);
      double* tmp = (double*)malloc(sizeof(double) * 2 * D);
      double* diff = (double*)malloc(sizeof(double) * D);
      for (int64_t i = lo; i < hi; ++i) {
        for (int d = 0; d < D; ++d) x[d] = x_at(Xb, xtype, xoff + i * D + d);
        double lse = responsibilities(&c, x, l, r, tmp);
        *pll += lse;
        for (int k = 0; k < K; ++k) {
          double rk = r[k];
          const double* m = c.mu + (size_t)k * D;
          pnk[k] += rk;
          for (int d = 0; d < D; ++d) { psx[(size_t)k * D + d] += rk * x[d]; diff[d] = x[d] - m[d]; }
          if (cov == OC_SPHERICAL) {
            double s = 0;
            for (int d = 0; d < D; ++d) s += diff[d] * diff[d];
            psxx[k] += rk * s;
          } else if (cov == OC_DIAG) {
            for (int d = 0; d < D; ++d) psxx[(size_t)k * D + d] += rk * diff[d] * diff[d];
          } else {
            double* S = (cov == OC_FULL) ? psxx + (size_t)k * D * D : psxx;
            for (int d = 0; d < D; ++d)
              for (int e = 0; e < D; ++e) S[d * D + e] += rk * diff[d] * diff[e];
          }
        }
      }
      free(x); free(l); free(r); free(tmp); free(diff);
    }
    /* merge per-thread partials in thread order */
    double* onk = nk + (size_t)b * K;
    double* osx = sx + (size_t)b * K * D;
    double* osxx = sxx + (size_t)b * L2;
    memset(onk, 0, sizeof(double) * K);
    memset(osx, 0, sizeof(double) * (size_t)K * D);
    memset(osxx, 0, sizeof(double) * (size_t)L2);
    ll[b] = 0;
    for (int t = 0; t < nthreads; ++t) {
      const double* p = part + (size_t)plen * t;
      for (int k = 0; k < K; ++k) onk[k] += p[k];
      for (int64_t j = 0; j < (int64_t)K * D; ++j) osx[j] += p[K + j];
      for (int64_t j = 0; j < L2; ++j) osxx[j] += p[K + (int64_t)K * D + j];
      ll[b] += p[plen - 1];
    }
    if (flags) for (int k = 0; k < K; ++k) flags[(size_t)b * K + k] = ok[k] ? 0 : 4;
  }
  free(part); free(logdet); free(chol); free(ok);
  return 0;
}

/*
 * M-step from the statistics (Flash-GMM Section 2, eqs. 1-3; ML0094
 * Mathematical Formulation for the covariance forms), for B problems of
 * n rows each.  Inputs theta_in are the parameters that entered the E-step.
 *   pi_k  = N_k / n
 *   mu'_k = sx_k / N_k
 *   delta = mu'_k - mu_k
 *   spherical  var' = (sxx_k / N_k - |delta|^2) / D + eps
 *   diag       var'_d = sxx_kd / N_k - delta_d^2 + eps
 *   full       Sigma' = sxx_k / N_k - delta delta^T + eps I
 *   tied       Sigma' = (sxx - sum_k N_k delta_k delta_k^T) / n + eps I
 * flags (B,K): 1 empty component kept, 2 covariance not PD -> old kept.
 */
int oracle_mstep(int cov, int B, int64_t n, int D, int K,
                 const double* nk, const double* sx, const double* sxx,
                 const double* w_in, const double* mu_in, const double* cv_in, double eps,
                 double* w_out, double* mu_out, double* cv_out, int* flags) {
  if (B < 1 || n < 1 || D < 1 || K < 1) return -1;
  int64_t L2 = sxx_len(cov, D, K);
  double* L = (double*)malloc(sizeof(double) * (size_t)D * D);
  double* delta = (double*)malloc(sizeof(double) * (size_t)K * D);
  for (int b = 0; b < B; ++b) {
    const double* Nk = nk + (size_t)b * K;
    const double* S1 = sx + (size_t)b * K * D;
    const double* S2 = sxx + (size_t)b * L2;
    const double* m0 = mu_in + (size_t)b * K * D;
    const double* c0 = cv_in + (size_t)b * L2;
    double* wo = w_out + (size_t)b * K;
    double* mo = mu_out + (size_t)b * K * D;
    double* co = cv_out + (size_t)b * L2;
    int* fl = flags ? flags + (size_t)b * K : NULL;
    for (int k = 0; k < K; ++k) {
      wo[k] = Nk[k] / (double)n;
      if (fl) fl[k] = 0;
      for (int d = 0; d < D; ++d) {
        if (Nk[k] > 0) {
          mo[(size_t)k * D + d] = S1[(size_t)k * D + d] / Nk[k];
          delta[(size_t)k * D + d] = mo[(size_t)k * D + d] - m0[(size_t)k * D + d];
        } else {
          mo[(size_t)k * D + d] = m0[(size_t)k * D + d];
          delta[(size_t)k * D + d] = 0;
        }
      }
      if (!(Nk[k] > 0) && fl) fl[k] = 1;
    }
    if (cov == OC_TIED) {
      for (int d = 0; d < D; ++d)
        for (int e = 0; e < D; ++e) {
          double s = S2[d * D + e];
          for (int k = 0; k < K; ++k) s -= Nk[k] * delta[(size_t)k * D + d] * delta[(size_t)k * D + e];
          co[d * D + e] = s / (double)n + (d == e ? eps : 0.0);
        }
      if (cholesky(D, co, L)) {   /* keep the whole previous model */
        memcpy(co, c0, sizeof(double) * (size_t)D * D);
        memcpy(mo, m0, sizeof(double) * (size_t)K * D);
        if (fl) for (int k = 0; k < K; ++k) fl[k] |= 2;
      }
      continue;
    }
    for (int k = 0; k < K; ++k) {
      double nkk = Nk[k];
      const double* dk = delta + (size_t)k * D;
      if (!(nkk > 0)) {
        if (cov == OC_SPHERICAL) co[k] = c0[k];
        else if (cov == OC_DIAG) memcpy(co + (size_t)k * D, c0 + (size_t)k * D, sizeof(double) * D);
        else memcpy(co + (size_t)k * D * D, c0 + (size_t)k * D * D, sizeof(double) * (size_t)D * D);
        continue;
      }
      if (cov == OC_SPHERICAL) {
        double dd = 0;
        for (int d = 0; d < D; ++d) dd += dk[d] * dk[d];
        co[k] = (S2[k] / nkk - dd) / (double)D + eps;
      } else if (cov == OC_DIAG) {
        for (int d = 0; d < D; ++d)
          co[(size_t)k * D + d] = S2[(size_t)k * D + d] / nkk - dk[d] * dk[d] + eps;
      } else {
        double* C = co + (size_t)k * D * D;
        const double* S = S2 + (size_t)k * D * D;
        for (int d = 0; d < D; ++d)
          for (int e = 0; e < D; ++e)
            C[d * D + e] = S[d * D + e] / nkk - dk[d] * dk[e] + (d == e ? eps : 0.0);
        if (cholesky(D, C, L)) {
          memcpy(C, c0 + (size_t)k * D * D, sizeof(double) * (size_t)D * D);
          memcpy(mo + (size_t)k * D, m0 + (size_t)k * D, sizeof(double) * D);
          if (fl) fl[k] |= 2;
        }
      }
    }
  }
  free(L); free(delta);
  return 0;
}

/*
 * Literal two-pass M-step (cross-check of the identity used above): pass 1
 * computes N_k and the new means from the responsibilities; pass 2 recomputes
 * the responsibilities and accumulates sum_i r_ik (x_i - mu'_k)(...) directly.
 * Single thread, single problem.  Same output conventions as oracle_mstep.
 */
int oracle_mstep_twopass(int cov, int64_t N, int D, int K, const void* X, int xtype,
                         const double* w, const double* mu, const double* cv, double eps,
                         double* w_out, double* mu_out, double* cv_out) {
  int64_t L2 = sxx_len(cov, D, K);
  double* logdet = (double*)malloc(sizeof(double) * K);
  double* chol = (double*)malloc(sizeof(double) * (size_t)(cov == OC_FULL ? K : 1) * D * D);
  int* ok = (int*)malloc(sizeof(int) * K);
  comp_t c = {cov, D, K, w, mu, cv, logdet, chol, ok};
  comp_prepare(&c);
  double* x = (double*)malloc(sizeof(double) * D);
  double* l = (double*)malloc(sizeof(double) * K);
  double* r = (double*)malloc(sizeof(double) * K);
  double* tmp = (double*)malloc(sizeof(double) * 2 * D);
  double* Nk = (double*)calloc(K, sizeof(double));
  double* acc = (double*)calloc((size_t)L2, sizeof(double));
  memset(mu_out, 0, sizeof(double) * (size_t)K * D);
  for (int64_t i = 0; i < N; ++i) {
    for (int d = 0; d < D; ++d) x[d] = x_at(X, xtype, i * D + d);
    responsibilities(&c, x, l, r, tmp);
    for (int k = 0; k < K; ++k) {
      Nk[k] += r[k];
      for (int d = 0; d < D; ++d) mu_out[(size_t)k * D + d] += r[k] * x[d];
    }
  }
  for (int k = 0; k < K; ++k) {
    w_out[k] = Nk[k] / (double)N;
    for (int d = 0; d < D; ++d)
      mu_out[(size_t)k * D + d] = Nk[k] > 0 ? mu_out[(size_t)k * D + d] / Nk[k] : mu[(size_t)k * D + d];
  }
  for (int64_t i = 0; i < N; ++i) {
    for (int d = 0; d < D; ++d) x[d] = x_at(X, xtype, i * D + d);
    responsibilities(&c, x, l, r, tmp);
    for (int k = 0; k < K; ++k) {
      const double* m = mu_out + (size_t)k * D;
      if (cov == OC_SPHERICAL) {
        double s = 0;
        for (int d = 0; d < D; ++d) s += (x[d] - m[d]) * (x[d] - m[d]);
        acc[k] += r[k] * s;
      } else if (cov == OC_DIAG) {
        for (int d = 0; d < D; ++d) acc[(size_t)k * D + d] += r[k] * (x[d] - m[d]) * (x[d] - m[d]);
      } else {
        double* S = (cov == OC_FULL) ? acc + (size_t)k * D * D : acc;
        for (int d = 0; d < D; ++d)
          for (int e = 0; e < D; ++e) S[d * D + e] += r[k] * (x[d] - m[d]) * (x[e] - m[e]);
      }
    }
  }
  for (int64_t j = 0; j < L2; ++j) cv_out[j] = 0;
  for (int k = 0; k < K; ++k) {
    if (cov == OC_SPHERICAL) cv_out[k] = Nk[k] > 0 ? acc[k] / Nk[k] / D + eps : cv[k];
    else if (cov == OC_DIAG)
      for (int d = 0; d < D; ++d)
        cv_out[(size_t)k * D + d] = Nk[k] > 0 ? acc[(size_t)k * D + d] / Nk[k] + eps : cv[(size_t)k * D + d];
    else if (cov == OC_FULL)
      for (int d = 0; d < D; ++d)
        for (int e = 0; e < D; ++e)
          cv_out[(size_t)k * D * D + d * D + e] = Nk[k] > 0
              ? acc[(size_t)k * D * D + d * D + e] / Nk[k] + (d == e ? eps : 0.0)
              : cv[(size_t)k * D * D + d * D + e];
  }
  if (cov == OC_TIED)
    for (int d = 0; d < D; ++d)
      for (int e = 0; e < D; ++e) cv_out[d * D + e] = acc[d * D + e] / (double)N + (d == e ? eps : 0.0);
  free(logdet); free(chol); free(ok); free(x); free(l); free(r); free(tmp); free(Nk); free(acc);
  return 0;
}

/*
 * Per-row log scores and responsibilities (small inputs only, single problem):
 *   logscore (N,K) = log pi_k + log N(x_i | theta_k),  resp (N,K) = r_ik,  lse (N).
 */
int oracle_responsibilities(int cov, int64_t N, int D, int K, const void* X, int xtype,
                            const double* w, const double* mu, const double* cv,
                            double* logscore, double* resp, double* lse) {
  double* logdet = (double*)malloc(sizeof(double) * K);
  double* chol = (double*)malloc(sizeof(double) * (size_t)(cov == OC_FULL ? K : 1) * D * D);
  int* ok = (int*)malloc(sizeof(int) * K);
  comp_t c = {cov, D, K, w, mu, cv, logdet, chol, ok};
  comp_prepare(&c);
  double* x = (double*)malloc(sizeof(double) * D);
  double* tmp = (double*)malloc(sizeof(double) * 2 * D);
  for (int64_t i = 0; i < N; ++i) {
    for (int d = 0; d < D; ++d) x[d] = x_at(X, xtype, i * D + d);
    lse[i] = responsibilities(&c, x, logscore + i * K, resp + i * K, tmp);
  }
  free(logdet); free(chol); free(ok); free(x); free(tmp);
  return 0;
}

/*
 * Soft multi-assignment (Flash-GMM Section 4 / Conclusion): for each row,
 * order the components by descending responsibility (ties: lower index
 * first), keep the first always and ranks 2..m whose responsibility is at
 * least `thr`.  Single problem.
 *   idx (N,m) int32, -1 padded;  resp (N,m);  count (N);  logp (N) = LSE_i
 *   margin (N): smallest gap that decides the output.  With c kept ranks,
 *   the output is fixed by the order of ranks 1..c+1 (the gaps between
 *   consecutive ones) and by the threshold tests of ranks 2..min(c+1, m);
 *   the order of the ranks after c+1 does not show in it.
 */
int oracle_topm(int cov, int64_t N, int D, int K, const void* X, int xtype,
                const double* w, const double* mu, const double* cv, int m, double thr,
                int32_t* idx, double* resp, int32_t* count, double* logp, double* margin, int nthreads) {
  if (m < 1 || K < 1) return -1;
  if (nthreads < 1) nthreads = omp_get_max_threads();
  double* logdet = (double*)malloc(sizeof(double) * K);
  double* chol = (double*)malloc(sizeof(double) * (size_t)(cov == OC_FULL ? K : 1) * D * D);
  int* ok = (int*)malloc(sizeof(int) * K);
  comp_t c = {cov, D, K, w, mu, cv, logdet, chol, ok};
  comp_prepare(&c);
#pragma omp parallel num_threads(nthreads)
  {
    double* x = (double*)malloc(sizeof(double) * D);
    double* l = (double*)malloc(sizeof(double) * K);
    double* r = (double*)malloc(sizeof(double) * K);
    double* tmp = (double*)malloc(sizeof(double) * 2 * D);
    int* rank = (int*)malloc(sizeof(int) * (m + 1));
#pragma omp for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
      for (int d = 0; d < D; ++d) x[d] = x_at(X, xtype, i * D + d);
      logp[i] = responsibilities(&c, x, l, r, tmp);
      /* selection of the m+1 best by repeated scan (ties -> lower k) */
      int nr = (m + 1 < K) ? m + 1 : K;
      for (int j = 0; j < nr; ++j) {
        int best = -1;
        for (int k = 0; k < K; ++k) {
          int used = 0;
          for (int p = 0; p < j; ++p) if (rank[p] == k) used = 1;
          if (used) continue;
          if (best < 0 || r[k] > r[best]) best = k;
        }
        rank[j] = best;
      }
      int cnt = 0;
      for (int j = 0; j < m; ++j) {
        int keep = (j < nr) && (j == 0 || r[rank[j]] >= thr);
        if (keep && cnt == j) {
          idx[i * m + j] = rank[j];
          resp[i * m + j] = r[rank[j]];
          ++cnt;
        } else {
          idx[i * m + j] = -1;
          resp[i * m + j] = 0.0;
        }
      }
      count[i] = cnt;
      double mg = INFINITY;
      for (int j = 0; j < cnt && j + 1 < nr; ++j) {
        double g = r[rank[j]] - r[rank[j + 1]];
        if (g < mg) mg = g;
      }
      for (int j = 1; j <= cnt && j < nr && j < m; ++j) {
        double g = fabs(r[rank[j]] - thr);
        if (g < mg) mg = g;
      }
      margin[i] = mg;
    }
    free(x); free(l); free(r); free(tmp); free(rank);
  }
  free(logdet); free(chol); free(ok);
  return 0;
}

/*
 * One k-means (Lloyd) iteration: the hard-assignment limit of EM ("ML0094
 * GMM vs K-Means": k-means assigns each point to the centroid at the smallest
 * distance and is the limit of a GMM with one shared spherical variance going
 * to zero, where the posterior collapses to an argmax; the mean update with
 * 0/1 responsibilities is the mean of the cluster's points).  Flash-GMM
 * Section 4: k-means is the usual coarse quantizer of an IVF index.
 * Single problem, centroids C (K,D).
 *   labels (N): argmin_k |x_i - c_k|^2 by direct differences, ties to the
 *     lower k;  gap (N): second smallest minus smallest distance (INFINITY
 *     when K == 1) -- the margin that decides the label;
 *   newC (K,D): mean of the rows labelled k (summed in row order); a cluster
 *     with no rows keeps its centroid;  counts (K);
 *   inertia: sum over rows of the smallest distance, in row order.
 */
int oracle_kmeans_step(int64_t N, int D, int K, const void* X, int xtype, const double* C,
                       int32_t* labels, double* gap, double* newC, int64_t* counts, double* inertia,
                       int nthreads) {
  if (K < 1 || D < 1 || N < 0) return -1;
  if (nthreads < 1) nthreads = omp_get_max_threads();
  double* qmin = (double*)malloc(sizeof(double) * (N > 0 ? N : 1));
#pragma omp parallel num_threads(nthreads)
  {
    double* x = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
      for (int d = 0; d < D; ++d) x[d] = x_at(X, xtype, i * D + d);
      double best = INFINITY, second = INFINITY;
      int arg = 0;
      for (int k = 0; k < K; ++k) {
        double q = 0.0;
        for (int d = 0; d < D; ++d) {
          const double t = x[d] - C[(size_t)k * D + d];
          q += t * t;
        }
        if (q < best) {
          second = best;
          best = q;
          arg = k;
        } else if (q < second) {
          second = q;
        }
      }
      labels[i] = arg;
      qmin[i] = best;
      gap[i] = second - best;
    }
    free(x);
  }
  double* sum = (double*)calloc((size_t)K * D, sizeof(double));
  for (int k = 0; k < K; ++k) counts[k] = 0;
  double in = 0.0;
  for (int64_t i = 0; i < N; ++i) {
    const int k = labels[i];
    for (int d = 0; d < D; ++d) sum[(size_t)k * D + d] += x_at(X, xtype, i * D + d);
    counts[k] += 1;
    in += qmin[i];
  }
  for (int k = 0; k < K; ++k)
    for (int d = 0; d < D; ++d)
      newC[(size_t)k * D + d] = counts[k] > 0 ? sum[(size_t)k * D + d] / (double)counts[k] : C[(size_t)k * D + d];
  *inertia = in;
  free(sum);
  free(qmin);
  return 0;
}

/* The stored input elements as the oracle reads them (exact decoding). */
int oracle_decode(int xtype, int64_t n, const void* X, double* out) {
  if (n < 0 || xtype < OX_F64 || xtype > OX_F16) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = x_at(X, xtype, i);
  return 0;
}

int oracle_version(void) { return 1; }
