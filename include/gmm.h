/*
 * gmm.h -- C ABI of the MI355X (gfx950) fused EM library for Gaussian mixture
 * models.
 *
 * The method: one EM iteration for a mixture of K Gaussians, as described in
 * "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft Clustering",
 * Section 2 (E-step score pi_k N(x_i | mu_k, Sigma_k), responsibilities r_ik
 * normalised in log space with log-sum-exp, M-step eqs. 1-3: N_k, pi_k = N_k/N,
 * mu_k = sum_i r_ik x_i / N_k, updated variance) and Section 3 (the N x K
 * responsibility matrix is never written to device memory: each tile of rows
 * folds its responsibilities straight into O(K D) sufficient statistics).
 * Covariance types and parameter shapes follow the GMMXX README, "Covariance
 * Coverage"; soft multi-assignment follows Flash-GMM Section 4 / Conclusion
 * (a threshold on the final responsibilities).
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer owned by the caller, except the
 *     descriptor structs themselves, which live in host memory and are read
 *     during the call only.
 *   - The library allocates no device memory.  Scratch space is the caller's
 *     workspace `ws` of `ws_bytes` bytes (256-byte aligned), sized with
 *     gmm_workspace_bytes(); for the fit / statistics calls its size does not
 *     grow with N once N exceeds a few hundred thousand rows per problem.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued asynchronously on it; nothing synchronises the host.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     status other than GMM_OK means nothing was enqueued;
 *     gmm_last_error() then returns a message for the calling thread.
 *   - Numerical events are reported per component in `comp_status` (B,K)
 *     int32 (nullable), never as call failures:
 *        1  N_k == 0 after the E-step: mu_k and Sigma_k kept, pi_k = 0;
 *        2  the updated full/tied covariance is not positive definite: the
 *           previous mu_k and Sigma_k are kept;
 *        4  the input full/tied covariance is not positive definite: the
 *           component gets zero responsibility in this E-step.
 *   - Results are deterministic: no global-memory atomics, and every reduction
 *     runs in a fixed order for a given shape.  Two kernels hand out slots of
 *     per-row candidate lists with LDS atomic counters (top-m: the waves of a
 *     workgroup; kernel density: the 16 lanes of one row); the lists are
 *     sorted by (score, index), or walked in increasing index order, before
 *     any result depends on them, so the slot order never shows.
 *   - Calls on distinct streams with distinct workspaces may run concurrently.
 */
#ifndef GMM_H
#define GMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GMM_COV_SPHERICAL = 0, /* Sigma_k = sigma_k^2 I; covars (B,K)            */
  GMM_COV_DIAG = 1,      /* Sigma_k = diag(sigma_k^2); covars (B,K,D)      */
  GMM_COV_TIED = 2,      /* Sigma_k = Sigma for all k; covars (B,D,D)      */
  GMM_COV_FULL = 3       /* one full Sigma_k per component; (B,K,D,D)      */
} gmm_cov_type;

/* Row types.  16-bit rows are read exactly (every bf16 and half value is a
 * float32 value).  bf16 rows of one problem with spherical components take
 * the large-K path (bf16 MFMA, any K <= 16384, D <= 128); every other 16-bit
 * case takes the fused path of float32 rows (its K and D window), the rows
 * decoded to float32 as a tile is staged in LDS. */
typedef enum {
  GMM_DT_F32 = 0,  /* IEEE float32 rows                                     */
  GMM_DT_BF16 = 1, /* bfloat16 rows                                         */
  GMM_DT_F16 = 2   /* IEEE half rows                                        */
} gmm_dtype;

typedef enum {
  GMM_OK = 0,
  GMM_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad stride, ...  */
  GMM_ERR_UNSUPPORTED = 2, /* valid but outside the supported shape/type window */
  GMM_ERR_WORKSPACE = 3,   /* ws is NULL, misaligned or smaller than required   */
  GMM_ERR_HIP = 4,         /* a HIP launch or runtime call failed               */
  GMM_ERR_NOT_PD = 5       /* a covariance is not positive definite (returned by
                              gmm_check_components only: the compute calls run
                              asynchronously and report it per component)      */
} gmm_status;

/* Operation selector for gmm_workspace_bytes. */
enum { GMM_OP_FIT = 0, GMM_OP_ESTEP = 1, GMM_OP_TOPM = 2 };

/* Input rows: problem b, row i, dimension d is element
 *   x[b * stride_b + i * ld_x + d]   (elements of `dtype`),
 * with ld_x >= D and stride_b >= N * ld_x (stride_b ignored when B == 1).
 * x must be 16-byte aligned and ld_x * sizeof(element) a multiple of 16 bytes
 * for the vectorised loads; other layouts return GMM_ERR_UNSUPPORTED. */
typedef struct {
  const void* x;
  int32_t dtype;  /* gmm_dtype */
  int64_t B, N, D;
  int64_t ld_x, stride_b;
} gmm_data;

/* Mixture parameters theta, float32, row-major:
 *   weights (B,K); means (B,K,D);
 *   covars  spherical (B,K) | diag (B,K,D) | tied (B,D,D) | full (B,K,D,D). */
typedef struct {
  int32_t K;
  int32_t cov;  /* gmm_cov_type */
  float* weights;
  float* means;
  float* covars;
} gmm_params;

/* Sufficient statistics of one E-step, float64, device:
 *   nk (B,K)      N_k = sum_i r_ik                        (Flash-GMM eq. 1)
 *   sx (B,K,D)    sum_i r_ik x_i                           (numerator of eq. 2)
 *   sxx           sum_i r_ik (x_i - mu_k)(x_i - mu_k)^T about the means that
 *                 entered the E-step: spherical (B,K) trace form
 *                 sum_i r_ik |x_i - mu_k|^2; diag (B,K,D) diagonal;
 *                 full (B,K,D,D); tied (B,D,D) summed over k
 *   loglik (B)    sum_i log p(x_i) under the parameters that entered the step */
typedef struct {
  double* nk;
  double* sx;
  double* sxx;
  double* loglik;
} gmm_stats;

/* Options.  reg_covar is added to every variance / covariance diagonal after
 * the update (the covariance floor; 1e-6 is the usual value).  flags must be 0.
 * event_begin / event_end: optional hipEvent_t handles; when non-NULL they are
 * recorded on `stream` immediately before and after the fused E-step kernel,
 * so a caller can time that kernel alone. */
typedef struct {
  double reg_covar;
  uint32_t flags;
  void* event_begin;
  void* event_end;
} gmm_options;

/* Bytes of workspace needed by an operation on `data` with K components of
 * type `cov` (op: GMM_OP_FIT / GMM_OP_ESTEP / GMM_OP_TOPM; m: the top-m width,
 * ignored otherwise).  Returns 0 when the arguments are invalid or the shape is
 * unsupported (the compute call then reports why).  Host-only; no HIP call.
 *
 * Shape window of the fit / statistics calls on float32 rows (and 16-bit rows
 * outside the bf16 large-K path): spherical and diagonal components with
 * D <= 128 and K <= 8192, full and tied components with D <= 16 and K <= 256.
 * Spherical and diagonal problems with more components than one workgroup
 * holds (256; 128 for diagonal at D = 128) run their E-step in blocks of
 * components over chunks of 2^20 rows (the rows' log-sum-exp taken over
 * every block, Flash-GMM Section 3); their workspace then also holds two
 * float2 per (problem, row of a chunk) and one per (problem, row, block). */
size_t gmm_workspace_bytes(const gmm_data* data, int32_t K, int32_t cov, int32_t op, int32_t m);

/* E-step with statistics (Flash-GMM Section 2; the fused, R-free form of
 * Section 3).  Computes the statistics of `data` under `params` and writes
 * them to `out`, or adds them to `out` when accumulate != 0 (chunked
 * streaming: call once per chunk of rows with the same params, then
 * gmm_mstep with n_total = all rows).  The sxx centre is params->means. */
gmm_status gmm_estep_stats(const gmm_data* data, const gmm_params* params, gmm_stats* out,
                           int32_t accumulate, void* ws, size_t ws_bytes, void* stream);

/* M-step (Flash-GMM Section 2, eqs. 1-3, extended to diag/tied/full as in
 * "ML0094 GMM vs K-Means", Mathematical Formulation) from statistics `st` of
 * B problems of dimension D over n_total rows each.  `inout` holds on entry
 * the parameters the statistics were computed with and receives theta':
 *   pi_k = N_k / n_total;  mu'_k = sx_k / N_k;  delta_k = mu'_k - mu_k;
 *   spherical  var' = (sxx_k / N_k - |delta_k|^2) / D + reg_covar
 *   diag       var'_d = sxx_kd / N_k - delta_kd^2 + reg_covar
 *   full       Sigma'_k = sxx_k / N_k - delta_k delta_k^T + reg_covar I
 *   tied       Sigma' = (sxx - sum_k N_k delta_k delta_k^T) / n_total + reg_covar I
 * comp_status (B,K) int32, nullable.  opts may be NULL (reg_covar = 1e-6). */
gmm_status gmm_mstep(int64_t B, int64_t D, const gmm_stats* st, int64_t n_total, gmm_params* inout,
                     const gmm_options* opts, int32_t* comp_status, void* stream);

/* One EM iteration (E-step statistics + M-step) in place on `inout`.
 * mean_loglik (B) float64 device, nullable: (1/N) sum_i log p(x_i) under the
 * parameters that ENTERED the step.  comp_status nullable. */
gmm_status gmm_fit_step(const gmm_data* data, gmm_params* inout, const gmm_options* opts,
                        double* mean_loglik, int32_t* comp_status, void* ws, size_t ws_bytes,
                        void* stream);

/* n_iter EM iterations in one call (Flash-GMM Section 2, the EM iteration
 * repeated), with the same results, bit for bit, as n_iter calls of
 * gmm_fit_step on this workspace.  Spherical, diagonal and full components:
 * after the first iteration the prologue (the log-score weights and
 * constants) is not launched; each iteration's M-step, in the reduction's
 * component blocks, forms it for the next one right after the parameters
 * (one launch fewer per iteration).  Tied components and the large-K path
 * run n_iter fit steps.  n_iter >= 1.  mean_loglik: (n_iter, B) float64
 * device, nullable; row t is the mean log-likelihood of the parameters that
 * entered iteration t.  comp_status (B,K) nullable: the last iteration's
 * flags.  The workspace is gmm_fit_step's (GMM_OP_FIT).  opts->event_begin /
 * event_end, when set, bracket the last iteration's E-step. */
gmm_status gmm_fit(const gmm_data* data, gmm_params* inout, const gmm_options* opts, int32_t n_iter,
                   double* mean_loglik, int32_t* comp_status, void* ws, size_t ws_bytes, void* stream);

/* One EM iteration exactly as gmm_fit_step (same kernels, same results), for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  It takes no
 * workspace: its scratch is a static device array of 64 MiB per GPU, which
 * the library holds from its first use on that GPU until the process ends.
 * A problem whose workspace (gmm_workspace_bytes with GMM_OP_FIT) exceeds
 * 64 MiB returns GMM_ERR_WORKSPACE before anything is enqueued (bf16 rows
 * stream in shorter chunks when the part that does not grow with N fits).
 * The array belongs to the current HIP device; every call on that device
 * uses the same array, so calls that overlap in time on one GPU (other
 * streams, other threads) race: serialise them.  Nothing in the array needs
 * to start at zero.  No hipMalloc, hipFree or allocating library call. */
gmm_status gmm_fit_step_noalloc(const gmm_data* data, gmm_params* inout, const gmm_options* opts,
                                double* mean_loglik, int32_t* comp_status, void* stream);

/* One EM iteration (as gmm_fit_step) over rows that stay in HOST memory
 * (Flash-GMM Section 1: datasets beyond what fits; Section 3: the statistics
 * are O(K D); GMMXX README, "CUDA backend (experimental)": large-N streaming
 * of CPU-resident data through the E/M kernels).  host_data describes the
 * rows exactly as gmm_data does, but host_data->x is a host pointer; for
 * copies that overlap the compute it must be pinned (hipHostMalloc, or a
 * torch tensor made with pin_memory=True), pageable memory works but its
 * copies do not overlap.  The rows go through two device buffers of
 * chunk_rows rows per problem in the workspace: chunk c is copied on
 * copy_stream while the E-step of chunk c - 1 runs on stream (events order
 * them; copy_stream NULL = everything on stream), each chunk's statistics
 * are added to one float64 set, then one M-step updates `inout`.  Device
 * memory: gmm_fit_step_streamed_workspace_bytes, which depends on K, D, B
 * and chunk_rows but not on N.  mean_loglik / comp_status as gmm_fit_step.
 * The results equal gmm_fit_step's up to the order of the float64 sums.
 * The host rows must stay unchanged until the call's work on `stream` has
 * completed. */
size_t gmm_fit_step_streamed_workspace_bytes(const gmm_data* host_data, int32_t K, int32_t cov, int64_t chunk_rows);
gmm_status gmm_fit_step_streamed(const gmm_data* host_data, gmm_params* inout, const gmm_options* opts,
                                 int64_t chunk_rows, double* mean_loglik, int32_t* comp_status, void* ws,
                                 size_t ws_bytes, void* stream, void* copy_stream);

/* Soft multi-assignment (Flash-GMM Section 4 / Conclusion): for every row,
 * components ordered by decreasing responsibility (ties: lower index first);
 * the first is always kept, ranks 2..m are kept while r >= threshold.
 *   idx   (B,N,m) int32, -1 padded      resp (B,N,m) float32, 0 padded
 *   count (B,N) int32, nullable          logp (B,N) float32 = log p(x_i), nullable
 * The ranking and the kept responsibilities are decided in float64 for every
 * component whose single-precision score lies within a safety band of the
 * best one.  1 <= m <= 16.  Window: bf16 rows of one problem with spherical
 * components, K <= 16384 (the large-K path); other rows, full and tied
 * components with K <= 256 (D <= 16), spherical and diagonal components with
 * K <= 8192 (D <= 128) -- above 256 every score of a row is computed exactly
 * in float64 instead of through the band. */
gmm_status gmm_predict_proba_topm(const gmm_data* data, const gmm_params* params, int32_t m,
                                  float threshold, int32_t* idx, float* resp, int32_t* count,
                                  float* logp, void* ws, size_t ws_bytes, void* stream);

/* Inverted lists (IVF posting lists) from a soft multi-assignment
 * (Flash-GMM Section 4 -- the GMM as the IVF coarse quantizer, with the
 * multi-assignment of Section 4.3 -- and Conclusion: boundary vectors are
 * stored in several posting lists).  For every problem b and component k, the
 * rows whose assignment kept k, in increasing row order, as CSR.
 *   idx  (B,N,m) int32, as written by gmm_predict_proba_topm: a row's entries
 *        are its leading values in [0, K); the first value outside ends the row
 *        (-1 padding does); values within a row are expected distinct
 *   resp (B,N,m) float32, nullable: copied to list_resp when that is non-NULL
 *   offsets   (B,K+1) int64: list k of problem b is
 *             rows[b, offsets[b,k] .. offsets[b,k+1]-1]; offsets[b,K] = its entries
 *   rows      (B,N*m) int32: row indices; entries past offsets[b,K] untouched
 *   list_resp (B,N*m) float32, nullable: the responsibility of each entry
 * 1 <= m <= 16, 1 <= K <= 16384, N*m < 2^31.  Workspace:
 * gmm_ivf_workspace_bytes (4 bytes per (problem, 4096-row block, component)).
 * Deterministic (no atomics), bit-identical across runs. */
size_t gmm_ivf_workspace_bytes(int64_t B, int64_t N, int32_t m, int32_t K);
gmm_status gmm_ivf_lists(int64_t B, int64_t N, int32_t m, int32_t K, const int32_t* idx, const float* resp,
                         int64_t* offsets, int32_t* rows, float* list_resp, void* ws, size_t ws_bytes,
                         void* stream);

/* One k-means (Lloyd) iteration: the hard-assignment limit of EM ("ML0094
 * GMM vs K-Means": k-means gives each point to the centroid at the smallest
 * distance, the limit of a GMM with one shared spherical variance going to
 * zero, where the posterior collapses to an argmax; Flash-GMM Section 4: the
 * usual IVF coarse quantizer).  For each problem b of `data`:
 *   labels (B,N) int32 out: argmin_k |x_i - c_k|^2 under the centroids that
 *     enter the call, decided on float64 distances, ties to the lower k;
 *   centroids (B,K,D) float32 in/out: replaced by the mean of the rows
 *     labelled k (summed in float64, in increasing row order); a cluster with
 *     no rows keeps its centroid;
 *   counts (B,K) int64 out, nullable: rows per cluster;
 *   inertia (B) float64 out, nullable: sum_i min_k |x_i - c_k|^2 under the
 *     entering centroids.
 * Same row types and shape window as gmm_predict_proba_topm with spherical
 * components (float32 and half rows: K <= 8192, any B; bf16 rows: B = 1,
 * K <= 16384, or as float32 rows for several problems), and N < 2^31.  Workspace: gmm_kmeans_workspace_bytes (it grows with N: the
 * labels' posting lists and a responsibility per row).  The assignment is the
 * library's exact top-1 under equal weights and one shared variance, so its
 * labels agree with a float64 nearest-centroid search wherever the two
 * smallest distances differ by more than their rounding.  Deterministic. */
size_t gmm_kmeans_workspace_bytes(const gmm_data* data, int32_t K);
gmm_status gmm_kmeans_step(const gmm_data* data, int32_t K, float* centroids, int32_t* labels, int64_t* counts,
                           double* inertia, void* ws, size_t ws_bytes, void* stream);

/* One approximate top-k EM iteration (the approx_top_k training mode of the
 * GMMXX README, "Useful Options" and "CUDA backend (experimental)"; statistics
 * and M-step as Flash-GMM Section 2): each row keeps the topk components of
 * largest log-score log pi_k N(x | theta_k) (decided on float64 scores, ties to
 * the lower index), its responsibilities renormalised over that subset; only
 * those enter N_k, sum r x and sum r (x - mu)^2 (float64, summed per
 * component in increasing row order); then the M-step of gmm_mstep updates
 * `inout` in place.  topk >= K keeps every component: the exact EM step.
 * mean_loglik (B) float64, nullable: the mean over rows of log sum over each
 * row's kept components of pi_k N(x | theta_k), under the entering theta.
 * Spherical and diagonal components; the top-m window (float32 rows: K <=
 * 8192, any B; bf16 rows: spherical, B = 1, K <= 16384); 1 <= topk <= 16;
 * N * topk < 2^31.  The candidates of a row are the components whose score can reach
 * a lower bound of its topk-th best score; with bf16 rows of D != 128 (or not
 * 16-byte aligned) that bound is not formed and every component of the row
 * is rescored (correct, slower).  Workspace: gmm_topk_fit_workspace_bytes (it
 * grows with N * topk).  Deterministic. */
size_t gmm_topk_fit_workspace_bytes(const gmm_data* data, int32_t K, int32_t cov, int32_t topk);
gmm_status gmm_topk_fit_step(const gmm_data* data, gmm_params* inout, int32_t topk, const gmm_options* opts,
                             double* mean_loglik, int32_t* comp_status, void* ws, size_t ws_bytes, void* stream);

/* Fisher vectors of B sets of N rows (data as (B, N, D) float32) under ONE
 * diagonal model (model: K, cov = GMM_COV_DIAG, weights (K), means (K, D),
 * covars (K, D) variances) -- the encoding Flash-GMM's closing discussion
 * names as the same fused log-sum-exp and weighted-statistics pattern
 * (Perronnin et al. 2010, improved form).  Per set b, with r the
 * responsibilities:
 *   fv[b][k D + d]       = (sum_i r_ik x_id - N_k mu_kd) / (sigma_kd N sqrt(w_k))
 *   fv[b][K D + k D + d] = (sum_i r_ik (x_id - mu_kd)^2 / sigma_kd^2 - N_k) / (N sqrt(2 w_k))
 * then, per flags, bit 0: signed square root of every value; bit 1: L2
 * normalisation of each set's 2 K D values.  fv (B, 2 K D) float32 out.  A
 * component with w_k <= 0 or a variance <= 0 gives zeros; N = 0 gives zeros.
 * The statistics are those of gmm_estep_stats (float64); the window is its
 * diagonal one.  Workspace: gmm_fisher_vector_workspace_bytes (it holds the
 * model replicated per set and the sets' statistics).  Deterministic. */
size_t gmm_fisher_vector_workspace_bytes(const gmm_data* data, int32_t K);
gmm_status gmm_fisher_vector(const gmm_data* data, const gmm_params* model, uint32_t flags, float* fv, void* ws,
                             size_t ws_bytes, void* stream);

/* Gaussian kernel density estimate (Flash-GMM's closing discussion names
 * kernel density estimation as another user of the fused log-sum-exp): for
 * each query row y (queries as (B, N, D) float32, D <= 128) and the M
 * reference rows x_j of ref ((M, D) float32, row j at ref[j * ld_ref], any
 * alignment), with bandwidth h,
 *   logdens[b N + i] = log( (1/M) sum_j N(y_bi | x_j, h^2 I) )
 *                    = LSE_j(-|y - x_j|^2 / (2 h^2)) - log M - (D/2) log(2 pi h^2),
 * float32 out (B, N); the references are shared by every problem.  The
 * cross terms run in float32 on the matrix cores after the references are
 * centred at their mean; the terms within 2^-30 of a row's largest are then
 * recomputed in float64 from direct differences (up to 8 per row), which
 * makes the log density exact to float32 rounding.  A row with more than 8
 * such terms keeps the float32 terms: within about
 *   ln 2 * lam * eps * (2 DP |y - c| |x - c| + |y - c|^2 + |x - c|^2)
 * of exact (lam = log2(e) / (2 h^2), c the reference mean, DP = D rounded up
 * to 16, 32, 64 or 128, eps = 2^-24; the |x - c| of the terms that dominate
 * the sum).  1 <= M <= 2^30, h > 0 with 1 / (2 h^2) finite in float32.  N = 0 returns
 * GMM_OK and launches nothing.  Workspace: gmm_kde_workspace_bytes (the
 * centred references, (M rounded up to 64) * (DP + 1) floats).  Deterministic. */
size_t gmm_kde_workspace_bytes(const gmm_data* queries, int64_t M);
gmm_status gmm_kde_score(const gmm_data* queries, const float* ref, int64_t M, int64_t ld_ref, double bandwidth,
                         float* logdens, void* ws, size_t ws_bytes, void* stream);

/* Host-side summary of a comp_status array that the caller copied to host
 * memory (count int32 values, as written by gmm_mstep / gmm_fit_step /
 * gmm_topk_fit_step): GMM_ERR_NOT_PD if any component carries flag 2 (its
 * updated covariance was not positive definite) or flag 4 (its input
 * covariance was not), else GMM_OK; GMM_ERR_INVALID_ARG for a NULL array or
 * count < 0.  *first (nullable) receives the index of the first such
 * component, or -1.  No HIP call.  The compute calls cannot return
 * GMM_ERR_NOT_PD themselves: detecting it would need a device-to-host
 * synchronisation in every call. */
gmm_status gmm_check_components(const int32_t* comp_status_host, int64_t count, int64_t* first);

/* Static description of a status code. */
const char* gmm_status_str(int32_t status);

/* Message describing the last failed call on the calling thread ("" if none). */
const char* gmm_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t gmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GMM_H */
