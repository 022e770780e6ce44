// gmm_internal.h -- launch plan and kernel entry points shared by the host
// side of the library (gmm_api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gmm {

enum Cov { SPH = 0, DIAG = 1, TIED = 2, FULL = 3 };

constexpr int kNumCU = 256;          // MI355X compute units (8 XCDs x 32)
constexpr size_t kLdsBytes = 163840; // LDS per workgroup on gfx950
constexpr int kMaxWaves = 8;         // waves per workgroup (512 threads)
constexpr int kBlockedMaxK = 8192;   // float32-path spherical / diagonal components in blocks, at most
constexpr int64_t kBlockedChunk = 1 << 20;  // rows per chunk of the blocked E-step
constexpr size_t kAlign = 256;

// Number of logit features F and statistic rows G for a covariance type and a
// padded dimension DP (both multiples of 16).
//   spherical: phi = x                          (the |x|^2 term is added on the VALU)
//   diag:      phi = [x, x*x]
//   full:      phi = [x, x_d x_e (d <= e)]       (upper triangle, row-major)
//   tied:      same features as full; the quadratic weights are shared by all k
__host__ __device__ constexpr int quad_count(int dp) { return dp * (dp + 1) / 2; }
__host__ __device__ constexpr int round16(int v) { return (v + 15) / 16 * 16; }
__host__ __device__ constexpr int feat_F(int cov, int dp) {
  return cov == DIAG ? 2 * dp : (cov == FULL || cov == TIED) ? round16(dp + quad_count(dp)) : dp;
}
__host__ __device__ constexpr int feat_G(int cov, int dp) { return feat_F(cov, dp); }
// LDS row stride (floats) of the feature tile: >= F and == 2 (mod 32), which
// keeps the MFMA A-operand reads of the logit step free of bank conflicts.
__host__ __device__ constexpr int feat_stride(int f) { return (f + 29) / 32 * 32 + 2; }

struct Plan {
  int cov = 0, dtype = 0;
  int64_t B = 0, N = 0, D = 0, K = 0, ld_x = 0, stride_b = 0;
  int DP = 0, F = 0, G = 0, FS = 0;
  int KW = 0, NW = 0, KP = 0, T = 0;
  int PR = 0;               // doubles per component in a workgroup partial: [N_k, Q_k, G rows]
  int Gb = 0;               // workgroups per problem
  int llG = 0;              // log-likelihood partials per problem
  int op = 0;               // GMM_OP_* the plan was made for
  bool largek = false;      // spherical bf16 rows through the slice-parallel three-pass E-step
  int S = 0;                // 256-component slices (large K, pass A)
  int SC = 0;               // 128-component slices (large K, pass C)
  int GbA = 0;              // row groups of pass A (pass C uses Gb)
  int64_t chunk_rows = 0;   // rows per chunk (large K)
  int lse_blocks = 0;       // blocks of the large-K LSE pass
  size_t lds_a = 0, lds_t = 0, lds_c = 0;
  size_t off_W32 = 0, off_P = 0, off_lse = 0, off_xsq = 0, off_ext = 0, off_eall = 0, off_mmk = 0, off_kconst = 0, off_prem = 0, off_mrow = 0, off_cmask = 0;
  size_t off_lmx = 0, off_kthr = 0;  // large-K top-k: per-(row, slice) lower-bound maxima, per-row threshold
  size_t off_hv = 0;                 // large-K top-m: rows handed to the heavy rescoring kernel
  size_t off_egb = 0;                // large-K top-m: the largest error bound over the components
  size_t off_err = 0;                // small-K top-m: per-component error coefficients (float2)
  int64_t ntiles = 0;       // row tiles per problem (of a row chunk when blocked)
  // fused path with components in blocks (float32-path rows, K above one
  // workgroup): KP, NW and the workspace arrays cover a problem's nblk blocks
  // of KPB components; the rows go in chunks of chunk_rows, each through the
  // (max, sum) pass, the row combine and the statistics pass
  int nblk = 1, KPB = 0;
  bool topm_exact = false;  // top-m of more spherical / diagonal components than the tiled kernel holds
  size_t off_pb = 0, off_lrow = 0;
  size_t lds = 0;           // dynamic LDS of the fused kernel
  bool direct = false;      // tiles of rows can be copied to LDS with 16-byte DMA loads
  // workspace layout (byte offsets)
  size_t off_W = 0, off_prec = 0, off_c0 = 0, off_c = 0, off_a = 0, off_flag = 0, off_sharp = 0, off_part = 0,
         off_llp = 0;
  int prec_stride = 0;      // doubles of precision data per component
  size_t off_nk = 0, off_sx = 0, off_sxx = 0, off_ll = 0, off_aux = 0;
  size_t ws_bytes = 0;
};

struct EStepArgs {
  const void* x;
  int xtype;           // gmm_dtype of the rows (16-bit rows are staged element-wise, decoded to float32)
  int64_t N, D, ld_x, stride_b;
  int K, KP, NW, Gb;
  int64_t ntiles;
  int direct;          // rows of a tile are contiguous and 16-byte aligned (LDS-DMA loads)
  const float* W;      // (B, KP*F) fragment-ordered logit weights (log2 units)
  const double* c;     // (B, KP) logit constants (log2 units), -inf for absent
  const double* a;     // (B, KP) spherical |x|^2 coefficient (log2 units)
  const int32_t* sharp;  // (B, KP) 1: top log-scores of this component are recomputed exactly
  const float* mu;     // (B, K, D) means (the parameters)
  const double* prec;  // (B, KP, prec_stride) precisions / inverse Cholesky factors, float64
  const double* c0;    // (B, KP) log2 pi_k - 1/2 log2 det(2 pi Sigma_k)
  int prec_stride;
  double* part;        // (B*Gb, KPT, PR)
  double* llpart;      // (B*Gb)
  // Components in blocks (more than one workgroup's components): the launch's
  // problem index runs over (problem, block), KP is one block's components and
  // KPT a problem's (the stride of W, c, a, sharp, prec, c0 and the partials);
  // without blocks nblk = 1 and KPT = KP.
  int KPT, nblk;
  int accumulate;      // blocked statistics pass: add to the partials (row chunks after the first)
  int64_t ldl;         // row stride of pb and lrow per problem
  float2* pb;          // blocked (max, sum) pass: (B, ldl, nblk) per row and block, max and sum of 2^(l - max)
  const float2* lrow;  // blocked statistics pass: (B, ldl) per row, its maximum and log2 of its sum over all blocks
};

// spherical E-step for large K and bfloat16 rows (gmm_largek.hip)
constexpr int kLargeKSlice = 256;          // components per workgroup
constexpr int64_t kLargeKChunk = 1 << 20;  // rows per chunk (scratch is O(chunk))

struct LargeKArgs {
  const void* x;        // bf16 rows of the current chunk
  int64_t N, D, ld_x;   // N: rows in the chunk
  int vec16;            // rows can be read with 16-byte loads
  int K, KP, S, G;      // S slices of kLargeKSlice components; G row groups of the launch
  const void* W;        // (KP/16, 2, DP/32, 64, 8) bf16 weights, hi and lo parts, fragment order
  const void* W32;      // (KP/32, 2, DP/16, 64, 8) the same weights in the operand order of the 32x32 MFMA
  const void* W32C;     // (KP/32, 64, 8) bf16: c and a in three terms each, the 32x32 MFMA step that adds
                        // c + a |x|^2 in the barrier-free pass A
  const double* c;      // (KP)
  const double* a;      // (KP)
  const float* mu;      // (K, D) means, for the exact scores of sharp components
  const double* c0;     // (KP) log2(pi_k) - (D log2(2 pi var_k)) / 2
  const double* lam;    // (KP) 1 / var_k
  const float* esh;     // (KP, 2) error bound of the expanded score (0: component not sharp)
  float2* P;            // (chunk, S) per-slice (max, sum)
  float* lse;           // (chunk) row log-sum-exp, log2 units
  double* xsq;          // (chunk) |x|^2 of each row (pass A writes, passes B and C read)
  void* ext;            // (chunk, 8) bf16 per row: 1 and |x|^2 as five bf16 terms, then 0, 0 (pass B
                        // writes for the statistics MFMA of pass C; null when no pass C runs)
  double* llpart;       // (lse blocks)
  double* part;         // (G, KP, 2 + DP)
  int accumulate;       // add to part / llpart (every chunk after the first)
  // top-m
  const float* eall;    // (KP, 2) error bound of every component's expanded score
  const double* mmk;    // (KP) |mu_k|^2
  const double2* kconst; // (KP) (c0 - lambda |mu|^2 log2(e) / 2, lambda log2(e)) for exact scores
  float* prem;          // (chunk, S) below-band mass of each slice, relative to mrow
  float* mrow;          // (chunk) row maximum of the log-scores (pass B)
  uint32_t* cmask;      // (chunk, KP/32) candidate components of each row, one bit per component
  int topm;             // pass B: write mrow
  // one-pass marking of each row's best component alone (fused_t, set by the
  // caller for k-means labels and taken on full-width rows with m = 1 and no
  // counts or log-likelihoods): P.x holds per (row, slice) the slice maximum,
  // egb the largest error bound over every component (slope in |x|^2,
  // offset); the rescoring forms the row maximum and drops far slices
  int fused_t;
  float* egb;           // (2)
  // top-k mode (topk > 0): each row keeps its topk best components, normalised over them
  int topk;
  float4* lmx;          // (chunk, S) per (row, slice): 4 lane-group maxima of (score - error bound), or null
  float* kthr;          // (chunk) per row: a lower bound of its topk-th best score (candidate threshold)
  unsigned char* hv;    // (chunk / 4) rescoring: rows with many candidates, a 4-bit mask per four rows
  int m;
  float thr;
  int32_t* idx;         // outputs of the chunk's rows
  float* resp;
  int32_t* count;
  float* logp;
};
constexpr int64_t kLargeKTopmChunk = 1 << 18;
constexpr int kLargeKMaxK = 16384;     // components of one large-K problem at most
// A component is "sharp" on the large-K path when the terms of its expanded
// log-score reach lambda (|mu|^2 + D sigma^2) > kLargeKSharp: with bf16
// weights (two-term split) their rounding would reach about 1% of a
// responsibility, so its scores near a row's top are recomputed in float64.
constexpr double kLargeKSharp = 2.0e3;
hipError_t launch_largek_topm(const Plan& p, const LargeKArgs& a, const float* w, const float* mu, const float* cv,
                              hipStream_t s);
hipError_t launch_largek(const Plan& p, const LargeKArgs& a, const float* w, const float* mu, const float* cv,
                         hipStream_t s);
size_t largek_lds_bytes(int DP, int pass);  // dynamic LDS of pass A (0) / C (2)

// soft multi-assignment (gmm_topm.hip)
constexpr int kTopmRows = 16;   // rows per tile
constexpr int kTopmCap = 64;    // candidates per row kept in LDS before the all-K path
constexpr int kTopmMaxK = 256;

struct TopmArgs {
  const void* x;
  int xtype;           // gmm_dtype of the rows
  int64_t N, D, ld_x, stride_b;
  int K, KP, NW, Gb;
  int64_t ntiles;
  const float* W;
  const double* c;
  const double* a;
  const float* mu;
  const double* prec;
  const double* c0;
  const float2* err;   // (B, KP) error coefficients of the approximate score: err.x |x| + err.y |x|^2
  int prec_stride;
  int m;
  float thr;
  int topk;            // 1: keep the m best components of every row, normalised over them (no threshold)
  int32_t* idx;
  float* resp;
  int32_t* count;
  float* logp;
};
hipError_t launch_topm(const Plan& p, const TopmArgs& a, hipStream_t s);
// spherical / diagonal problems above kTopmMaxK components: every score
// exactly in float64 (Plan::topm_exact)
hipError_t launch_topm_exact(const Plan& p, const TopmArgs& a, hipStream_t s);

// IVF posting lists from a soft multi-assignment (gmm_ivf.hip)
constexpr int kIvfBlock = 4096;     // rows per walking wave
constexpr int kIvfMaxK = 16384;     // components (one int of LDS each per wave)
struct IvfArgs {
  const int32_t* idx;  // (B,N,m)
  const float* resp;   // (B,N,m) or null
  int64_t N;
  int B, m, K, KB;     // KB: bits of the largest component index
  int nblk;            // row blocks per problem
  int32_t* cnt;        // workspace (B,nblk,K): block counts, then their prefixes
  int64_t* offsets;    // (B,K+1)
  int32_t* rows;       // (B,N*m)
  float* lresp;        // (B,N*m) or null
};
hipError_t launch_ivf_lists(const IvfArgs& a, hipStream_t s);

// k-means (Lloyd) iteration pieces (gmm_kmeans.hip)
hipError_t launch_kmeans_params(int64_t B, int K, int D, const float* C, float* w, float* cv, hipStream_t s);

// approximate top-k EM statistics (gmm_topk.hip)
// approximate top-k EM statistics (gmm_topk.hip)
struct TopkStepArgs {
  const void* x;              // rows, float32, bf16 or half bits
  int xtype;                  // gmm_dtype of the rows
  int64_t B, N, ld_x, stride_b;
  int K, D, m, cov, S;        // S: contiguous parts each component's list is split into
  const float* resp;          // (B, N, m) kept responsibilities (normalised over the kept set), best first
  const float* logp;          // (B, N) log sum over the kept components of pi N(x)
  const float* mu;            // (B, K, D) means entering the step
  const int64_t* offsets;     // (B, K+1) list offsets
  const int32_t* rows;        // (B, N m) list rows
  const float* lresp;         // (B, N m) list responsibilities
  double* rinv;               // (B, N) scratch: 1 / sum of the kept responsibilities
  double* llpart;             // (B, ceil(N / 256)) scratch: per-block row log-likelihoods
  double* part;               // (B, K, S, 1 + 2 D) scratch: per-part statistics
  double *nk, *sx, *sxx;      // (B, K), (B, K, D), (B, K) or (B, K, D)
  double *ll, *mean_ll;       // (B); mean_ll may be null
};
// parts per component list: about 512 entries each on average, at most 64,
// and at most 65536 workgroups over all (problem, component, part)
inline int topk_parts(int64_t B, int64_t N, int m, int K) {
  int64_t S = (N * m / K + 511) / 512;
  if (S > 64) S = 64;
  const int64_t cap = 65536 / (B * K);
  if (S > cap) S = cap;
  return S < 1 ? 1 : (int)S;
}
hipError_t launch_topk_stats(const TopkStepArgs& a, hipStream_t s);

// Gaussian kernel density estimate (gmm_kde.hip)
struct KdeArgs {
  const float* y;            // query rows: problem b, row i, feature d at y[b stride_b + i ld + d]
  int64_t B, N, ld, stride_b;
  int D;
  const float* cen;          // (DP) reference mean, zero past D
  const float* xc;           // (Mp, DP) centred references, zero-padded
  const float* bx;           // (Mp) -lam |x - c|^2, -inf past M
  int64_t Mp;                // references padded to whole tiles
  double lam;                // log2(e) / (2 h^2), the float32 value widened
  float s2;                  // 2 lam
  double lam_exact;          // log2(e) / (2 h^2) in float64, for the exact rescoring
  const float* ref;          // the caller's references, row j at ref[j ld_ref]
  int64_t ld_ref;
  double cnst;               // -log M - (D / 2) log(2 pi h^2)
  float* out;                // (B, N) log densities
};
int kde_query_rows();        // query rows per workgroup
int kde_tile_rows();         // reference rows per tile (Mp is a multiple)
hipError_t launch_kde_prep(const float* x, int64_t M, int64_t ld, int D, int DP, int64_t Mp, double lam, float* cen,
                           float* xc, float* bx, hipStream_t s);
hipError_t launch_kde(const KdeArgs& a, int DP, hipStream_t s);

// Fisher vectors (gmm_fisher.hip)
hipError_t launch_fisher_replicate(int64_t B, int K, int D, const float* w, const float* mu, const float* var,
                                   float* wr, float* mur, float* varr, hipStream_t s);
hipError_t launch_fisher(int64_t B, int K, int D, int64_t N, uint32_t flags, const float* w, const float* mu,
                         const float* var, const double* nk, const double* sx, const double* sxx, float* fv,
                         hipStream_t s);
hipError_t launch_kmeans_update(const void* x, int xtype, int64_t B, int64_t N, int64_t ld_x, int64_t stride_b, int K,
                                int D, const int64_t* offsets, const int32_t* rows, float* C, int64_t* counts,
                                double* ip, double* inertia, hipStream_t s);

// fused E-step + statistics (gmm_estep.hip)
hipError_t launch_estep(const Plan& p, const EStepArgs& a, hipStream_t s);
// blocked components: mode 1 the per-(row, block) (max, sum) pass, 2 the
// statistics pass against the rows' combined maxima and sums (grid over
// B * nblk * Gb workgroups); the row combine between them
hipError_t launch_estep_blocked(const Plan& p, const EStepArgs& a, int mode, hipStream_t s);
hipError_t launch_block_combine(int64_t B, int64_t N, int nblk, int64_t ldl, int Gb, const float2* pb, float2* lrow,
                                double* llpart, int accumulate, hipStream_t s);
bool estep_variant_exists(int cov, int dp, int kw, int t);

// prologue / reduction / M-step (gmm_aux.hip)
hipError_t launch_prologue(const Plan& p, const float* w, const float* mu, const float* cv, float2* err, float* W,
                           double* prec, double* c0, double* c, double* a, int32_t* flag, int32_t* sharp,
                           hipStream_t s);
hipError_t launch_mean_ll(int64_t B, const double* ll, int64_t n_total, double* mean_ll, hipStream_t s);
// The M-step fused into the statistics reduction (spherical, diag, full;
// not when accumulating): w == nullptr means no M-step.
// The prologue outputs of a fit step's workspace (log-score weights and
// constants), for an M-step that forms the next iteration's prologue right
// after the parameters (W null: it does not).
struct PrologueOut {
  int DP, F, KW, KP, prec_stride;
  float* W;
  double* prec;
  double* c0;
  double* c;
  double* a;
  int32_t* flag;
  int32_t* sharp;
};
struct MstepFuse {
  float* w;
  float* mu;
  float* cv;
  int64_t n_total;
  double reg;
  const int32_t* in_flag;
  int in_flag_stride;
  int32_t* comp_status;
  PrologueOut next;
};
hipError_t launch_reduce_raw(const Plan& p, const double* part, const double* llpart, const float* mu,
                             double* raw, double* nk, double* sx, double* sxx, double* ll, double* mean_ll,
                             int accumulate, hipStream_t s, const MstepFuse* fuse = nullptr);
hipError_t launch_mstep_strided(int cov, int64_t B, int64_t D, int64_t K, const double* nk, const double* sx,
                                const double* sxx, int64_t n_total, float* w, float* mu, float* cv, double reg,
                                const int32_t* in_flag, int in_flag_stride, int32_t* comp_status, hipStream_t s);

}  // namespace gmm
