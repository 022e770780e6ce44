// gmm_api.hip -- the C ABI declared in include/gmm.h: argument validation,
// the launch plan (tiling, workgroup count, workspace layout) and the kernel
// sequence of each entry point.
#include "gmm.h"
#include "gmm_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>

namespace gmm {

static thread_local std::string g_err;

static gmm_status fail(gmm_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static gmm_status fail(gmm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

static size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

static int64_t cov_len(int cov, int64_t D, int64_t K) {
  switch (cov) {
    case SPH: return K;
    case DIAG: return K * D;
    case TIED: return D * D;
    default: return K * D * D;
  }
}

static gmm_status check_data(const gmm_data* d) {
  if (!d) return fail(GMM_ERR_INVALID_ARG, "data descriptor is NULL");
  if (d->B < 1 || d->N < 0 || d->D < 1)
    return fail(GMM_ERR_INVALID_ARG, "need B >= 1, N >= 0, D >= 1 (got B=%lld N=%lld D=%lld)", (long long)d->B,
                (long long)d->N, (long long)d->D);
  if (d->ld_x < d->D) return fail(GMM_ERR_INVALID_ARG, "ld_x (%lld) < D (%lld)", (long long)d->ld_x, (long long)d->D);
  if (d->B > 1 && d->stride_b < d->N * d->ld_x)
    return fail(GMM_ERR_INVALID_ARG, "stride_b (%lld) < N*ld_x", (long long)d->stride_b);
  if (d->N > 0 && !d->x) return fail(GMM_ERR_INVALID_ARG, "x is NULL");
  if (d->dtype != GMM_DT_F32 && d->dtype != GMM_DT_BF16 && d->dtype != GMM_DT_F16)
    return fail(GMM_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (d->N > ((int64_t)1 << 40)) return fail(GMM_ERR_UNSUPPORTED, "N too large");
  return GMM_OK;
}

static gmm_status check_params(const gmm_params* p, int64_t B, int64_t D, bool need_ptrs) {
  if (!p) return fail(GMM_ERR_INVALID_ARG, "params descriptor is NULL");
  if (p->K < 1) return fail(GMM_ERR_INVALID_ARG, "K must be >= 1 (got %d)", p->K);
  if (p->cov < SPH || p->cov > FULL) return fail(GMM_ERR_INVALID_ARG, "unknown covariance type %d", p->cov);
  if (need_ptrs && (!p->weights || !p->means || !p->covars))
    return fail(GMM_ERR_INVALID_ARG, "weights/means/covars must be non-NULL");
  (void)B;
  (void)D;
  return GMM_OK;
}

// Workspace of the large-K E-step for chunks of `chunk` rows (a multiple of
// the 32-row tile): weights and constants, per-(row, slice) maxima and sums,
// row LSE, statistics partials, and (fit) the reduced statistics.
static void largek_layout(Plan& q, int64_t chunk) {
  q.chunk_rows = chunk;
  size_t o = 0;
  q.off_W = o;    o = align_up(o + (size_t)q.KP * q.DP * 2 * 2);
  q.off_W32 = o;  o = align_up(o + (size_t)q.KP * q.DP * 2 * 2 + (size_t)q.KP * 32);
  q.off_c = o;    o = align_up(o + sizeof(double) * (size_t)q.KP);
  q.off_a = o;    o = align_up(o + sizeof(double) * (size_t)q.KP);
  q.off_c0 = o;   o = align_up(o + sizeof(double) * (size_t)q.KP);
  q.off_prec = o; o = align_up(o + sizeof(double) * (size_t)q.KP);
  q.off_sharp = o; o = align_up(o + sizeof(float) * 2 * (size_t)q.KP);
  q.off_eall = o; o = align_up(o + sizeof(float) * 2 * (size_t)q.KP);
  q.off_mmk = o;  o = align_up(o + sizeof(double) * (size_t)q.KP);
  q.off_kconst = o; o = align_up(o + sizeof(double) * 2 * (size_t)q.KP);
  q.off_P = o;    o = align_up(o + sizeof(float) * 2 * (size_t)chunk * q.S);
  q.off_lse = o;  o = align_up(o + sizeof(float) * (size_t)chunk);
  q.off_xsq = o;  o = align_up(o + sizeof(double) * (size_t)chunk);
  q.off_ext = 0;
  if (q.op != GMM_OP_TOPM) {
    q.off_ext = o; o = align_up(o + 16 * (size_t)chunk);
  }
  if (q.op == GMM_OP_TOPM) {
    q.off_mrow = o; o = align_up(o + sizeof(float) * (size_t)chunk);
    q.off_cmask = o; o = align_up(o + sizeof(uint32_t) * (size_t)chunk * (q.KP / 32));
    q.off_prem = o; o = align_up(o + sizeof(float) * (size_t)chunk * q.S);
    q.off_lmx = o;  o = align_up(o + sizeof(float) * 4 * (size_t)chunk * q.S);
    q.off_kthr = o; o = align_up(o + sizeof(float) * (size_t)chunk);
    q.off_hv = o;   o = align_up(o + (size_t)chunk / 4 + 1);
    q.off_egb = o;  o = align_up(o + 2 * sizeof(float));
  }
  q.off_part = o; o = align_up(o + sizeof(double) * (size_t)q.Gb * q.KP * q.PR);
  q.off_llp = o;  o = align_up(o + sizeof(double) * (size_t)q.llG);
  q.off_aux = o;  o = align_up(o + sizeof(double) * (size_t)q.KP * q.PR);
  if (q.op == GMM_OP_FIT) {
    q.off_nk = o;  o = align_up(o + sizeof(double) * (size_t)q.K);
    q.off_sx = o;  o = align_up(o + sizeof(double) * (size_t)q.K * q.D);
    q.off_sxx = o; o = align_up(o + sizeof(double) * (size_t)q.K);
    q.off_ll = o;  o = align_up(o + sizeof(double));
  }
  q.ws_bytes = o;
}

// Choose the tiling of the fused kernel and lay out the workspace.
static gmm_status make_plan(const gmm_data* d, int K, int cov, int op, Plan* p) {
  gmm_status st = check_data(d);
  if (st != GMM_OK) return st;
  if (K < 1) return fail(GMM_ERR_INVALID_ARG, "K must be >= 1");
  if (cov < SPH || cov > FULL) return fail(GMM_ERR_INVALID_ARG, "unknown covariance type %d", cov);
  Plan q;
  q.cov = cov;
  q.dtype = d->dtype;
  q.B = d->B;
  q.N = d->N;
  q.D = d->D;
  q.K = K;
  q.ld_x = d->ld_x;
  q.stride_b = d->B > 1 ? d->stride_b : 0;
  if (d->dtype == GMM_DT_BF16 && cov == SPH && d->B == 1) {
    // bf16 rows of one problem with spherical components: the slice-parallel
    // three-pass E-step (any K; x is exact in the bf16 MFMA operand).  Other
    // 16-bit cases take the fused path below, the rows decoded to float32.
    if (d->D > 128) return fail(GMM_ERR_UNSUPPORTED, "bf16 rows: D <= 128");
    if (K > kLargeKMaxK) return fail(GMM_ERR_UNSUPPORTED, "bf16 rows: K <= %d", kLargeKMaxK);
    q.largek = true;
    q.DP = 128;
    q.F = q.G = q.DP;
    q.PR = 2 + q.G;
    q.KW = 32;
    q.NW = kLargeKSlice / 32;
    q.S = (K + kLargeKSlice - 1) / kLargeKSlice;
    q.KP = q.S * kLargeKSlice;
    q.T = 32;
    q.SC = q.KP / (kLargeKSlice / 2);
    // row groups: about one workgroup per CU; a multiple of 8 keeps a row
    // group's slices on one XCD
    q.GbA = (std::max(1, kNumCU / q.S) + 7) / 8 * 8;
    q.Gb = (std::max(1, kNumCU / q.SC) + 7) / 8 * 8;
    q.lse_blocks = 512;
    q.llG = q.lse_blocks;
    q.ntiles = (q.N + 31) / 32;
    q.lds_a = largek_lds_bytes(q.DP, 0);
    q.lds_t = largek_lds_bytes(q.DP, 1);
    q.lds_c = largek_lds_bytes(q.DP, 2);
    q.prec_stride = 1;
    q.op = op;
    largek_layout(q, std::min<int64_t>((q.N + 31) / 32 * 32, op == GMM_OP_TOPM ? kLargeKTopmChunk : kLargeKChunk));
    *p = q;
    return GMM_OK;
  }
  if (cov == SPH || cov == DIAG) {
    q.DP = d->D <= 16 ? 16 : d->D <= 32 ? 32 : d->D <= 64 ? 64 : d->D <= 128 ? 128 : 0;
  } else {
    q.DP = d->D <= 8 ? 8 : d->D <= 16 ? 16 : 0;
  }
  if (!q.DP)
    return fail(GMM_ERR_UNSUPPORTED, "D=%lld is outside the supported window for this covariance type",
                (long long)d->D);
  q.F = feat_F(cov, q.DP);
  q.G = feat_G(cov, q.DP);
  q.FS = feat_stride(std::max(q.F, q.G));
  q.PR = 2 + q.G;
  const bool direct_ok = d->dtype == GMM_DT_F32 && (((uintptr_t)d->x) % 16 == 0) && (q.ld_x == q.D) &&
                         (q.D % 4 == 0) && (q.stride_b % 4 == 0);
  auto lds_for = [&](int T, int nraw) {
    // weights, feature tile, raw row tile(s), |x|^2 (float64), per-wave (max, sum), product table
    return sizeof(float) * ((size_t)q.KP * q.F + (size_t)T * q.FS + (size_t)nraw * T * q.DP + 2 * (size_t)T +
                            2 * (size_t)q.NW * T + q.F);
  };
  // Components per wave: 16 gives more waves per workgroup; from K = 64 on,
  // spherical and diagonal E-steps take 32 where a tile fits, so each feature
  // operand read from LDS feeds two MFMA column tiles (diag_batched: 1.65 ->
  // 1.34 ms per E-step).  The top-m tiling keeps 16 first.
  int kws[2] = {16, 32};
  if (op != GMM_OP_TOPM && K >= 64 && (cov == SPH || cov == DIAG)) {
    kws[0] = 32;
    kws[1] = 16;
  }
  if (op == GMM_OP_TOPM && K > kTopmMaxK && (cov == SPH || cov == DIAG)) {
    // top-m of more components than the tiled kernel holds: the exact kernel
    // (every score in float64); the prologue's layout with 32 per wave
    if (K > kBlockedMaxK) return fail(GMM_ERR_UNSUPPORTED, "top-m: K=%d above %d", K, kBlockedMaxK);
    q.topm_exact = true;
    q.op = op;
    q.KW = 32;
    q.NW = (K + 31) / 32;
    q.KP = q.KW * q.NW;
    q.T = 256;
    q.Gb = 1;
    q.llG = 1;
    q.ntiles = (q.N + 255) / 256;
    q.KPB = q.KP;
    q.chunk_rows = q.N;
    size_t o = 0;
    q.off_W = o;    o = align_up(o + sizeof(float) * (size_t)q.B * q.KP * q.F);
    q.prec_stride = (cov == SPH) ? 1 : (int)q.D;
    q.off_prec = o; o = align_up(o + sizeof(double) * (size_t)q.B * q.KP * q.prec_stride);
    q.off_c0 = o;   o = align_up(o + sizeof(double) * (size_t)q.B * q.KP);
    q.off_c = o;    o = align_up(o + sizeof(double) * (size_t)q.B * q.KP);
    q.off_a = o;    o = align_up(o + sizeof(double) * (size_t)q.B * q.KP);
    q.off_flag = o; o = align_up(o + sizeof(int32_t) * (size_t)q.B * q.KP);
    q.off_sharp = o; o = align_up(o + sizeof(int32_t) * (size_t)q.B * q.KP);
    q.off_err = o;  o = align_up(o + sizeof(float2) * (size_t)q.B * q.KP);
    q.ws_bytes = o;
    *p = q;
    return GMM_OK;
  }
  // more spherical / diagonal components than one workgroup's tiling holds:
  // blocks of kMaxWaves waves, the rows' normaliser over every block
  // (launch_estep_blocked)
  const bool can_block = op != GMM_OP_TOPM && (cov == SPH || cov == DIAG);
  bool blocked = false;
  bool waves_ok = false;
  for (int attempt = 0; attempt < 2 && !q.T; ++attempt) {
    blocked = attempt == 1;
    if (blocked && !can_block) break;
    for (int kw : kws) {
      const int Kc = blocked ? kw * kMaxWaves : K;  // components of one workgroup
      if ((Kc + kw - 1) / kw > kMaxWaves) continue;
      waves_ok = true;
      q.KW = kw;
      q.NW = (Kc + q.KW - 1) / q.KW;
      q.KP = q.KW * q.NW;
      if (op == GMM_OP_TOPM) {
        if (K > kTopmMaxK) return fail(GMM_ERR_UNSUPPORTED, "top-m supports K <= %d", kTopmMaxK);
        const size_t T = kTopmRows, C = kTopmCap;
        q.T = (int)T;
        q.direct = false;
        q.lds = sizeof(float) * ((size_t)q.KP * q.F + T * q.FS + T * q.DP + T * C + (size_t)q.NW * T + T + q.F + 3 * T) +
                sizeof(double) * (T + (size_t)q.NW * T + T * C);
        if (q.lds > kLdsBytes)
          return fail(GMM_ERR_UNSUPPORTED, "K=%d x D=%lld top-m tile does not fit in LDS", K, (long long)d->D);
        break;
      }
      // largest tile that fits: double-buffered asynchronous row loads first, then one synchronous buffer
      for (int nraw : {2, 1}) {
        if (nraw == 2 && !direct_ok) continue;
        for (int T : {64, 32, 16}) {
          if (lds_for(T, nraw) <= kLdsBytes && estep_variant_exists(cov, q.DP, q.KW, T)) {
            q.T = T;
            q.direct = nraw == 2;
            break;
          }
        }
        if (q.T) break;
      }
      if (q.T) break;
    }
  }
  if (!waves_ok) return fail(GMM_ERR_UNSUPPORTED, "K=%d is above the single-pass window (<= %d)", K, 32 * kMaxWaves);
  if (!q.T) return fail(GMM_ERR_UNSUPPORTED, "K=%d x D=%lld does not fit in LDS", K, (long long)d->D);
  if (op != GMM_OP_TOPM) q.lds = lds_for(q.T, q.direct ? 2 : 1);
  q.KPB = q.KP;
  q.chunk_rows = q.N;
  if (blocked) {
    if (K > kBlockedMaxK) return fail(GMM_ERR_UNSUPPORTED, "K=%d: spherical / diagonal components <= %d", K, kBlockedMaxK);
    q.nblk = (K + q.KPB - 1) / q.KPB;
    q.KP = q.nblk * q.KPB;
    // rows in chunks (the per-row block maxima and sums are O(chunk)); a
    // multiple of 4 keeps the chunks' float32 rows 16-byte aligned
    q.chunk_rows = std::min<int64_t>((q.N + 3) / 4 * 4, kBlockedChunk);
  }
  q.ntiles = (q.chunk_rows + q.T - 1) / q.T;
  const int wg_lds = (int)std::max<size_t>(1, kLdsBytes / q.lds);
  const int wg_per_cu = std::max(1, std::min(wg_lds, 8 / q.NW));
  const int64_t total = (int64_t)kNumCU * wg_per_cu;
  int64_t gb = std::max<int64_t>(1, total / (q.B * q.nblk));
  gb = std::min<int64_t>(gb, std::max<int64_t>(1, q.ntiles));
  q.Gb = (int)gb;
  q.llG = q.Gb;
  // workspace
  size_t o = 0;
  q.off_W = o;    o = align_up(o + sizeof(float) * (size_t)q.B * q.KP * q.F);
  // full / tied: L^{-1} as DP x DP, zero past D (the exact score runs over DP)
  q.prec_stride = (cov == SPH) ? 1 : (cov == DIAG) ? (int)q.D : q.DP * q.DP;
  q.off_prec = o; o = align_up(o + sizeof(double) * (size_t)q.B * q.KP * q.prec_stride);
  q.off_c0 = o;   o = align_up(o + sizeof(double) * (size_t)q.B * q.KP);
  q.off_c = o;    o = align_up(o + sizeof(double) * (size_t)q.B * q.KP);
  q.off_a = o;    o = align_up(o + sizeof(double) * (size_t)q.B * q.KP);
  q.off_flag = o; o = align_up(o + sizeof(int32_t) * (size_t)q.B * q.KP);
  q.off_sharp = o; o = align_up(o + sizeof(int32_t) * (size_t)q.B * q.KP);
  q.off_err = o;  o = align_up(o + sizeof(float2) * (size_t)q.B * q.KP);
  if (op != GMM_OP_TOPM) {
    q.off_part = o; o = align_up(o + sizeof(double) * (size_t)q.B * q.Gb * q.KP * q.PR);
    q.off_llp = o;  o = align_up(o + sizeof(double) * (size_t)q.B * q.Gb);
    q.off_aux = o;  o = align_up(o + sizeof(double) * (size_t)q.B * q.KP * q.PR);
  }
  if (q.nblk > 1) {
    q.off_pb = o;   o = align_up(o + sizeof(float2) * (size_t)q.B * q.chunk_rows * q.nblk);
    q.off_lrow = o; o = align_up(o + sizeof(float2) * (size_t)q.B * q.chunk_rows);
  }
  if (op == GMM_OP_FIT) {
    q.off_nk = o;  o = align_up(o + sizeof(double) * (size_t)q.B * K);
    q.off_sx = o;  o = align_up(o + sizeof(double) * (size_t)q.B * K * q.D);
    q.off_sxx = o; o = align_up(o + sizeof(double) * (size_t)q.B * cov_len(cov, q.D, K));
    q.off_ll = o;  o = align_up(o + sizeof(double) * (size_t)q.B);
  }
  q.ws_bytes = o;
  *p = q;
  return GMM_OK;
}

// Whether ws_bytes of workspace hold the plan (the large-K path then streams
// its rows in chunks that fit); host-only.
static gmm_status fit_ws(Plan& p, size_t ws_bytes) {
  if (p.largek && ws_bytes < p.ws_bytes) {
    // a smaller workspace streams the rows in shorter chunks (multiples of 32 rows)
    Plan q = p;
    largek_layout(q, 32);
    if (ws_bytes >= q.ws_bytes) {
      size_t per_row = sizeof(float) * (2 * (size_t)p.S + 1) + sizeof(double);
      if (p.op != GMM_OP_TOPM) per_row += 16;
      if (p.op == GMM_OP_TOPM) per_row += sizeof(float) * (2 + 5 * (size_t)p.S) + sizeof(uint32_t) * (p.KP / 32) + 1;
      int64_t chunk = (int64_t)((ws_bytes - q.ws_bytes) / per_row) / 32 * 32 + 32;
      chunk = std::min<int64_t>(chunk, p.chunk_rows);
      for (largek_layout(q, chunk); q.ws_bytes > ws_bytes && chunk > 32; largek_layout(q, chunk)) chunk -= 32;
      if (q.ws_bytes <= ws_bytes) {
        p = q;
        return GMM_OK;
      }
    }
  }
  if (ws_bytes < p.ws_bytes)
    return fail(GMM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, p.ws_bytes);
  return GMM_OK;
}

static gmm_status check_ws(Plan& p, void* ws, size_t ws_bytes) {
  if (!ws) return fail(GMM_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)ws) % kAlign) return fail(GMM_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  return fit_ws(p, ws_bytes);
}

static gmm_status hip_fail(hipError_t e, const char* where) {
  return fail(GMM_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ---- allocation-free fit step: its workspace is this file-scope device array
// (one copy per GPU, alive until the process ends).  Host code never passes
// the array's name to a kernel -- on the host that name is a stand-in, not a
// device address -- but the address hipGetSymbolAddress returns for the
// current device, fetched once per device.
static constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static void* scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

// prologue + fused E-step + reduction; statistics to the given buffers
static LargeKArgs largek_args(const Plan& p, const gmm_data* d, const gmm_params* prm, void* ws) {
  char* w = static_cast<char*>(ws);
  LargeKArgs A{};
  A.x = d->x;
  A.N = p.N;
  A.D = p.D;
  A.ld_x = p.ld_x;
  A.vec16 = (((uintptr_t)d->x) % 16 == 0) && (p.ld_x % 8 == 0);
  A.K = (int)p.K;
  A.KP = p.KP;
  A.S = p.S;
  A.G = p.Gb;
  A.W = w + p.off_W;
  A.W32 = w + p.off_W32;
  A.W32C = w + p.off_W32 + (size_t)p.KP * p.DP * 2 * 2;
  A.c = reinterpret_cast<double*>(w + p.off_c);
  A.a = reinterpret_cast<double*>(w + p.off_a);
  A.mu = prm->means;
  A.c0 = reinterpret_cast<double*>(w + p.off_c0);
  A.lam = reinterpret_cast<double*>(w + p.off_prec);
  A.esh = reinterpret_cast<float*>(w + p.off_sharp);
  A.P = reinterpret_cast<float2*>(w + p.off_P);
  A.lse = reinterpret_cast<float*>(w + p.off_lse);
  A.xsq = reinterpret_cast<double*>(w + p.off_xsq);
  A.ext = p.off_ext ? static_cast<void*>(w + p.off_ext) : nullptr;
  A.llpart = reinterpret_cast<double*>(w + p.off_llp);
  A.part = reinterpret_cast<double*>(w + p.off_part);
  A.accumulate = 0;
  A.eall = reinterpret_cast<float*>(w + p.off_eall);
  A.mmk = reinterpret_cast<double*>(w + p.off_mmk);
  A.kconst = reinterpret_cast<double2*>(w + p.off_kconst);
  if (p.op == GMM_OP_TOPM) {
    A.mrow = reinterpret_cast<float*>(w + p.off_mrow);
    A.cmask = reinterpret_cast<uint32_t*>(w + p.off_cmask);
    A.prem = reinterpret_cast<float*>(w + p.off_prem);
    A.lmx = reinterpret_cast<float4*>(w + p.off_lmx);
    A.kthr = reinterpret_cast<float*>(w + p.off_kthr);
    A.hv = reinterpret_cast<unsigned char*>(w + p.off_hv);
    A.egb = reinterpret_cast<float*>(w + p.off_egb);
  }
  return A;
}

static gmm_status run_estep_largek(const Plan& p, const gmm_data* d, const gmm_params* prm, void* ws, double* nk,
                                   double* sx, double* sxx, double* ll, double* mean_ll, int accumulate,
                                   const gmm_options* opts, hipStream_t s, const MstepFuse* fuse) {
  char* w = static_cast<char*>(ws);
  LargeKArgs A = largek_args(p, d, prm, ws);
  hipError_t e;
  if (opts && opts->event_begin && (e = hipEventRecord((hipEvent_t)opts->event_begin, s)) != hipSuccess)
    return hip_fail(e, "event record");
  e = launch_largek(p, A, prm->weights, prm->means, prm->covars, s);
  if (e != hipSuccess) return hip_fail(e, "large-K E-step launch");
  if (opts && opts->event_end && (e = hipEventRecord((hipEvent_t)opts->event_end, s)) != hipSuccess)
    return hip_fail(e, "event record");
  e = launch_reduce_raw(p, A.part, A.llpart, prm->means, reinterpret_cast<double*>(w + p.off_aux), nk, sx, sxx, ll,
                        mean_ll, accumulate, s, fuse);
  if (e != hipSuccess) return hip_fail(e, "reduction launch");
  return GMM_OK;
}

// fuse (nullable): the M-step of gmm_fit_step, run by the reduction's
// component blocks (spherical, diag, full).  skip_prologue: the workspace
// already holds this step's prologue (formed by the previous step's M-step).
static gmm_status run_estep(const Plan& p, const gmm_data* d, const gmm_params* prm, void* ws, double* nk, double* sx,
                            double* sxx, double* ll, double* mean_ll, int accumulate, const gmm_options* opts,
                            hipStream_t s, const MstepFuse* fuse = nullptr, bool skip_prologue = false) {
  if (p.largek) return run_estep_largek(p, d, prm, ws, nk, sx, sxx, ll, mean_ll, accumulate, opts, s, fuse);
  char* w = static_cast<char*>(ws);
  float* W = reinterpret_cast<float*>(w + p.off_W);
  double* prec = reinterpret_cast<double*>(w + p.off_prec);
  double* c0 = reinterpret_cast<double*>(w + p.off_c0);
  int32_t* sharp = reinterpret_cast<int32_t*>(w + p.off_sharp);
  double* c = reinterpret_cast<double*>(w + p.off_c);
  double* a = reinterpret_cast<double*>(w + p.off_a);
  int32_t* flag = reinterpret_cast<int32_t*>(w + p.off_flag);
  double* part = reinterpret_cast<double*>(w + p.off_part);
  double* llp = reinterpret_cast<double*>(w + p.off_llp);
  double* raw = reinterpret_cast<double*>(w + p.off_aux);
  hipError_t e = hipSuccess;
  if (!skip_prologue) {
    e = launch_prologue(p, prm->weights, prm->means, prm->covars, nullptr, W, prec, c0, c, a, flag, sharp, s);
    if (e != hipSuccess) return hip_fail(e, "prologue launch");
  }
  EStepArgs A;
  A.x = d->x;
  A.xtype = p.dtype;
  A.N = p.N;
  A.D = p.D;
  A.ld_x = p.ld_x;
  A.stride_b = p.stride_b;
  A.K = (int)p.K;
  A.KP = p.KP;
  A.NW = p.NW;
  A.Gb = p.Gb;
  A.ntiles = p.ntiles;
  A.direct = p.direct ? 1 : 0;
  A.W = W;
  A.mu = prm->means;
  A.prec = prec;
  A.c0 = c0;
  A.prec_stride = p.prec_stride;
  A.sharp = sharp;
  A.c = c;
  A.a = a;
  A.part = part;
  A.llpart = llp;
  A.KPT = p.KP;
  A.nblk = 1;
  A.accumulate = 0;
  A.ldl = 0;
  A.pb = nullptr;
  A.lrow = nullptr;
  if (opts && opts->event_begin) {
    e = hipEventRecord((hipEvent_t)opts->event_begin, s);
    if (e != hipSuccess) return hip_fail(e, "event record");
  }
  if (p.nblk > 1) {
    // components in blocks: per chunk of rows the (max, sum) pass, the row
    // combine and the statistics pass, the chunks' partials added up
    A.KP = p.KPB;
    A.nblk = p.nblk;
    A.ldl = p.chunk_rows;
    A.pb = reinterpret_cast<float2*>(w + p.off_pb);
    float2* lrow = reinterpret_cast<float2*>(w + p.off_lrow);
    A.lrow = lrow;
    const size_t esz = p.dtype == GMM_DT_F32 ? 4 : 2;
    for (int64_t r0 = 0; r0 < p.N; r0 += p.chunk_rows) {
      const int64_t rows = std::min<int64_t>(p.chunk_rows, p.N - r0);
      A.x = static_cast<const char*>(d->x) + (size_t)r0 * p.ld_x * esz;
      A.N = rows;
      A.ntiles = (rows + p.T - 1) / p.T;
      A.accumulate = r0 > 0;
      if ((e = launch_estep_blocked(p, A, 1, s)) != hipSuccess) return hip_fail(e, "blocked E-step (max, sum) launch");
      if ((e = launch_block_combine(p.B, rows, p.nblk, p.chunk_rows, p.Gb, A.pb, lrow, llp, r0 > 0, s)) != hipSuccess)
        return hip_fail(e, "blocked E-step row combine launch");
      if ((e = launch_estep_blocked(p, A, 2, s)) != hipSuccess) return hip_fail(e, "blocked E-step statistics launch");
    }
  } else {
    e = launch_estep(p, A, s);
    if (e != hipSuccess) return hip_fail(e, "fused E-step launch");
  }
  if (opts && opts->event_end) {
    e = hipEventRecord((hipEvent_t)opts->event_end, s);
    if (e != hipSuccess) return hip_fail(e, "event record");
  }
  e = launch_reduce_raw(p, part, llp, prm->means, raw, nk, sx, sxx, ll, mean_ll, accumulate, s, fuse);
  if (e != hipSuccess) return hip_fail(e, "reduction launch");
  return GMM_OK;
}

// The top-m launch sequence of a planned call (N >= 1, workspace checked).
// topk != 0: the top-k mode (every row keeps its m best components, normalised
// over them; threshold unused).  one_pass != 0 (large K, m = 1, no counts or
// log-likelihoods): k-means labels -- each row's best component alone, its
// candidates marked against each slice's running maximum within the error
// band in one pass instead of against the row maximum found by a pass of its
// own, and no mass summed (the responsibility written is relative to the
// candidates only).
static gmm_status run_topm(const Plan& p, const gmm_data* data, const gmm_params* params, int32_t m, float threshold,
                           int32_t* idx, float* resp, int32_t* count, float* logp, void* ws, hipStream_t s,
                           int topk = 0, int one_pass = 0) {
  if (p.largek) {
    LargeKArgs A = largek_args(p, data, params, ws);
    A.topm = 1;
    A.topk = topk;
    A.fused_t = one_pass;
    A.m = m;
    A.thr = threshold;
    A.idx = idx;
    A.resp = resp;
    A.count = count;
    A.logp = logp;
    hipError_t e = launch_largek_topm(p, A, params->weights, params->means, params->covars, s);
    if (e != hipSuccess) return hip_fail(e, "large-K top-m launch");
    return GMM_OK;
  }
  char* w = static_cast<char*>(ws);
  float* W = reinterpret_cast<float*>(w + p.off_W);
  double* prec = reinterpret_cast<double*>(w + p.off_prec);
  double* c0 = reinterpret_cast<double*>(w + p.off_c0);
  double* c = reinterpret_cast<double*>(w + p.off_c);
  double* a = reinterpret_cast<double*>(w + p.off_a);
  int32_t* flag = reinterpret_cast<int32_t*>(w + p.off_flag);
  int32_t* sharp = reinterpret_cast<int32_t*>(w + p.off_sharp);
  float2* err = reinterpret_cast<float2*>(w + p.off_err);
  hipError_t e = launch_prologue(p, params->weights, params->means, params->covars, err, W, prec, c0, c, a, flag, sharp, s);
  if (e != hipSuccess) return hip_fail(e, "prologue launch");
  TopmArgs A;
  A.x = data->x;
  A.xtype = p.dtype;
  A.N = p.N;
  A.D = p.D;
  A.ld_x = p.ld_x;
  A.stride_b = p.stride_b;
  A.K = (int)p.K;
  A.KP = p.KP;
  A.NW = p.NW;
  A.Gb = p.Gb;
  A.ntiles = p.ntiles;
  A.W = W;
  A.c = c;
  A.a = a;
  A.mu = params->means;
  A.prec = prec;
  A.c0 = c0;
  A.err = err;
  A.prec_stride = p.prec_stride;
  A.m = m;
  A.thr = threshold;
  A.topk = topk;
  A.idx = idx;
  A.resp = resp;
  A.count = count;
  A.logp = logp;
  e = p.topm_exact ? launch_topm_exact(p, A, s) : launch_topm(p, A, s);
  if (e != hipSuccess) return hip_fail(e, "top-m launch");
  return GMM_OK;
}


}  // namespace gmm

using namespace gmm;

extern "C" {

size_t gmm_workspace_bytes(const gmm_data* data, int32_t K, int32_t cov, int32_t op, int32_t m) {
  (void)m;
  Plan p;
  if (make_plan(data, K, cov, op, &p) != GMM_OK) return 0;
  return p.ws_bytes;
}

gmm_status gmm_estep_stats(const gmm_data* data, const gmm_params* params, gmm_stats* out, int32_t accumulate,
                           void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  gmm_status st = check_params(params, 0, 0, true);
  if (st != GMM_OK) return st;
  Plan p;
  st = make_plan(data, params->K, params->cov, GMM_OP_ESTEP, &p);
  if (st != GMM_OK) return st;
  if (!out || !out->nk || !out->sx || !out->sxx || !out->loglik)
    return fail(GMM_ERR_INVALID_ARG, "statistics buffers must be non-NULL");
  st = check_ws(p, ws, ws_bytes);
  if (st != GMM_OK) return st;
  return run_estep(p, data, params, ws, out->nk, out->sx, out->sxx, out->loglik, nullptr, accumulate ? 1 : 0,
                   nullptr, (hipStream_t)stream);
}

gmm_status gmm_mstep(int64_t B, int64_t D, const gmm_stats* st_in, int64_t n_total, gmm_params* inout,
                     const gmm_options* opts, int32_t* comp_status, void* stream) {
  g_err.clear();
  gmm_status st = check_params(inout, B, D, true);
  if (st != GMM_OK) return st;
  if (B < 1 || D < 1) return fail(GMM_ERR_INVALID_ARG, "need B >= 1 and D >= 1");
  if (n_total < 1) return fail(GMM_ERR_INVALID_ARG, "n_total must be >= 1");
  if (!st_in || !st_in->nk || !st_in->sx || !st_in->sxx)
    return fail(GMM_ERR_INVALID_ARG, "statistics buffers must be non-NULL");
  if (D > 128) return fail(GMM_ERR_UNSUPPORTED, "D > 128");
  if ((inout->cov == FULL || inout->cov == TIED) && D > 16)
    return fail(GMM_ERR_UNSUPPORTED, "full/tied covariance supports D <= 16");
  if (opts && opts->flags) return fail(GMM_ERR_INVALID_ARG, "options.flags must be 0");
  const double reg = opts ? opts->reg_covar : 1e-6;
  if (!(reg >= 0.0)) return fail(GMM_ERR_INVALID_ARG, "reg_covar must be >= 0");
  hipError_t e = launch_mstep_strided(inout->cov, B, D, inout->K, st_in->nk, st_in->sx, st_in->sxx, n_total,
                                      inout->weights, inout->means, inout->covars, reg, nullptr, 0, comp_status,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "M-step launch");
  return GMM_OK;
}

// Host validation of a fit step; fills the plan.
static gmm_status fit_step_check(const gmm_data* data, const gmm_params* inout, const gmm_options* opts, Plan* p) {
  gmm_status st = check_params(inout, 0, 0, true);
  if (st != GMM_OK) return st;
  st = make_plan(data, inout->K, inout->cov, GMM_OP_FIT, p);
  if (st != GMM_OK) return st;
  if (p->N < 1) return fail(GMM_ERR_INVALID_ARG, "a fit step needs N >= 1");
  if (opts && opts->flags) return fail(GMM_ERR_INVALID_ARG, "options.flags must be 0");
  const double reg = opts ? opts->reg_covar : 1e-6;
  if (!(reg >= 0.0)) return fail(GMM_ERR_INVALID_ARG, "reg_covar must be >= 0");
  return GMM_OK;
}

// The launches of one EM iteration on a checked plan and workspace.
// skip_prologue / prepare_next (fused path, spherical, diag, full only): the
// workspace holds this step's prologue already / the M-step forms the next
// step's.
static gmm_status fit_step_run(const Plan& p, const gmm_data* data, gmm_params* inout, const gmm_options* opts,
                               double* mean_loglik, int32_t* comp_status, void* ws, void* stream,
                               bool skip_prologue = false, bool prepare_next = false) {
  gmm_status st;
  const double reg = opts ? opts->reg_covar : 1e-6;
  char* w = static_cast<char*>(ws);
  double* nk = reinterpret_cast<double*>(w + p.off_nk);
  double* sx = reinterpret_cast<double*>(w + p.off_sx);
  double* sxx = reinterpret_cast<double*>(w + p.off_sxx);
  double* ll = reinterpret_cast<double*>(w + p.off_ll);
  hipStream_t s = (hipStream_t)stream;
  const int32_t* flag = p.largek ? nullptr : reinterpret_cast<const int32_t*>(w + p.off_flag);
  // spherical, diag, full: the M-step runs in the reduction's component blocks
  const bool fused = p.cov != TIED;
  MstepFuse fuse{inout->weights, inout->means, inout->covars, p.N, reg, flag, p.KP, comp_status, PrologueOut{}};
  if (prepare_next && fused && !p.largek)
    fuse.next = PrologueOut{p.DP, p.F, p.KW, p.KP, p.prec_stride,
                            reinterpret_cast<float*>(w + p.off_W), reinterpret_cast<double*>(w + p.off_prec),
                            reinterpret_cast<double*>(w + p.off_c0), reinterpret_cast<double*>(w + p.off_c),
                            reinterpret_cast<double*>(w + p.off_a), reinterpret_cast<int32_t*>(w + p.off_flag),
                            reinterpret_cast<int32_t*>(w + p.off_sharp)};
  st = run_estep(p, data, inout, ws, nk, sx, sxx, ll, mean_loglik, 0, opts, s, fused ? &fuse : nullptr,
                 skip_prologue && fused && !p.largek);
  if (st != GMM_OK || fused) return st;
  hipError_t e = launch_mstep_strided(p.cov, p.B, p.D, p.K, nk, sx, sxx, p.N, inout->weights, inout->means,
                                      inout->covars, reg, flag, p.KP, comp_status, s);
  if (e != hipSuccess) return hip_fail(e, "M-step launch");
  return GMM_OK;
}

gmm_status gmm_fit_step(const gmm_data* data, gmm_params* inout, const gmm_options* opts, double* mean_loglik,
                        int32_t* comp_status, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  Plan p;
  gmm_status st = fit_step_check(data, inout, opts, &p);
  if (st != GMM_OK) return st;
  st = check_ws(p, ws, ws_bytes);
  if (st != GMM_OK) return st;
  return fit_step_run(p, data, inout, opts, mean_loglik, comp_status, ws, stream);
}

gmm_status gmm_fit(const gmm_data* data, gmm_params* inout, const gmm_options* opts, int32_t n_iter,
                   double* mean_loglik, int32_t* comp_status, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  if (n_iter < 1) return fail(GMM_ERR_INVALID_ARG, "n_iter must be >= 1");
  Plan p;
  gmm_status st = fit_step_check(data, inout, opts, &p);
  if (st != GMM_OK) return st;
  st = check_ws(p, ws, ws_bytes);
  if (st != GMM_OK) return st;
  // the next step's prologue is formed in the M-step's blocks where the
  // M-step runs there (spherical, diag, full on the fused path)
  const bool fold = !p.largek && p.cov != TIED;
  for (int32_t t = 0; t < n_iter; ++t) {
    st = fit_step_run(p, data, inout, opts, mean_loglik ? mean_loglik + (size_t)t * p.B : nullptr, comp_status, ws,
                      stream, fold && t > 0, fold && t + 1 < n_iter);
    if (st != GMM_OK) return st;
  }
  return GMM_OK;
}

gmm_status gmm_fit_step_noalloc(const gmm_data* data, gmm_params* inout, const gmm_options* opts,
                                double* mean_loglik, int32_t* comp_status, void* stream) {
  g_err.clear();
  Plan p;
  gmm_status st = fit_step_check(data, inout, opts, &p);
  if (st != GMM_OK) return st;
  if (fit_ws(p, kScratchBytes) != GMM_OK)
    return fail(GMM_ERR_WORKSPACE,
                "gmm_fit_step_noalloc: this problem needs %zu bytes of scratch, more than its static %zu-byte "
                "array; use gmm_fit_step with a workspace",
                p.ws_bytes, kScratchBytes);
  void* ws = scratch_ptr();
  if (!ws) return fail(GMM_ERR_HIP, "gmm_fit_step_noalloc: the device address of the static scratch array");
  return fit_step_run(p, data, inout, opts, mean_loglik, comp_status, ws, stream);
}

// ---- rows in host memory streamed through two device chunk buffers: the
// fused E-step of every chunk adds into one set of statistics, then one
// M-step (Flash-GMM Section 3: the statistics are O(K D); the rows never need
// to be resident at once)
struct StreamLayout {
  Plan p;                 // plan of a full chunk (its workspace is at offset 0)
  int64_t C = 0;          // rows per chunk
  size_t esize = 0;       // bytes per element
  size_t buf_bytes = 0;   // one device chunk buffer: B * C * ld_x elements
  size_t off_buf[2] = {0, 0}, off_nk = 0, off_sx = 0, off_sxx = 0, off_ll = 0, bytes = 0;
};

static gmm_data chunk_view(const gmm_data* hd, const StreamLayout& L, const void* dev_x, int64_t rows) {
  gmm_data cd = *hd;
  cd.x = dev_x;
  cd.N = rows;
  cd.stride_b = L.C * hd->ld_x;
  return cd;
}

static gmm_status stream_plan(const gmm_data* hd, int32_t K, int32_t cov, int64_t chunk_rows, StreamLayout* L) {
  gmm_status st = check_data(hd);
  if (st != GMM_OK) return st;
  if (chunk_rows < 1) return fail(GMM_ERR_INVALID_ARG, "chunk_rows must be >= 1");
  if (hd->N < 1) return fail(GMM_ERR_INVALID_ARG, "a fit step needs N >= 1");
  L->C = std::min<int64_t>(chunk_rows, hd->N);
  L->esize = hd->dtype == GMM_DT_F32 ? 4 : 2;
  // the chunk buffers are 256-byte aligned, so the chunk plan sees aligned rows
  const gmm_data cd = chunk_view(hd, *L, reinterpret_cast<const void*>(kAlign), L->C);
  st = make_plan(&cd, K, cov, GMM_OP_FIT, &L->p);
  if (st != GMM_OK) return st;
  size_t o = align_up(L->p.ws_bytes);
  const size_t B = (size_t)hd->B;
  L->buf_bytes = B * (size_t)L->C * (size_t)hd->ld_x * L->esize;
  L->off_buf[0] = o; o = align_up(o + L->buf_bytes);
  L->off_buf[1] = o; o = align_up(o + L->buf_bytes);
  L->off_nk = o;     o = align_up(o + sizeof(double) * B * K);
  L->off_sx = o;     o = align_up(o + sizeof(double) * B * K * (size_t)hd->D);
  L->off_sxx = o;    o = align_up(o + sizeof(double) * B * (size_t)cov_len(cov, hd->D, K));
  L->off_ll = o;     o = align_up(o + sizeof(double) * B);
  L->bytes = o;
  return GMM_OK;
}

size_t gmm_fit_step_streamed_workspace_bytes(const gmm_data* host_data, int32_t K, int32_t cov, int64_t chunk_rows) {
  StreamLayout L;
  if (stream_plan(host_data, K, cov, chunk_rows, &L) != GMM_OK) return 0;
  return L.bytes;
}

gmm_status gmm_fit_step_streamed(const gmm_data* host_data, gmm_params* inout, const gmm_options* opts,
                                 int64_t chunk_rows, double* mean_loglik, int32_t* comp_status, void* ws,
                                 size_t ws_bytes, void* stream, void* copy_stream) {
  g_err.clear();
  gmm_status st = check_params(inout, 0, 0, true);
  if (st != GMM_OK) return st;
  StreamLayout L;
  st = stream_plan(host_data, inout->K, inout->cov, chunk_rows, &L);
  if (st != GMM_OK) return st;
  if (opts && opts->flags) return fail(GMM_ERR_INVALID_ARG, "options.flags must be 0");
  const double reg = opts ? opts->reg_covar : 1e-6;
  if (!(reg >= 0.0)) return fail(GMM_ERR_INVALID_ARG, "reg_covar must be >= 0");
  if (!ws) return fail(GMM_ERR_WORKSPACE, "workspace is NULL");
  if (((uintptr_t)ws) % kAlign) return fail(GMM_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (ws_bytes < L.bytes) return fail(GMM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.bytes);
  const int64_t N = host_data->N, B = host_data->B, C = L.C;
  const int64_t nchunks = (N + C - 1) / C;
  // every chunk plan fits the full chunk's workspace (it has fewer rows)
  Plan cp[2];
  for (int i = 0; i < 2; ++i) {
    const int64_t rows = i == 0 ? C : N - (nchunks - 1) * C;
    const gmm_data cd = chunk_view(host_data, L, reinterpret_cast<const void*>(kAlign), rows);
    st = make_plan(&cd, inout->K, inout->cov, GMM_OP_FIT, &cp[i]);
    if (st != GMM_OK) return st;
    st = fit_ws(cp[i], L.p.ws_bytes);
    if (st != GMM_OK) return st;
  }
  char* w = static_cast<char*>(ws);
  double* nk = reinterpret_cast<double*>(w + L.off_nk);
  double* sx = reinterpret_cast<double*>(w + L.off_sx);
  double* sxx = reinterpret_cast<double*>(w + L.off_sxx);
  double* ll = reinterpret_cast<double*>(w + L.off_ll);
  hipStream_t s = (hipStream_t)stream;
  hipStream_t cs = copy_stream ? (hipStream_t)copy_stream : s;
  // start: the copies wait for what the compute stream already holds (an
  // earlier call may still read the buffers); copied[i]: buffer i is filled;
  // freed[i]: the E-step that read buffer i is done
  hipEvent_t start = nullptr, copied[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr};
  hipError_t e = hipSuccess;
  auto cleanup = [&]() {
    for (hipEvent_t ev : {start, copied[0], copied[1], freed[0], freed[1]})
      if (ev) (void)hipEventDestroy(ev);
  };
  for (hipEvent_t* ev : {&start, &copied[0], &copied[1], &freed[0], &freed[1]}) {
    if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) {
      cleanup();
      return hip_fail(e, "event create");
    }
  }
  const unsigned char* hx = static_cast<const unsigned char*>(host_data->x);
  const size_t es = L.esize, ld = (size_t)host_data->ld_x;
  const size_t spitch = (B > 1 ? (size_t)host_data->stride_b : 0) * es;
  if ((e = hipEventRecord(start, s)) != hipSuccess || (e = hipStreamWaitEvent(cs, start, 0)) != hipSuccess) {
    cleanup();
    return hip_fail(e, "stream ordering");
  }
  for (int64_t c = 0; c < nchunks; ++c) {
    const int bi = (int)(c & 1);
    const int64_t r0 = c * C, rows = std::min<int64_t>(C, N - r0);
    void* buf = w + L.off_buf[bi];
    if (c >= 2 && (e = hipStreamWaitEvent(cs, freed[bi], 0)) != hipSuccess) break;
    // rows r0 .. r0 + rows - 1 of every problem (the last row up to its D-th element)
    const size_t width = ((size_t)(rows - 1) * ld + (size_t)host_data->D) * es;
    const size_t dpitch = (size_t)C * ld * es;
    e = hipMemcpy2DAsync(buf, dpitch, hx + (size_t)r0 * ld * es, B > 1 ? spitch : width, width, (size_t)B,
                         hipMemcpyHostToDevice, cs);
    if (e != hipSuccess) break;
    if ((e = hipEventRecord(copied[bi], cs)) != hipSuccess || (e = hipStreamWaitEvent(s, copied[bi], 0)) != hipSuccess)
      break;
    const gmm_data cd = chunk_view(host_data, L, buf, rows);
    st = run_estep(c + 1 < nchunks || nchunks == 1 ? cp[0] : cp[1], &cd, inout, ws, nk, sx, sxx, ll, nullptr,
                   c > 0 ? 1 : 0, nullptr, s);
    if (st != GMM_OK) {
      cleanup();
      return st;
    }
    if ((e = hipEventRecord(freed[bi], s)) != hipSuccess) break;
  }
  if (e != hipSuccess) {
    cleanup();
    return hip_fail(e, "streamed chunk");
  }
  if (mean_loglik && (e = launch_mean_ll(B, ll, N, mean_loglik, s)) != hipSuccess) {
    cleanup();
    return hip_fail(e, "mean log-likelihood launch");
  }
  const int32_t* flag = L.p.largek ? nullptr : reinterpret_cast<const int32_t*>(w + L.p.off_flag);
  e = launch_mstep_strided(L.p.cov, B, host_data->D, inout->K, nk, sx, sxx, N, inout->weights, inout->means,
                           inout->covars, reg, flag, L.p.KP, comp_status, s);
  cleanup();
  if (e != hipSuccess) return hip_fail(e, "M-step launch");
  return GMM_OK;
}

gmm_status gmm_predict_proba_topm(const gmm_data* data, const gmm_params* params, int32_t m, float threshold,
                                  int32_t* idx, float* resp, int32_t* count, float* logp, void* ws, size_t ws_bytes,
                                  void* stream) {
  g_err.clear();
  gmm_status st = check_params(params, 0, 0, true);
  if (st != GMM_OK) return st;
  if (m < 1 || m > 16) return fail(GMM_ERR_INVALID_ARG, "m must be in [1, 16] (got %d)", m);
  if (!(threshold >= 0.0f && threshold <= 1.0f)) return fail(GMM_ERR_INVALID_ARG, "threshold must be in [0, 1]");
  Plan p;
  st = make_plan(data, params->K, params->cov, GMM_OP_TOPM, &p);
  if (st != GMM_OK) return st;
  if (p.N > 0 && (!idx || !resp)) return fail(GMM_ERR_INVALID_ARG, "idx and resp must be non-NULL");
  st = check_ws(p, ws, ws_bytes);
  if (st != GMM_OK) return st;
  if (p.N == 0) return GMM_OK;
  return run_topm(p, data, params, m, threshold, idx, resp, count, logp, ws, (hipStream_t)stream);
}

// ---- IVF posting lists
static gmm_status ivf_check(int64_t B, int64_t N, int32_t m, int32_t K) {
  if (B < 1 || N < 0) return fail(GMM_ERR_INVALID_ARG, "need B >= 1 and N >= 0");
  if (m < 1 || m > 16) return fail(GMM_ERR_INVALID_ARG, "m must be in [1, 16] (got %d)", m);
  if (K < 1) return fail(GMM_ERR_INVALID_ARG, "K must be >= 1");
  if (K > kIvfMaxK) return fail(GMM_ERR_UNSUPPORTED, "IVF lists: K <= %d", kIvfMaxK);
  if (N * (int64_t)m > INT32_MAX) return fail(GMM_ERR_UNSUPPORTED, "IVF lists: N * m must fit in int32");
  if (B > INT32_MAX / 64) return fail(GMM_ERR_UNSUPPORTED, "IVF lists: B too large");
  return GMM_OK;
}

static size_t ivf_ws(int64_t B, int64_t N, int32_t K) {
  const int64_t nblk = (N + kIvfBlock - 1) / kIvfBlock;
  return align_up(sizeof(int32_t) * (size_t)B * (size_t)nblk * (size_t)K);
}

size_t gmm_ivf_workspace_bytes(int64_t B, int64_t N, int32_t m, int32_t K) {
  if (ivf_check(B, N, m, K) != GMM_OK) return 0;
  return std::max<size_t>(ivf_ws(B, N, K), kAlign);
}

gmm_status gmm_ivf_lists(int64_t B, int64_t N, int32_t m, int32_t K, const int32_t* idx, const float* resp,
                         int64_t* offsets, int32_t* rows, float* list_resp, void* ws, size_t ws_bytes,
                         void* stream) {
  g_err.clear();
  gmm_status st = ivf_check(B, N, m, K);
  if (st != GMM_OK) return st;
  if (!offsets) return fail(GMM_ERR_INVALID_ARG, "offsets must be non-NULL");
  if (N > 0 && (!idx || !rows)) return fail(GMM_ERR_INVALID_ARG, "idx and rows must be non-NULL");
  if (list_resp && !resp) return fail(GMM_ERR_INVALID_ARG, "list_resp needs resp");
  if (!ws || ((uintptr_t)ws) % kAlign != 0) return fail(GMM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < ivf_ws(B, N, K))
    return fail(GMM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, ivf_ws(B, N, K));
  IvfArgs A;
  A.idx = idx;
  A.resp = list_resp ? resp : nullptr;
  A.N = N;
  A.B = (int)B;
  A.m = m;
  A.K = K;
  A.KB = 0;
  while ((1 << A.KB) < K) ++A.KB;
  A.nblk = (int)((N + kIvfBlock - 1) / kIvfBlock);
  A.cnt = static_cast<int32_t*>(ws);
  A.offsets = offsets;
  A.rows = rows;
  A.lresp = list_resp;
  hipError_t e = launch_ivf_lists(A, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "IVF list launch");
  return GMM_OK;
}

// ---- k-means (Lloyd) iteration: exact top-1 under equal weights and one
// shared variance, posting lists of the labels, list-ordered cluster means
struct KmLayout {
  Plan p;
  size_t off_w, off_cv, off_resp, off_cnt, off_offsets, off_rows, off_ip, bytes;
};

static gmm_status kmeans_plan(const gmm_data* d, int32_t K, KmLayout* L) {
  Plan p;
  gmm_status st = make_plan(d, K, SPH, GMM_OP_TOPM, &p);
  if (st != GMM_OK) return st;
  st = ivf_check(p.B, p.N, 1, K);
  if (st != GMM_OK) return st;
  const size_t B = (size_t)p.B, N = (size_t)p.N, k = (size_t)K;
  size_t o = align_up(p.ws_bytes);
  L->off_w = o;       o = align_up(o + sizeof(float) * B * k);
  L->off_cv = o;      o = align_up(o + sizeof(float) * B * k);
  L->off_resp = o;    o = align_up(o + sizeof(float) * B * N);
  L->off_cnt = o;     o = align_up(o + ivf_ws(p.B, p.N, K));
  L->off_offsets = o; o = align_up(o + sizeof(int64_t) * B * (k + 1));
  L->off_rows = o;    o = align_up(o + sizeof(int32_t) * B * N);
  L->off_ip = o;      o = align_up(o + sizeof(double) * B * k);
  L->bytes = o;
  L->p = p;
  return GMM_OK;
}

size_t gmm_kmeans_workspace_bytes(const gmm_data* data, int32_t K) {
  KmLayout L;
  if (kmeans_plan(data, K, &L) != GMM_OK) return 0;
  return L.bytes;
}

gmm_status gmm_kmeans_step(const gmm_data* data, int32_t K, float* centroids, int32_t* labels, int64_t* counts,
                           double* inertia, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  KmLayout L;
  gmm_status st = kmeans_plan(data, K, &L);
  if (st != GMM_OK) return st;
  const Plan& p = L.p;
  if (!centroids) return fail(GMM_ERR_INVALID_ARG, "centroids must be non-NULL");
  if (p.N > 0 && !labels) return fail(GMM_ERR_INVALID_ARG, "labels must be non-NULL");
  if (!ws || ((uintptr_t)ws) % kAlign != 0) return fail(GMM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L.bytes) return fail(GMM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.bytes);
  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  float* wk = reinterpret_cast<float*>(w + L.off_w);
  float* cv = reinterpret_cast<float*>(w + L.off_cv);
  hipError_t e = launch_kmeans_params(p.B, K, (int)p.D, centroids, wk, cv, s);
  if (e != hipSuccess) return hip_fail(e, "k-means parameter launch");
  if (p.N > 0) {
    gmm_params prm;
    prm.K = K;
    prm.cov = SPH;
    prm.weights = wk;
    prm.means = centroids;
    prm.covars = cv;
    st = run_topm(p, data, &prm, 1, 0.0f, labels, reinterpret_cast<float*>(w + L.off_resp), nullptr, nullptr, ws, s,
                  0, 1);
    if (st != GMM_OK) return st;
  }
  IvfArgs A;
  A.idx = labels;
  A.resp = nullptr;
  A.N = p.N;
  A.B = (int)p.B;
  A.m = 1;
  A.K = K;
  A.KB = 0;
  while ((1 << A.KB) < K) ++A.KB;
  A.nblk = (int)((p.N + kIvfBlock - 1) / kIvfBlock);
  A.cnt = reinterpret_cast<int32_t*>(w + L.off_cnt);
  A.offsets = reinterpret_cast<int64_t*>(w + L.off_offsets);
  A.rows = reinterpret_cast<int32_t*>(w + L.off_rows);
  A.lresp = nullptr;
  e = launch_ivf_lists(A, s);
  if (e != hipSuccess) return hip_fail(e, "k-means list launch");
  e = launch_kmeans_update(data->x, data->dtype, p.B, p.N, p.ld_x, p.stride_b, K, (int)p.D,
                           A.offsets, A.rows, centroids, counts, reinterpret_cast<double*>(w + L.off_ip), inertia, s);
  if (e != hipSuccess) return hip_fail(e, "k-means update launch");
  return GMM_OK;
}

// ---- Fisher vectors: the batched E-step's per-problem statistics under one
// replicated diagonal model, turned into gradient blocks by fisher_kernel
struct FvLayout {
  Plan p;
  size_t off_w, off_mu, off_var, off_nk, off_sx, off_sxx, off_ll, bytes;
};

static gmm_status fisher_plan(const gmm_data* d, int32_t K, FvLayout* L) {
  Plan p;
  gmm_status st = make_plan(d, K, DIAG, GMM_OP_ESTEP, &p);
  if (st != GMM_OK) return st;
  const size_t B = (size_t)p.B, k = (size_t)K, D = (size_t)p.D;
  size_t o = align_up(p.ws_bytes);
  L->off_w = o;   o = align_up(o + sizeof(float) * B * k);
  L->off_mu = o;  o = align_up(o + sizeof(float) * B * k * D);
  L->off_var = o; o = align_up(o + sizeof(float) * B * k * D);
  L->off_nk = o;  o = align_up(o + sizeof(double) * B * k);
  L->off_sx = o;  o = align_up(o + sizeof(double) * B * k * D);
  L->off_sxx = o; o = align_up(o + sizeof(double) * B * k * D);
  L->off_ll = o;  o = align_up(o + sizeof(double) * B);
  L->bytes = o;
  L->p = p;
  return GMM_OK;
}

size_t gmm_fisher_vector_workspace_bytes(const gmm_data* data, int32_t K) {
  FvLayout L;
  if (fisher_plan(data, K, &L) != GMM_OK) return 0;
  return L.bytes;
}

gmm_status gmm_fisher_vector(const gmm_data* data, const gmm_params* model, uint32_t flags, float* fv, void* ws,
                             size_t ws_bytes, void* stream) {
  g_err.clear();
  if (!model || !model->weights || !model->means || !model->covars)
    return fail(GMM_ERR_INVALID_ARG, "model parameters must be non-NULL");
  if (model->cov != DIAG) return fail(GMM_ERR_UNSUPPORTED, "Fisher vectors take a diagonal model");
  if (flags & ~3u) return fail(GMM_ERR_INVALID_ARG, "flags: bit 0 power, bit 1 L2; other bits must be 0");
  FvLayout L;
  gmm_status st = fisher_plan(data, model->K, &L);
  if (st != GMM_OK) return st;
  if (!fv) return fail(GMM_ERR_INVALID_ARG, "fv must be non-NULL");
  if (!ws || ((uintptr_t)ws) % kAlign != 0) return fail(GMM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L.bytes) return fail(GMM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.bytes);
  const Plan& p = L.p;
  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  float* wr = reinterpret_cast<float*>(w + L.off_w);
  float* mur = reinterpret_cast<float*>(w + L.off_mu);
  float* varr = reinterpret_cast<float*>(w + L.off_var);
  double* nk = reinterpret_cast<double*>(w + L.off_nk);
  double* sx = reinterpret_cast<double*>(w + L.off_sx);
  double* sxx = reinterpret_cast<double*>(w + L.off_sxx);
  double* ll = reinterpret_cast<double*>(w + L.off_ll);
  hipError_t e = launch_fisher_replicate(p.B, model->K, (int)p.D, model->weights, model->means, model->covars, wr,
                                         mur, varr, s);
  if (e != hipSuccess) return hip_fail(e, "Fisher model replication launch");
  gmm_params rep;
  rep.K = model->K;
  rep.cov = DIAG;
  rep.weights = wr;
  rep.means = mur;
  rep.covars = varr;
  st = run_estep(p, data, &rep, ws, nk, sx, sxx, ll, nullptr, 0, nullptr, s);
  if (st != GMM_OK) return st;
  e = launch_fisher(p.B, model->K, (int)p.D, p.N, flags, model->weights, model->means, model->covars, nk, sx, sxx, fv,
                    s);
  if (e != hipSuccess) return hip_fail(e, "Fisher vector launch");
  return GMM_OK;
}

// ---- approximate top-k EM: the top-m pass in its top-k mode (m = k, each row's
// k best normalised over themselves), the posting lists of its entries,
// weighted statistics per component, M-step

struct TkLayout {
  Plan p;
  size_t off_idx, off_resp, off_logp, off_rinv, off_llpart, off_cnt, off_offsets, off_rows, off_lresp;
  size_t off_part, off_nk, off_sx, off_sxx, off_ll, bytes;
  int S;
};

static gmm_status topk_plan(const gmm_data* d, int32_t K, int32_t cov, int32_t topk, TkLayout* L) {
  if (cov != SPH && cov != DIAG) return fail(GMM_ERR_UNSUPPORTED, "top-k EM takes spherical or diagonal components");
  if (topk < 1 || topk > 16) return fail(GMM_ERR_INVALID_ARG, "topk must be in [1, 16] (got %d)", topk);
  Plan p;
  gmm_status st = make_plan(d, K, cov, GMM_OP_TOPM, &p);
  if (st != GMM_OK) return st;
  st = ivf_check(p.B, p.N, topk, K);
  if (st != GMM_OK) return st;
  const size_t B = (size_t)p.B, N = (size_t)p.N, k = (size_t)K, D = (size_t)p.D, m = (size_t)topk;
  size_t o = align_up(p.ws_bytes);
  L->off_idx = o;     o = align_up(o + sizeof(int32_t) * B * N * m);
  L->off_resp = o;    o = align_up(o + sizeof(float) * B * N * m);
  L->off_logp = o;    o = align_up(o + sizeof(float) * B * N);
  L->off_rinv = o;    o = align_up(o + sizeof(double) * B * N);
  L->off_llpart = o;  o = align_up(o + sizeof(double) * B * ((N + 255) / 256));
  L->off_cnt = o;     o = align_up(o + ivf_ws(p.B, p.N, K));
  L->off_offsets = o; o = align_up(o + sizeof(int64_t) * B * (k + 1));
  L->off_rows = o;    o = align_up(o + sizeof(int32_t) * B * N * m);
  L->off_lresp = o;   o = align_up(o + sizeof(float) * B * N * m);
  L->S = topk_parts(p.B, p.N, topk, K);
  L->off_part = o;    o = align_up(o + sizeof(double) * B * k * (size_t)L->S * (1 + 2 * D));
  L->off_nk = o;      o = align_up(o + sizeof(double) * B * k);
  L->off_sx = o;      o = align_up(o + sizeof(double) * B * k * D);
  L->off_sxx = o;     o = align_up(o + sizeof(double) * B * (cov == DIAG ? k * D : k));
  L->off_ll = o;      o = align_up(o + sizeof(double) * B);
  L->bytes = o;
  L->p = p;
  return GMM_OK;
}

size_t gmm_topk_fit_workspace_bytes(const gmm_data* data, int32_t K, int32_t cov, int32_t topk) {
  TkLayout L;
  if (topk_plan(data, K, cov, topk, &L) != GMM_OK) return 0;
  return L.bytes;
}

gmm_status gmm_topk_fit_step(const gmm_data* data, gmm_params* inout, int32_t topk, const gmm_options* opts,
                             double* mean_loglik, int32_t* comp_status, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  gmm_status st = check_params(inout, 0, 0, true);
  if (st != GMM_OK) return st;
  TkLayout L;
  st = topk_plan(data, inout->K, inout->cov, topk, &L);
  if (st != GMM_OK) return st;
  const Plan& p = L.p;
  if (p.N < 1) return fail(GMM_ERR_INVALID_ARG, "a fit step needs N >= 1");
  if (opts && opts->flags) return fail(GMM_ERR_INVALID_ARG, "options.flags must be 0");
  const double reg = opts ? opts->reg_covar : 1e-6;
  if (!(reg >= 0.0)) return fail(GMM_ERR_INVALID_ARG, "reg_covar must be >= 0");
  if (!ws || ((uintptr_t)ws) % kAlign != 0) return fail(GMM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L.bytes) return fail(GMM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.bytes);
  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  int32_t* idx = reinterpret_cast<int32_t*>(w + L.off_idx);
  float* resp = reinterpret_cast<float*>(w + L.off_resp);
  float* logp = reinterpret_cast<float*>(w + L.off_logp);
  // kept: each row's topk best components, decided on float64 scores, with
  // their responsibilities and log-sum-exp over those topk only
  st = run_topm(p, data, inout, topk, 0.0f, idx, resp, nullptr, logp, ws, s, 1);
  if (st != GMM_OK) return st;
  IvfArgs A;
  A.idx = idx;
  A.resp = resp;
  A.N = p.N;
  A.B = (int)p.B;
  A.m = topk;
  A.K = inout->K;
  A.KB = 0;
  while ((1 << A.KB) < inout->K) ++A.KB;
  A.nblk = (int)((p.N + kIvfBlock - 1) / kIvfBlock);
  A.cnt = reinterpret_cast<int32_t*>(w + L.off_cnt);
  A.offsets = reinterpret_cast<int64_t*>(w + L.off_offsets);
  A.rows = reinterpret_cast<int32_t*>(w + L.off_rows);
  A.lresp = reinterpret_cast<float*>(w + L.off_lresp);
  hipError_t e = launch_ivf_lists(A, s);
  if (e != hipSuccess) return hip_fail(e, "top-k list launch");
  double* nk = reinterpret_cast<double*>(w + L.off_nk);
  double* sx = reinterpret_cast<double*>(w + L.off_sx);
  double* sxx = reinterpret_cast<double*>(w + L.off_sxx);
  TopkStepArgs T;
  T.x = data->x;
  T.xtype = data->dtype;
  T.B = p.B;
  T.N = p.N;
  T.ld_x = p.ld_x;
  T.stride_b = p.stride_b;
  T.K = inout->K;
  T.D = (int)p.D;
  T.m = topk;
  T.cov = inout->cov;
  T.S = L.S;
  T.resp = resp;
  T.logp = logp;
  T.mu = inout->means;
  T.offsets = A.offsets;
  T.rows = A.rows;
  T.lresp = A.lresp;
  T.rinv = reinterpret_cast<double*>(w + L.off_rinv);
  T.llpart = reinterpret_cast<double*>(w + L.off_llpart);
  T.part = reinterpret_cast<double*>(w + L.off_part);
  T.nk = nk;
  T.sx = sx;
  T.sxx = sxx;
  T.ll = reinterpret_cast<double*>(w + L.off_ll);
  T.mean_ll = mean_loglik;
  e = launch_topk_stats(T, s);
  if (e != hipSuccess) return hip_fail(e, "top-k statistics launch");
  e = launch_mstep_strided(inout->cov, p.B, p.D, inout->K, nk, sx, sxx, p.N, inout->weights, inout->means,
                           inout->covars, reg, nullptr, 0, comp_status, s);
  if (e != hipSuccess) return hip_fail(e, "M-step launch");
  return GMM_OK;
}

// ---- Gaussian kernel density estimate: centred references, then the
// streaming log-sum-exp kernel
struct KdeLayout {
  int DP;
  int64_t Mp;
  size_t off_cen, off_xc, off_bx, bytes;
};

static gmm_status kde_plan(const gmm_data* q, int64_t M, KdeLayout* L) {
  gmm_status st = check_data(q);
  if (st != GMM_OK) return st;
  if (q->dtype != GMM_DT_F32) return fail(GMM_ERR_UNSUPPORTED, "kernel density: float32 query rows only");
  if (q->D > 128) return fail(GMM_ERR_UNSUPPORTED, "kernel density: D <= 128 (got %lld)", (long long)q->D);
  if (M < 1) return fail(GMM_ERR_INVALID_ARG, "kernel density needs M >= 1 reference rows (got %lld)", (long long)M);
  if (M > ((int64_t)1 << 30)) return fail(GMM_ERR_UNSUPPORTED, "kernel density: M <= 2^30");
  const int64_t nqb = (q->N + kde_query_rows() - 1) / kde_query_rows();
  if (q->B * nqb >= ((int64_t)1 << 31)) return fail(GMM_ERR_UNSUPPORTED, "kernel density: too many query rows");
  L->DP = q->D <= 16 ? 16 : q->D <= 32 ? 32 : q->D <= 64 ? 64 : 128;
  const int64_t T = kde_tile_rows();
  L->Mp = (M + T - 1) / T * T;
  size_t o = 0;
  L->off_cen = o; o = align_up(o + sizeof(float) * (size_t)L->DP);
  L->off_xc = o;  o = align_up(o + sizeof(float) * (size_t)L->Mp * L->DP);
  L->off_bx = o;  o = align_up(o + sizeof(float) * (size_t)L->Mp);
  L->bytes = o;
  return GMM_OK;
}

size_t gmm_kde_workspace_bytes(const gmm_data* queries, int64_t M) {
  KdeLayout L;
  if (kde_plan(queries, M, &L) != GMM_OK) return 0;
  return L.bytes;
}

gmm_status gmm_kde_score(const gmm_data* queries, const float* ref, int64_t M, int64_t ld_ref, double bandwidth,
                         float* logdens, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  KdeLayout L;
  gmm_status st = kde_plan(queries, M, &L);
  if (st != GMM_OK) return st;
  if (!ref) return fail(GMM_ERR_INVALID_ARG, "ref must be non-NULL");
  if (ld_ref < queries->D)
    return fail(GMM_ERR_INVALID_ARG, "ld_ref (%lld) < D (%lld)", (long long)ld_ref, (long long)queries->D);
  if (!(bandwidth > 0.0) || !std::isfinite(bandwidth))
    return fail(GMM_ERR_INVALID_ARG, "bandwidth must be finite and > 0");
  const double LOG2E = 1.4426950408889634074;
  const float lamf = (float)(LOG2E / (2.0 * bandwidth * bandwidth));
  if (!(lamf > 0.f) || !std::isfinite(lamf))
    return fail(GMM_ERR_INVALID_ARG, "bandwidth %g is outside the float32 range of 1 / (2 h^2)", bandwidth);
  const int64_t rows = queries->B * queries->N;
  if (rows > 0 && !logdens) return fail(GMM_ERR_INVALID_ARG, "logdens must be non-NULL");
  if (!ws || ((uintptr_t)ws) % kAlign != 0) return fail(GMM_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L.bytes) return fail(GMM_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.bytes);
  if (rows == 0) return GMM_OK;
  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  float* cen = reinterpret_cast<float*>(w + L.off_cen);
  float* xc = reinterpret_cast<float*>(w + L.off_xc);
  float* bx = reinterpret_cast<float*>(w + L.off_bx);
  hipError_t e = launch_kde_prep(ref, M, ld_ref, (int)queries->D, L.DP, L.Mp, (double)lamf, cen, xc, bx, s);
  if (e != hipSuccess) return hip_fail(e, "kernel density reference launch");
  KdeArgs a;
  a.y = static_cast<const float*>(queries->x);
  a.B = queries->B;
  a.N = queries->N;
  a.ld = queries->ld_x;
  a.stride_b = queries->B > 1 ? queries->stride_b : 0;
  a.D = (int)queries->D;
  a.cen = cen;
  a.xc = xc;
  a.bx = bx;
  a.Mp = L.Mp;
  a.lam = (double)lamf;
  a.s2 = 2.f * lamf;
  a.lam_exact = LOG2E / (2.0 * bandwidth * bandwidth);
  a.ref = ref;
  a.ld_ref = ld_ref;
  a.cnst = -std::log((double)M) - 0.5 * (double)queries->D * std::log(2.0 * M_PI * bandwidth * bandwidth);
  a.out = logdens;
  e = launch_kde(a, L.DP, s);
  if (e != hipSuccess) return hip_fail(e, "kernel density launch");
  return GMM_OK;
}

const char* gmm_status_str(int32_t status) {
  switch (status) {
    case GMM_OK: return "ok";
    case GMM_ERR_INVALID_ARG: return "invalid argument";
    case GMM_ERR_UNSUPPORTED: return "unsupported shape or type";
    case GMM_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case GMM_ERR_HIP: return "HIP runtime error";
    case GMM_ERR_NOT_PD: return "covariance not positive definite";
    default: return "unknown status";
  }
}

gmm_status gmm_check_components(const int32_t* comp_status_host, int64_t count, int64_t* first) {
  g_err.clear();
  if (first) *first = -1;
  if (!comp_status_host || count < 0) return fail(GMM_ERR_INVALID_ARG, "comp_status must be non-NULL, count >= 0");
  for (int64_t i = 0; i < count; ++i) {
    if (comp_status_host[i] & (2 | 4)) {
      if (first) *first = i;
      return fail(GMM_ERR_NOT_PD, "component %lld: covariance not positive definite (flag %d)", (long long)i,
                  comp_status_host[i]);
    }
  }
  return GMM_OK;
}

const char* gmm_last_error(void) { return g_err.c_str(); }

int32_t gmm_version(void) { return 200; }

}  // extern "C"
