// gmm_largek.hip -- the E-step for spherical components when K is too large
// for one workgroup to hold every component's statistics (the IVF-sized
// workload: K = 4096, D = 128, bfloat16 rows).
//
// What it computes is the same as the fused kernel of gmm_estep.hip ("Flash-
// GMM: A Memory-Efficient Kernel for Scalable Soft Clustering", Sections 2 and
// 3): log-scores, row log-sum-exp, responsibilities, and the statistics N_k,
// sum r x, sum r |x|^2 and sum LSE, with no N x K matrix in memory.  The
// difference is the decomposition.  Components are cut into slices; a
// workgroup owns one slice (its logit weights in LDS, its statistics in
// registers) and streams rows.  A row's normaliser needs every slice, so each
// chunk of rows takes three passes:
//   A  per (row, 256-component slice): max and sum of 2^(l - max)
//   B  per row: combine the slices -> LSE (log2 units) and sum LSE
//   C  per (row, 128-component slice): logits again, r = 2^(l - LSE),
//      statistics
// Scratch is O(chunk), not O(N).
//
// gfx950 specifics: the x . (lambda mu) contraction runs on bf16 MFMA with
// the weights split into bf16 hi + lo parts (x itself is exact in bf16):
// v_mfma_f32_32x32x16_bf16 in the barrier-free pass A (which also adds
// c + a |x|^2 as one more MFMA step), v_mfma_f32_16x16x32_bf16 in pass C and
// the barrier-based passes; the statistics contraction X^T R runs on the
// 16x16x32 instruction with r rounded to bf16.  Every statistic (N_k, sum r x,
// sum r |x|^2) uses that same rounded r, so the M-step sees the exact moments
// of one set of weights; N_k and sum r |x|^2 ride on the same MFMAs as extra
// features (1, and |x|^2 as five bf16 terms).  The responsibilities are summed in two magnitude
// classes (r >= 2^-8 and below) by separate MFMAs into separate float32
// accumulators, added in float64 at the chunk's partial: a component
// collapsed onto a row far from the origin has a variance many orders below
// |mu|^2, carried by rows of tiny r that a float32 sum with its own row
// (r near 1) would bury; within a class the terms are of like magnitude.  The logit accumulator layout
// (lane l: component l%16, rows 4(l/16)+v of a 16-row block) provides R as
// the B operand of the statistics MFMA directly when the 32 rows of a tile
// are ordered k = 8g + j <-> row 4g + j (j < 4), 16 + 4g + (j - 4) (j >= 4);
// the A operand X^T comes straight from the row tile in LDS by the
// transposing 64-bit LDS load (ds_read_b64_tr_b16), two per 16-feature
// block, one for each half of that row order.  Workgroups of one row
// group and different slices have ids that differ by multiples of 8, so they
// share an XCD and its L2 copy of the rows.
#include "gmm_device.h"
#include "gmm_internal.h"

#include <math.h>

#include <algorithm>
#include <type_traits>

namespace gmm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
// LDS pointers: address arithmetic in 32 bits
typedef __attribute__((address_space(3))) unsigned short lds_u16;
typedef __attribute__((address_space(3))) u16x8 lds_u16x8;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) floatx4 lds_floatx4;
typedef __attribute__((address_space(3))) double lds_f64;

namespace {

constexpr int KSA = kLargeKSlice;      // components per workgroup in pass A (256)
constexpr int KSC = kLargeKSlice / 2;  // components per workgroup in pass C (128)
constexpr int LNW = 8;                 // waves per workgroup
constexpr int LT = 32;                 // rows per tile
constexpr int LRS = 136;               // LDS row stride of the row tile, in bf16 (272 bytes)
constexpr double kSharpLowp = kLargeKSharp;
// responsibilities at or above this go to the "big" class of the statistics
// MFMA; r >= 0, so the class test compares bf16 bit patterns
constexpr float kBigR = 0x1p-8f;
constexpr short kBigRBits = 0x3B80;
static_assert(__builtin_bit_cast(unsigned, kBigR) == (unsigned)kBigRBits << 16, "bf16 pattern of kBigR");
// log-score constant of padded and dead components: finite, so that maxima
// and differences stay finite, and far enough down that 2^(l - max) is 0
constexpr float kDead = -1.0e30f;
// top-m: components scored within this many log2 units of a row's maximum
// are rescored exactly; the others (each below 2^-20 of the maximum's mass)
// enter the row's LSE with their expanded-form scores
constexpr float kTopmBand = 20.f;


__device__ __forceinline__ float bf16_to_f32(unsigned short h) { return __uint_as_float((unsigned)h << 16); }

// The 16-byte piece of a row tile that thread j loads: row j / 16, dims
// 8 (j % 16) .. +7 -- a row's 256 bytes come from 16 consecutive lanes, so a
// wave's load touches 8 cache lines.
// Row r = 16 b + 8 h + j of a tile sits in LDS slot 16 b + 2 j + h.  With
// slots 68 dwords apart (4 banks), the 16-byte logit reads of a 16-row block
// (16 lanes, one row each) still cover all 64 banks once, and each half-wave
// of pass C's transposing reads -- 8 rows, 32 bytes each -- now takes every
// other slot, 8 banks apart: no two rows share a bank (next-slot rows would).
__device__ __forceinline__ int tile_slot(int r) { return (r & ~15) | ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ void piece_of(int j, int& r, int& c8) {
  r = j / 16;
  c8 = (j % 16) * 8;
}


struct Piece {
  u16x8 v;
  u16x8 ext;  // pass C: the statistics features 128..135 of row j (threads j < LT), from pass B
  double xs;  // pass C: |x|^2 of row j (threads j < LT), computed by pass A
  float ls;   // threads j < LT, row j: its LSE (pass C) or its maximum score (pass T)
  int nv;     // dims of v that belong to the row (the rest is zeroed when staged)
};

// Loads without branches: every address is clamped into the chunk (N >= 1),
// and what lies outside it is zeroed when the piece is staged.  Each call
// then issues the same loads in the same order, so the wait before a tile's
// staging covers only that tile's loads, not the later tiles' in flight.
// VEC: rows 16-byte aligned with a stride that is a multiple of 8.
template <int PASS, bool VEC, bool STATS = (PASS == 2)>
__device__ __forceinline__ Piece fetch_piece(const LargeKArgs& A, int64_t tile, int64_t ntiles) {
  const unsigned short* xb = reinterpret_cast<const unsigned short*>(A.x);
  const int j = threadIdx.x;
  int r, c8;
  piece_of(j, r, c8);
  // row indices within the chunk (at most 2^20 rows, tiles a few past the
  // end) in 32-bit arithmetic
  const int n = (int)A.N, tl = (int)tile, npad = (int)ntiles * LT;
  const int row = tl * LT + r;
  const int rc = min(row, n - 1);
  const int D = (int)A.D;
  Piece pc;
  pc.nv = (tl < (int)ntiles && row < n) ? min(max(D - c8, 0), 8) : 0;
  if constexpr (VEC) {
    pc.v = *reinterpret_cast<const u16x8*>(xb + (int64_t)rc * A.ld_x + min(c8, (int)A.ld_x - 8));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) pc.v[e] = xb[(int64_t)rc * A.ld_x + min(c8 + e, D - 1)];
  }
  pc.xs = 0.0;
  pc.ls = 0.f;
  pc.ext = u16x8{};
  // the per-row values: threads j < LT stage them, so only the first wave
  // loads (a wave-uniform branch: the others skip the address arithmetic)
  const int xrow = tl * LT + (j & (LT - 1));
  if (j < 64) {
    if constexpr (STATS) {
      // pass B padded the LSE (+inf) and the statistics features to whole
      // tiles (ntiles * LT rows)
      const int xpad = min(xrow, npad - 1);
      pc.xs = A.xsq[min(xrow, n - 1)];
      pc.ls = A.lse[xpad];
      pc.ext = reinterpret_cast<const u16x8*>(A.ext)[xpad];
    } else if constexpr (PASS == 1) {
      // top-m: the row maximum; top-k: the row's candidate threshold
      pc.ls = (A.topk ? A.kthr : A.mrow)[min(xrow, n - 1)];
    }
  }
  return pc;
}

// Write a thread's piece into the LDS tile.  Pass A also forms |x|^2 of each
// row: in the workgroups of slice 0 exactly (each bf16 square is exact in
// float32, their sum exact in float64), stored for pass C and the top-m
// rescoring; elsewhere in float32.  Pass C keeps |x|^2 as float32 (the first
// half of the area) and the LSE as loaded: pass B padded both to whole
// tiles, rows past N carry LSE = +inf (r = 0), and their loads were clamped
// to row N - 1, so with 128-dim rows (FULL) nothing past N needs zeroing.
template <bool STATS, bool FULL = false>
__device__ __forceinline__ void stage_piece(const LargeKArgs& A, const Piece& pc, int64_t row0, int slice,
                                            lds_u16* rows, lds_f64* xsq, lds_f32* ls) {
  const int j = threadIdx.x;
  int r, c8;
  piece_of(j, r, c8);
  u16x8 v = pc.v;
  if (!(STATS && FULL) && pc.nv < 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < pc.nv ? v[e] : (unsigned short)0;
  }
  *(lds_u16x8*)(rows + tile_slot(r) * LRS + c8) = v;
  const bool live = row0 + j < A.N;  // threads j < LT: row j of the tile
  if constexpr (STATS) {
    if (j < LT) {
      ls[j] = pc.ls;
      ((lds_f32*)xsq)[j] = (float)pc.xs;
      // columns 128.. of the row's slot: the statistics MFMA's features
      // 128..133 (1 and |x|^2 in five bf16 terms, formed by pass B)
      *(lds_u16x8*)(rows + tile_slot(j) * LRS + 128) = pc.ext;
    }
  } else if (j < LT) {
    ls[j] = live ? pc.ls : 0.f;
  }
  if constexpr (STATS) {
  } else if (slice == 0) {
    double sq = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = bf16_to_f32(v[e]);
      sq += (double)(f * f);
    }
    sq = row16_sum_f64(sq);
    if ((j & 15) == 0) {
      xsq[r] = sq;
      if (row0 + r < A.N) A.xsq[row0 + r] = sq;
    }
  } else {
    // the other slices use |x|^2 only in the float32 logits
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = bf16_to_f32(v[e]);
      sq = fmaf(f, f, sq);
    }
    sq = row16_sum(sq);
    if ((j & 15) == 0) xsq[r] = (double)sq;
  }
}

// log2-units score of one row against component k from direct differences:
// c0_k - (lambda_k / 2) |x - mu_k|^2 log2(e), in float64
__device__ __forceinline__ float largek_exact_score(const float* __restrict__ mu, double c0, double lam, int D,
                                                   const unsigned short* xrow) {
  constexpr double kLog2e = 1.4426950408889634074;
  double q = 0.0;
#pragma unroll 1
  for (int d = 0; d < D; ++d) {
    const double t = (double)bf16_to_f32(xrow[d]) - (double)mu[d];
    q += t * t;
  }
  return (float)(c0 - 0.5 * kLog2e * lam * q);
}

}  // namespace

size_t largek_lds_bytes(int DP, int pass) {
  // weights (pass C keeps them in registers)
  size_t b = pass != 2 ? (size_t)(KSA / 16) * 2 * (DP / 32) * 64 * 16 : 0;
  size_t tile = (size_t)LT * LRS * 2;                       // row tile
  tile += (size_t)LT * 8 + LT * 4;                          // |x|^2, LSE or maximum
  b += (pass == 2 ? 3 : 2) * tile;                          // buffers
  if (pass != 2) b += (size_t)2 * LNW * LT * 2 * 4;         // per-wave (max, sum), two tiles
  if (pass == 1) b += (size_t)2 * LT * LNW * 4;             // candidate masks, two tiles
  return b;
}

// PASS: 0 = A (slice max/sum), 1 = T (top-m candidates), 2 = C (statistics).
// FULL: rows of exactly DP dims (no staged piece needs zeroing in pass C).
// Weights in global memory: 16-component tiles, [tile][hi/lo][kstep][lane] x 16 bytes.
template <int DP, int PASS, bool FULL = false>
__global__ void __launch_bounds__(512) largek_kernel(LargeKArgs A) {
  constexpr bool STATS = (PASS == 2);
  constexpr int KSL = STATS ? KSC : KSA;  // components of this workgroup
  constexpr int NT = KSL / LNW / 16;      // 16-column tiles per wave (2 in A, 1 in C)
  constexpr int KSTEP = DP / 32;          // MFMA k-steps over the features
  constexpr int GM = DP / 16;             // statistic row tiles (dimensions)
  constexpr int GMX = GM + 1;             // and one for N_k and sum r |x|^2 (features 128..133)
  constexpr int WFRAG = (KSL / 16) * 2 * KSTEP * 64;
  // pass C holds its wave's logit weights in registers for the whole kernel
  // (NT * 2 * KSTEP fragments); passes A and T read them from LDS
  constexpr bool WREG = STATS;
  constexpr int WLDS = WREG ? 0 : WFRAG;  // 16-byte fragments in LDS
  constexpr int PF = STATS ? 3 : 2;       // row tiles in flight (registers)
  static_assert(DP == 128 && LT * DP / 8 == 64 * LNW, "one 16-byte piece per thread");

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int slice = blockIdx.x / A.G;
  const int g = blockIdx.x % A.G;
  const int64_t nrows = A.N;
  const int64_t ntiles = (nrows + LT - 1) / LT;

  // row-tile buffers (rows, |x|^2, per-row LSE or maximum): pass C keeps
  // three -- tile i's rows for its statistics, tile i + 1's for its logits,
  // tile i + 2 being staged -- and passes A and T
  // two (tile i, tile i + 1 being staged)
  constexpr int NB = STATS ? 3 : 2;
  constexpr int BUFB = LT * LRS * 2 + LT * 8 + LT * 4;  // bytes per buffer
  static_assert(BUFB % 16 == 0, "16-byte aligned buffers");
  extern __shared__ float lds[];
  bf16x8* Wl = reinterpret_cast<bf16x8*>(lds);
  unsigned char* bufs = reinterpret_cast<unsigned char*>(Wl + WLDS);
  __attribute__((address_space(3))) unsigned char* bufs3 = (__attribute__((address_space(3))) unsigned char*)bufs;
  auto rows_of = [&](int bi) { return (lds_u16*)(bufs3 + bi * BUFB); };
  auto xsq_of = [&](int bi) { return (lds_f64*)(rows_of(bi) + LT * LRS); };
  auto ls_of = [&](int bi) { return (lds_f32*)(xsq_of(bi) + LT); };
  float* red = reinterpret_cast<float*>(bufs + NB * BUFB);  // pass A: 2 buffers of LNW * LT * 2
  // pass T: 2 buffers of (LT rows, LNW waves) candidate masks, bit j of word
  // (row, w) = component w * 32 + j of the slice
  uint32_t* lmask = reinterpret_cast<uint32_t*>(red + 2 * LNW * LT * 2);

  bf16x8 wreg[WREG ? NT : 1][2][WREG ? KSTEP : 1];
  if constexpr (WREG) {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(A.W) + (size_t)slice * WFRAG;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks) wreg[nt][h][ks] = src[(((wv * NT + nt) * 2 + h) * KSTEP + ks) * 64 + lane];
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(A.W) + (size_t)slice * WFRAG;
    uint4* dst = reinterpret_cast<uint4*>(Wl);
    for (int i = threadIdx.x; i < WFRAG; i += blockDim.x) dst[i] = src[i];
  }
  // Pass A computes the logits transposed (weights as the MFMA's A operand):
  // lane l then holds rows rb * 16 + l % 16 against components
  // nt * 16 + 4 (l / 16) + v, so a row's max and sum over the wave's
  // components are an in-lane fold over (nt, v) plus two cross-row swaps.
  // Passes T and C keep rows 4 (l / 16) + v against component l % 16 (the
  // layout the statistics MFMA takes as its B operand).
  constexpr bool TR = (PASS == 0);
  constexpr int CV = TR ? 4 : 1;  // components per lane and 16-column tile
  auto comp_of = [&](int nt, int v) {
    return slice * KSL + (wv * NT + nt) * 16 + (TR ? 4 * (lane >> 4) + v : (lane & 15));
  };
  float creg[NT][CV], areg[NT][CV];
  float eb[NT][CV], e0[NT][CV];  // error bound of a sharp component's expanded score: eb |x|^2 + e0 (0: not sharp)
  float ea[NT], ea0[NT];         // pass T: the same bound for every component
  bool any_sharp = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int v = 0; v < CV; ++v) {
      const int k = comp_of(nt, v);
      creg[nt][v] = (float)A.c[k];
      areg[nt][v] = (float)A.a[k];
      eb[nt][v] = A.esh[2 * k];
      e0[nt][v] = A.esh[2 * k + 1];
      any_sharp = any_sharp || (__builtin_amdgcn_ballot_w64(eb[nt][v] > 0.f) != 0);
    }
    if constexpr (PASS == 1) {
      const int k = comp_of(nt, 0);
      ea[nt] = A.eall[2 * k];
      ea0[nt] = A.eall[2 * k + 1];
    }
  }
  // pass C: statistics of the r >= 2^-8 and r < 2^-8 classes, each in its
  // own float32 MFMA accumulator (float64 at the chunk's partial)
  floatx4 sbig[STATS ? GMX : 1][NT];
  floatx4 ssmall[STATS ? GMX : 1][NT];
#pragma unroll
  for (int mt = 0; mt < (STATS ? GMX : 1); ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      ssmall[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      sbig[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

  // pass A: combine the waves' (max, sum) of a finished tile into P; run by
  // one wave (rotating) while the others go on with the next tile
  // pass T: sum the waves' below-band mass of a finished tile into Prem
  auto combine = [&](int64_t prow0, const float* rb) {
    if (lane < LT) {
      const int p = lane;
      const int64_t row = prow0 + p;
      if (PASS == 1) {
        // this slice's below-band mass and its 8 candidate words of the row
        const int buf = (rb - red) / (LNW * LT * 2);
        if (row < nrows) {
          float S = 0.f;
#pragma unroll
          for (int w2 = 0; w2 < LNW; ++w2) S += rb[(w2 * LT + p) * 2 + 1];
          A.prem[(size_t)row * A.S + slice] = S;
          const uint32_t* src = lmask + (buf * LT + p) * LNW;
          uint4* dst = reinterpret_cast<uint4*>(A.cmask + (size_t)row * (A.KP / 32) + slice * LNW);
          dst[0] = uint4{src[0], src[1], src[2], src[3]};
          dst[1] = uint4{src[4], src[5], src[6], src[7]};
        }
      } else if (row < nrows) {
        float M = rb[p * 2];
#pragma unroll
        for (int w2 = 1; w2 < LNW; ++w2) M = fmaxf(M, rb[(w2 * LT + p) * 2]);
        float S = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < LNW; ++w2)
          S += rb[(w2 * LT + p) * 2 + 1] * __builtin_amdgcn_exp2f(rb[(w2 * LT + p) * 2] - M);
        A.P[(size_t)row * A.S + slice] = float2{M, S};
      }
    }
  };

  // ---- logits (log2 units) of the tile in buffer bi: c + a |x|^2 +
  // x . w_hi + x . w_lo, the MFMA chain starting from the constant part.
  // Lane's rows: q = rb * 4 + v <-> tile row rb * 16 + 4 (lane / 16) + v.
  auto logits = [&](int bi, floatx4 (&acc)[2][NT]) {
    const lds_u16* rows = rows_of(bi);
    const lds_f64* xsq = xsq_of(bi);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      floatx4 xs4;  // pass C: four consecutive rows' float32 |x|^2
      if constexpr (STATS) xs4 = *(const lds_floatx4*)((const lds_f32*)xsq + rb * 16 + 4 * (lane >> 4));
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float xs = STATS ? xs4[v] : (float)xsq[rb * 16 + (TR ? (lane & 15) : 4 * (lane >> 4) + v)];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[rb][nt][v] = fmaf(areg[nt][TR ? v : 0], xs, creg[nt][TR ? v : 0]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks) {
      bf16x8 av[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        av[rb] = *(const lds_bf16x8*)(rows + tile_slot(rb * 16 + (lane & 15)) * LRS + ks * 32 + 8 * (lane >> 4));
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          bf16x8 bw;
          if constexpr (WREG) bw = wreg[nt][h][ks];
          else bw = Wl[(((wv * NT + nt) * 2 + h) * KSTEP + ks) * 64 + lane];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[rb][nt] = TR ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw, av[rb], acc[rb][nt], 0, 0, 0)
                             : __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[rb], bw, acc[rb][nt], 0, 0, 0);
        }
    }
  };

  // ---- the rest of a tile (row0: its first row, it: its ordinal in this
  // workgroup, acc: its logits, bi: its buffer); SHARP (a compile-time
  // constant): this wave holds a sharp component
  auto finish = [&](int64_t row0, int it, auto sharp_c, const floatx4 (&acc)[2][NT], int bi) {
    constexpr bool SHARP = decltype(sharp_c)::value;
    const lds_u16* rows = rows_of(bi);
    const lds_f64* xsq = xsq_of(bi);
    const lds_f32* lsb = ls_of(bi);
    if constexpr (PASS == 0) {
      // ---- per-row max and sum of 2^(l - max) over this wave's components
      float lg[2][NT][4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) lg[rb][nt][v] = acc[rb][nt][v];
      if constexpr (SHARP) {
        // sharp components: every score that may come within 60 (log2 units)
        // of the best score of this wave's other components (accurate in
        // expanded form) is recomputed from direct differences in float64
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float ref = kDead;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) ref = fmaxf(ref, eb[nt][v] > 0.f ? kDead : lg[rb][nt][v]);
          ref = rows4_max(ref);
          const int p = rb * 16 + (lane & 15);
          const float xs = (float)xsq[p];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              if (eb[nt][v] > 0.f && row0 + p < nrows && lg[rb][nt][v] + eb[nt][v] * xs + e0[nt][v] >= ref - 60.f) {
                const int k = comp_of(nt, v);
                lg[rb][nt][v] = largek_exact_score(A.mu + (size_t)k * A.D, A.c0[k], A.lam[k], (int)A.D,
                                                   (const unsigned short*)(rows + tile_slot(p) * LRS));
              }
            }
        }
      }
      float m[2], sm[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        m[rb] = lg[rb][0][0];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = 0; v < 4; ++v) m[rb] = fmaxf(m[rb], lg[rb][nt][v]);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) m[rb] = rows4_max(m[rb]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        sm[rb] = __builtin_amdgcn_exp2f(lg[rb][0][0] - m[rb]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int v = (nt == 0 ? 1 : 0); v < 4; ++v) sm[rb] += __builtin_amdgcn_exp2f(lg[rb][nt][v] - m[rb]);
      }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) sm[rb] = rows4_sum(sm[rb]);
      float* rbuf = red + (it & 1) * (LNW * LT * 2);
      if (lane < 16) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          *reinterpret_cast<float2*>(rbuf + (wv * LT + rb * 16 + lane) * 2) = float2{m[rb], sm[rb]};
      }
      return;
    }
    floatx4 lse4[2];
    if constexpr (STATS) {
      // four consecutive rows per load; rows past N hold +inf (r = 0)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) lse4[rb] = *(const lds_floatx4*)(lsb + rb * 16 + 4 * (lane >> 4));
    }
    float lg[8][NT];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) lg[q][nt] = acc[q >> 2][nt][q & 3];
    if constexpr (SHARP) {
      // sharp components: every score that may come within 60 (log2 units)
      // of the row's top, recomputed from direct differences in float64.
      // The reference is the row LSE in pass C and, in pass A, the best
      // score of this wave's other components (accurate in expanded form).
      float ref[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t row = row0 + (q >> 2) * 16 + 4 * (lane >> 4) + (q & 3);
        ref[q] = row < nrows ? lsb[(q >> 2) * 16 + 4 * (lane >> 4) + (q & 3)] : INFINITY;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int p = (q >> 2) * 16 + 4 * (lane >> 4) + (q & 3);
        const float xs = STATS ? ((const lds_f32*)xsq)[p] : (float)xsq[p];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if (eb[nt][0] > 0.f && row0 + p < nrows && lg[q][nt] + eb[nt][0] * xs + e0[nt][0] >= ref[q] - 60.f) {
            const int k = comp_of(nt, 0);
            lg[q][nt] = largek_exact_score(A.mu + (size_t)k * A.D, A.c0[k], A.lam[k], (int)A.D,
                                           (const unsigned short*)(rows + tile_slot(p) * LRS));
          }
        }
      }
    }

    if constexpr (PASS == 1) {
      // ---- candidates: every component whose score may lie within kTopmBand
      // of the row's maximum (its expanded-form error counted twice); the
      // mass 2^(l - max) of the others, per row, for the LSE
      float rem[8];
      uint32_t* mbuf = lmask + (it & 1) * (LT * LNW);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int p = (q >> 2) * 16 + 4 * (lane >> 4) + (q & 3);
        const int64_t row = row0 + p;
        rem[q] = 0.f;
        // top-m: the row maximum (0 for rows past N, which have no candidates);
        // top-k: the row's threshold, a lower bound of its top-k-th score
        const float mr = lsb[p];
        const float floor_l = A.topk ? mr : mr - kTopmBand;
        const float emul = A.topk ? 1.f : 2.f;
        const float xs = (float)xsq[p];
        uint32_t word = 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const bool cand = row < nrows && lg[q][nt] + emul * fmaf(ea[nt], xs, ea0[nt]) >= floor_l;
          if (!cand && row < nrows && !A.topk) rem[q] += __builtin_amdgcn_exp2f(lg[q][nt] - mr);
          // lanes 16g..16g+15 hold row (q, g): their 16 bits are this row's components nt*16 .. +15
          const uint64_t b = __builtin_amdgcn_ballot_w64(cand);
          word |= (uint32_t)((b >> (16 * (lane >> 4))) & 0xFFFFu) << (16 * nt);
        }
        if ((lane & 15) == 0) mbuf[p * LNW + wv] = word;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) rem[q] += dpp_mov<0xB1>(rem[q]);
#pragma unroll
      for (int q = 0; q < 8; ++q) rem[q] += dpp_mov<0x4E>(rem[q]);
#pragma unroll
      for (int q = 0; q < 8; ++q) rem[q] += dpp_mov<0x141>(rem[q]);
#pragma unroll
      for (int q = 0; q < 8; ++q) rem[q] += dpp_mov<0x140>(rem[q]);
      float* rbuf = red + (it & 1) * (LNW * LT * 2);
      if ((lane & 15) == 0) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int p = (q >> 2) * 16 + 4 * (lane >> 4) + (q & 3);
          rbuf[(wv * LT + p) * 2 + 1] = rem[q];
        }
      }
    } else {
      // ---- responsibilities r = 2^(l - LSE), rounded to bf16 once; statistics
      // two magnitude classes, summed by separate MFMAs: a row with r near 1
      // would otherwise round away, in the float32 tile sum, the rows of tiny r
      // that carry a collapsed component's whole variance.  Pairs of r are
      // rounded to bf16 together (B-operand elements 2i, 2i + 1 = rows q = 2i,
      // 2i + 1) and split by 16-bit integer arithmetic: kBigRBits - bits is
      // negative exactly for the big class, and its sign fills the mask.
      bf16x8 bbig[NT], bsmall[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        u32x4 pb, ps;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q0 = 2 * i, q1 = 2 * i + 1;
          const float r0 = __builtin_amdgcn_exp2f(lg[q0][nt] - lse4[q0 >> 2][q0 & 3]);
          const float r1 = __builtin_amdgcn_exp2f(lg[q1][nt] - lse4[q1 >> 2][q1 & 3]);
          const unsigned P = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
          const i16x2 d = (i16x2{kBigRBits - 1, kBigRBits - 1} - __builtin_bit_cast(i16x2, P)) >> 15;
          const unsigned big = P & __builtin_bit_cast(unsigned, d);
          pb[i] = big;
          ps[i] = P ^ big;
        }
        bbig[nt] = __builtin_bit_cast(bf16x8, pb);
        bsmall[nt] = __builtin_bit_cast(bf16x8, ps);
      }
#pragma unroll
      for (int mt = 0; mt < (STATS ? GMX : 1); ++mt) {
        // lane 16 g + i: features 16 mt + i of rows 4 g + e (read 1) and
        // 16 + 4 g + e (read 2), e = 0..3 -- k = 8 g + e and 8 g + 4 + e
        // (slot(16 + r) = 16 + slot(r): read 2 is 16 slots further)
        const lds_u16* src = rows + tile_slot(lane >> 2) * LRS + 16 * mt + 4 * (lane & 3);
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)src);
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(src + 16 * LRS));
        // (the last block's features 136..143 lie past the slot's 136 columns:
        // other bytes of the buffer, which reach only accumulator rows
        // 136..143, never read)
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          sbig[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bbig[nt], sbig[mt][nt], 0, 0, 0);
          ssmall[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bsmall[nt], ssmall[mt][nt], 0, 0, 0);
        }
      }
    }
  };

  // tiles g, g + G, g + 2G, ...: tile i is staged from registers loaded PF
  // tiles earlier, and its slot then starts loading tile i + PF.  Waves with
  // and without sharp components run their own copy of the loop (the same
  // barriers in the same order), so the common one has no exact-score
  // branch; so do 16-byte and element-wise row loads (vec_c).
  auto run = [&](auto sharp_c, auto vec_c) {
    constexpr bool VEC = decltype(vec_c)::value;
    int it = 0;
    Piece pf[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) pf[u] = fetch_piece<PASS, VEC>(A, g + (int64_t)u * A.G, ntiles);
    const int64_t nmine = ntiles > g ? (ntiles - 1 - g) / A.G + 1 : 0;
    if constexpr (!STATS) {
      // One barrier per tile: iteration i stages tile i + 1 (= g + (i + 1) G,
      // buffer and prefetch slot (i + 1) % 2) while it computes tile i.  That
      // buffer was last read by tile i - 1, finished before the barrier that
      // closed iteration i - 1.  The rotating wave combines tile i - 1's
      // per-wave results, written before that barrier; tile i writes the
      // other half of the double buffer, last read by the combine of tile
      // i - 2 in iteration i - 1.
      static_assert(PF == NB, "prefetch slots follow the buffers");
      stage_piece<STATS, FULL>(A, pf[0], (int64_t)g * LT, slice, rows_of(0), xsq_of(0), ls_of(0));
      pf[0] = fetch_piece<PASS, VEC>(A, g + (int64_t)2 * A.G, ntiles);
      __syncthreads();
      for (int64_t i0 = 0; i0 < nmine; i0 += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t i = i0 + u;
          if (i >= nmine) break;
          const int bs = 1 - u;
          stage_piece<STATS, FULL>(A, pf[bs], (g + (i + 1) * A.G) * LT, slice, rows_of(bs), xsq_of(bs),
                             ls_of(bs));
          pf[bs] = fetch_piece<PASS, VEC>(A, g + (i + 3) * A.G, ntiles);
          if (i > 0 && wv == (i & (LNW - 1))) combine((g + (i - 1) * A.G) * LT, red + ((i - 1) & 1) * (LNW * LT * 2));
          floatx4 acc[2][NT];
          logits(u, acc);
          finish((g + i * A.G) * LT, (int)i, sharp_c, acc, u);
          __syncthreads();
          ++it;
        }
      }
    } else {
      // Software-pipelined: iteration i stages tile i + 2, runs the logit
      // MFMAs of tile i + 1 and finishes tile i, with one barrier.  Tile i
      // (= g + i G) lives in buffer i % 3 and was loaded into pf[i % 3].  The
      // buffer staged in iteration i was last read by tile i - 1's statistics,
      // which every wave finished before the barrier that closed iteration
      // i - 1.  Staging and logits past the workgroup's last tile touch only
      // a free buffer and are never used.
      static_assert(PF == NB, "prefetch slots follow the buffers");
      stage_piece<STATS, FULL>(A, pf[0], (int64_t)g * LT, slice, rows_of(0), xsq_of(0), ls_of(0));
      pf[0] = fetch_piece<PASS, VEC>(A, g + (int64_t)3 * A.G, ntiles);
      stage_piece<STATS, FULL>(A, pf[1], (g + (int64_t)A.G) * LT, slice, rows_of(1), xsq_of(1), ls_of(1));
      pf[1] = fetch_piece<PASS, VEC>(A, g + (int64_t)4 * A.G, ntiles);
      __syncthreads();
      // tile i's logits in acc[i % 2]: six tiles per round, so both the
      // buffer (i % 3) and the accumulator index are compile-time constants
      floatx4 acc[2][2][NT];
      logits(0, acc[0]);
      for (int64_t i0 = 0; i0 < nmine; i0 += 6) {
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          const int64_t i = i0 + u;
          if (i >= nmine) break;
          const int b = u % 3, bn = (u + 1) % 3, bs = (u + 2) % 3;
          stage_piece<STATS, FULL>(A, pf[bs], (g + (i + 2) * A.G) * LT, slice, rows_of(bs), xsq_of(bs),
                             ls_of(bs));
          pf[bs] = fetch_piece<PASS, VEC>(A, g + (i + 5) * A.G, ntiles);
          logits(bn, acc[(u + 1) % 2]);
          finish((g + i * A.G) * LT, (int)i, sharp_c, acc[u % 2], b);
          __syncthreads();
          ++it;
        }
      }
    }
    return it;
  };
  // (an empty chunk -- pass C only -- just writes its zero partial)
  int it = 0;
  if (nrows > 0) {
    if (A.vec16)
      it = any_sharp ? run(std::true_type{}, std::true_type{}) : run(std::false_type{}, std::true_type{});
    else
      it = any_sharp ? run(std::true_type{}, std::false_type{}) : run(std::false_type{}, std::false_type{});
  }
  if constexpr (PASS != 2) {
    __syncthreads();
    if (it > 0 && wv == 0) combine((g + (int64_t)(it - 1) * A.G) * LT, red + ((it - 1) & 1) * (LNW * LT * 2));
  }

  if constexpr (STATS) {
    // ---- this workgroup's float64 partial for its slice: part[g][k][2 + DP]
    constexpr int PR = 2 + DP;
    double* part = A.part + (size_t)g * A.KP * PR;
#pragma unroll
    for (int mt = 0; mt < GM; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int k = slice * KSL + (wv * NT + nt) * 16 + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int f = 16 * mt + 4 * (lane >> 4) + v;  // the feature of accumulator row 4 (lane / 16) + v
          double* dst = part + (size_t)k * PR + 2 + f;
          *dst = (A.accumulate ? *dst : 0.0) + ((double)sbig[mt][nt][v] + (double)ssmall[mt][nt][v]);
        }
      }
    // N_k and sum r |x|^2: features 128 and 129..133 of the last block; lane
    // l holds features 128 + 4 (l / 16) + v of component l % 16, so lanes
    // 0..15 take features 132, 133 from lanes 16..31
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      double f[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) f[v] = (double)sbig[GM][nt][v] + (double)ssmall[GM][nt][v];
      const double f4 = __shfl_down(f[0], 16, 64), f5 = __shfl_down(f[1], 16, 64);
      if ((lane >> 4) == 0) {
        const int k = slice * KSL + (wv * NT + nt) * 16 + (lane & 15);
        double* dst = part + (size_t)k * PR;
        dst[0] = (A.accumulate ? dst[0] : 0.0) + f[0];
        dst[1] = (A.accumulate ? dst[1] : 0.0) + (((f[1] + f[2]) + f[3]) + (f4 + f5));
      }
    }
  }
}

// Pass A without per-tile barriers, for full-width rows (D = 128, 16-byte
// aligned): the slice's weights and constants go to LDS once; then each wave
// streams its own row tiles (tile g + G (8 i + w) for wave w), reading a tile's
// rows from memory straight into registers as the B operand of the transposed
// logit MFMA, v_mfma_f32_32x32x16_bf16 (lane l: row l % 32 of each 32-row
// block, dims 16 s + 8 (l / 32) .. +7 of 16-dim step s), the next tile's loads
// in flight while it works.  The 32x32 shape sustains about twice the rate of
// the 16x16x32 one on gfx950, and its accumulator gives each lane 16 of a
// 32-component chunk's scores of one row (components 8 (v / 4) + 4 (l / 32) +
// v % 4), so a row's max and sum over the chunk are an in-lane fold and one
// swap of the wave's halves.  It covers all 256 components of the slice in
// 32-component chunks with a running per-row max and a per-lane running sum
// rescaled to it, so a row's (max, sum) for the slice needs no other wave and
// the waves never wait for each other.
// MODE: 0 = pass A of the fit (slice max and sum), 1 = pass T of the top-m
// (candidate masks and below-band mass against the row maximum), 2 = pass A of
// the top-m (slice max: its last kernel needs only the row maxima and pass T's
// masses), 3 = pass A of the top-k (slice max, and per lane group the maximum
// of score - error bound), 4 = pass T of the top-k (candidates against the
// row's top-k threshold), 5 = the one-pass marking of a row's best component
// alone (k-means labels): candidates against the slice's running maximum, and
// per (row, slice) the slice maximum; no mass (no row maximum needed first).
//
// Why mode 5 loses the best component of no row.  Write E_k(x) for component
// k's two-term error bound, E_s and E_g for the largest bound in slice s and
// over every component.  A slice with no sharp component scores with the hi
// weight term alone, within F = 17 times that bound (bf16 rounding of the
// weight, 2^-9 relative, against 2^-14), a slice with one with both terms
// (F = 1); write l~ for either score, |l~_k - l_k| <= F_s E_k.  Slice s marks k
// when l~_k >= m_run - F_s E_s - 17 E_g, m_run its running maximum at that
// chunk.  With M~ the largest slice maximum (from component j), the best
// component k* has l~_k* >= l_k* - F E_k* >= l_j - F E_k* >= M~ - 17 E_j -
// F E_k*, and m_run <= M~; so k* is marked.  A slice whose maximum m_s lies
// below M~ - 34 E_g cannot hold k* (l_k <= m_s + 17 E_g < M~ - 17 E_g <= l_j);
// the rescoring drops its candidates and scores the others' exactly.
template <int RB, int MODE>
__global__ void __launch_bounds__(512) largek_pass_a_kernel(LargeKArgs A) {
  constexpr bool FUSED = MODE == 5;
  constexpr bool MARK = MODE == 1 || MODE == 4 || FUSED;
  constexpr bool KLB = MODE == 3;  // lane-group lower-bound maxima
  constexpr int DP = 128, KSTEP = DP / 16, NCH = KSA / 32;
  constexpr int PT = 32 * RB;  // rows per tile
  constexpr int NCST = (MARK || KLB) ? 4 : 2;  // per-component error bounds in LDS
  constexpr int WFRAG = NCH * 2 * KSTEP * 64;
  constexpr int CFRAG = NCH * 64;  // the c + a |x|^2 step of each chunk
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 5;  // the wave half: components 4 hl + (v % 4) of each 8
  const int wv = threadIdx.x >> 6;
  const int slice = blockIdx.x / A.G;
  const int g = blockIdx.x % A.G;
  const int64_t nrows = A.N;
  const int64_t ntiles = (nrows + PT - 1) / PT;

  extern __shared__ float lds[];
  bf16x8* Wl = reinterpret_cast<bf16x8*>(lds);
  bf16x8* Wc = Wl + WFRAG;
  float* cst = reinterpret_cast<float*>(Wc + CFRAG);  // eb, e0 (and ea, ea0) of the slice's components
  // pass T: each wave's candidate words of its tile's rows, (row, chunk)
  uint32_t* wbuf = reinterpret_cast<uint32_t*>(cst + NCST * KSA) + (threadIdx.x >> 6) * PT * NCH;
  {
    const uint4* src = reinterpret_cast<const uint4*>(A.W32) + (size_t)slice * WFRAG;
    uint4* dst = reinterpret_cast<uint4*>(Wl);
    for (int i = threadIdx.x; i < WFRAG; i += blockDim.x) dst[i] = src[i];
    const uint4* srcc = reinterpret_cast<const uint4*>(A.W32C) + (size_t)slice * CFRAG;
    for (int i = threadIdx.x; i < CFRAG; i += blockDim.x) reinterpret_cast<uint4*>(Wc)[i] = srcc[i];
    for (int i = threadIdx.x; i < KSA; i += blockDim.x) {
      const int k = slice * KSA + i;
      cst[i] = A.esh[2 * k];
      cst[KSA + i] = A.esh[2 * k + 1];
      if constexpr (MARK || KLB) {
        cst[2 * KSA + i] = A.eall[2 * k];
        cst[3 * KSA + i] = A.eall[2 * k + 1];
      }
    }
  }
  __syncthreads();
  bool any_sharp = false;
  for (int i = lane; i < KSA; i += 64) any_sharp = any_sharp || cst[i] > 0.f;
  any_sharp = __builtin_amdgcn_ballot_w64(any_sharp) != 0;
  // pass T: the largest error bound of the slice's components (slope in |x|^2,
  // offset), so that a row's candidate threshold is one number: the band it
  // gives contains every component's own band, a superset that the exact
  // rescoring sorts out
  float eam = 0.f, ea0m = 0.f;
  // pass T of the top-m: the largest error bound over every component; the
  // row maximum may come from one-term logits (MODE 2), whose error is at most
  // 17 times the two-term bound (bf16 rounding of the weight, 2^-9 relative,
  // against 2^-14 for hi + lo and the float32 sums), and the band widens by it
  float egm = 0.f, eg0m = 0.f;
  if constexpr (MODE == 1 || FUSED) {
    // the waves' maxima meet in the candidate-word area, before its first use
    float* egred = reinterpret_cast<float*>(cst + NCST * KSA);
    for (int i = threadIdx.x; i < A.K; i += blockDim.x) {
      egm = fmaxf(egm, A.eall[2 * i]);
      eg0m = fmaxf(eg0m, A.eall[2 * i + 1]);
    }
    egm = (float)wave_max((double)egm);
    eg0m = (float)wave_max((double)eg0m);
    if (lane == 0) {
      egred[wv] = egm;
      egred[LNW + wv] = eg0m;
    }
    __syncthreads();
    for (int w2 = 0; w2 < LNW; ++w2) {
      egm = fmaxf(egm, egred[w2]);
      eg0m = fmaxf(eg0m, egred[LNW + w2]);
    }
    __syncthreads();
    // the rescoring's slice test takes the same bound (every workgroup
    // forms the same value; the first one stores it)
    if constexpr (FUSED)
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        A.egb[0] = egm;
        A.egb[1] = eg0m;
      }
  }
  if constexpr (MARK) {
    for (int i = lane; i < KSA; i += 64) {
      eam = fmaxf(eam, cst[2 * KSA + i]);
      ea0m = fmaxf(ea0m, cst[3 * KSA + i]);
    }
    eam = (float)wave_max((double)eam);
    ea0m = (float)wave_max((double)ea0m);
  }

  const unsigned short* xb = reinterpret_cast<const unsigned short*>(A.x);
  auto load_rows = [&](int64_t t, bf16x8 (&rv)[RB][KSTEP]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      int64_t row = t * PT + rb * 32 + (lane & 31);
      row = row < nrows ? row : nrows - 1;
#pragma unroll
      for (int ks = 0; ks < KSTEP; ++ks)
        rv[rb][ks] = *reinterpret_cast<const bf16x8*>(xb + row * A.ld_x + ks * 16 + 8 * hl);
    }
  };
  // the slice component of accumulator entry v of chunk cc
  auto comp = [&](int cc, int v) { return cc * 32 + 8 * (v >> 2) + 4 * hl + (v & 3); };
  // slices with and without a sharp component run their own copy of the row
  // loop, so the common one carries no exact-score code
  auto rows_loop = [&](auto sharp_c) {
  constexpr bool SHARP = decltype(sharp_c)::value;
  // weight terms per logit: the top-m's row maxima (MODE 2) and the one-pass
  // marking (MODE 5) take the hi term alone where no sharp component needs its
  // exact score (the bands widen by that error); everything else takes hi + lo
  constexpr int NHT = ((MODE == 2 || MODE == 5) && !SHARP) ? 1 : 2;
  int64_t t = g + (int64_t)A.G * wv;
  bf16x8 nxt[RB][KSTEP];
  if (t < ntiles) load_rows(t, nxt);
  for (; t < ntiles; t += (int64_t)A.G * LNW) {
    bf16x8 rv[RB][KSTEP];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ks = 0; ks < KSTEP; ++ks) rv[rb][ks] = nxt[rb][ks];
    if (t + (int64_t)A.G * LNW < ntiles) load_rows(t + (int64_t)A.G * LNW, nxt);
    // |x|^2 of the lane's rows: exact (float64) in slice 0, which stores it
    // for pass B, pass C and the top-m rescoring; float32 elsewhere and in
    // pass T, which stores nothing
    const bool exact = (!MARK || FUSED) && slice == 0;
    float xs[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (exact) {
        double q = 0.0;
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = (float)rv[rb][ks][e];
            q += (double)(f * f);
          }
        q = halves_sum_f64(q);
        xs[rb] = (float)q;
        const int64_t row = t * PT + rb * 32 + lane;
        if (lane < 32 && row < nrows) A.xsq[row] = q;
      } else {
        float q = 0.f;
#pragma unroll
        for (int ks = 0; ks < KSTEP; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = (float)rv[rb][ks][e];
            q = fmaf(f, f, q);
          }
        xs[rb] = halves_sum(q);
      }
    }
    // the B operand of the chunk's c + a |x|^2 step: lane l carries row
    // l % 32's features (1, 1, 1, x1, x2, x3, x1, x2 | x1, 0, ...), x1 + x2 + x3
    // the bf16 terms of |x|^2 (successive remainders), against the prologue's
    // (c1, c2, c3, a1, a1, a1, a2, a2 | a3, 0, ...)
    bf16x8 cfr[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float q = xs[rb];
      const __bf16 x1 = (__bf16)q;
      const float q2 = q - (float)x1;
      const __bf16 x2 = (__bf16)q2;
      const __bf16 x3 = (__bf16)(q2 - (float)x2);
      const __bf16 one = (__bf16)1.f, zero = (__bf16)0.f;
      cfr[rb] = hl == 0 ? bf16x8{one, one, one, x1, x2, x3, x1, x2} : bf16x8{x1, zero, zero, zero, zero, zero, zero, zero};
    }
    float M[RB], Sl[RB], R[RB], Lb[RB][2];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      M[rb] = kDead;
      Sl[rb] = 0.f;
      R[rb] = kDead;
      Lb[rb][0] = Lb[rb][1] = kDead;
    }
    // pass T: the row maximum (pass B) is the reference of the candidate band
    // and of the sharp rescoring; rows past N have no candidates and no mass
    float mr[RB], thr[RB];
    bool live[RB];
    if constexpr (MARK) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int64_t row = t * PT + rb * 32 + (lane & 31);
        live[rb] = row < nrows;
        if constexpr (FUSED) {
          // the band below the running maximum (rows past N: none)
          thr[rb] = live[rb] ? (NHT == 1 ? 17.f : 1.f) * fmaf(eam, xs[rb], ea0m) + 17.f * fmaf(egm, xs[rb], eg0m)
                             : -INFINITY;
          continue;
        }
        mr[rb] = A.mrow[live[rb] ? row : nrows - 1];
        R[rb] = mr[rb];
        if constexpr (MODE == 4)
          thr[rb] = live[rb] ? A.kthr[row] : INFINITY;  // a lower bound of the row's top-k-th score
        else
          thr[rb] = live[rb] ? mr[rb] - kTopmBand - 2.f * fmaf(eam, xs[rb], ea0m) - 17.f * fmaf(egm, xs[rb], eg0m)
                             : INFINITY;
      }
    }
#pragma unroll 1
    for (int cc = 0; cc < NCH; ++cc) {
      floatx16 acc[RB];
      {
        const bf16x8 wc = Wc[cc * 64 + lane];
        floatx16 z;
#pragma unroll
        for (int v = 0; v < 16; ++v) z[v] = 0.f;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wc, cfr[rb], z, 0, 0, 0);
      }
#pragma unroll
      for (int ks = 0; ks < KSTEP; ++ks)
#pragma unroll
        for (int h = 0; h < NHT; ++h) {
          const bf16x8 bw = Wl[((cc * 2 + h) * KSTEP + ks) * 64 + lane];
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            acc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw, rv[rb][ks], acc[rb], 0, 0, 0);
        }
      if constexpr (SHARP) {
        // sharp components: scores that may come within 60 (log2 units) of the
        // best other score of the row seen so far in the slice, again exactly
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if constexpr (!MARK || FUSED) {
            float r = R[rb];
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (!(cst[comp(cc, v)] > 0.f)) r = fmaxf(r, acc[rb][v]);
            R[rb] = halves_max(r);
          }
          const int64_t row = t * PT + rb * 32 + (lane & 31);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kl = comp(cc, v);
            const float eb = cst[kl], e0 = cst[KSA + kl];
            if (eb > 0.f && row < nrows && acc[rb][v] + eb * xs[rb] + e0 >= R[rb] - 60.f) {
              const int k = slice * KSA + kl;
              acc[rb][v] = largek_exact_score(A.mu + (size_t)k * A.D, A.c0[k], A.lam[k], (int)A.D, xb + row * A.ld_x);
            }
          }
        }
      }
      if constexpr (FUSED) {
        // running maximum of the slice per row; a component is a candidate
        // when it comes within the row's error band of that maximum (thr)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          float cm = acc[rb][0];
#pragma unroll
          for (int v = 1; v < 16; ++v) cm = fmaxf(cm, acc[rb][v]);
          cm = halves_max(cm);
          const float Mn = fmaxf(M[rb], cm);
          M[rb] = Mn;
          const float th = Mn - thr[rb];
          uint32_t word = 0;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const bool cand = acc[rb][v] >= th;  // never for rows past N (th = +inf)
            word |= cand ? (1u << (8 * (v >> 2) + (v & 3))) : 0u;
          }
          word = halves_or(word << (4 * hl));
          if (lane < 32) wbuf[(rb * 32 + lane) * NCH + cc] = word;
        }
        continue;
      }
      if constexpr (MARK) {
        // candidates: every component whose score may lie within kTopmBand of
        // the row's maximum (the slice's largest expanded-form error counted
        // twice); the mass 2^(l - max) of the others; bit j of word (row, cc)
        // is component cc 32 + j of the slice.  Every component adds
        // 2^(min(l, thr) - max): the others their own mass, each candidate
        // 2^(thr - max), taken off once per row at the end of the tile (all
        // these terms lie below 2^-20 of the row's mass, so the difference
        // loses nothing that matters).  Rows past N (thr = +inf) are never
        // written.
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          uint32_t word = 0;
          float rem = 0.f;
          const float tm = thr[rb] - mr[rb];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            bool cand;  // never for rows past N (thr = +inf)
            if constexpr (MODE == 4) {
              // top-k: the score's upper end reaches the row's threshold
              const int kl = comp(cc, v);
              cand = acc[rb][v] + fmaf(cst[2 * KSA + kl], xs[rb], cst[3 * KSA + kl]) >= thr[rb];
            } else {
              cand = acc[rb][v] >= thr[rb];
              rem += __builtin_amdgcn_exp2f(fminf(acc[rb][v] - mr[rb], tm));
            }
            // this half's bits first, moved to 4 (l / 32) below
            word |= cand ? (1u << (8 * (v >> 2) + (v & 3))) : 0u;
          }
          word = halves_or(word << (4 * hl));
          Sl[rb] += rem;
          if (lane < 32) wbuf[(rb * 32 + lane) * NCH + cc] = word;
        }
        continue;
      }
      // running max per row, and the lane's sum rescaled to it
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float cm = acc[rb][0];
#pragma unroll
        for (int v = 1; v < 16; ++v) cm = fmaxf(cm, acc[rb][v]);
        if constexpr (KLB) {
          // the largest lower end, score - its error bound, of this lane's
          // entries 0..7 and 8..15: four disjoint lane groups per row
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int kl = comp(cc, v);
            Lb[rb][v >> 3] = fmaxf(Lb[rb][v >> 3], acc[rb][v] - fmaf(cst[2 * KSA + kl], xs[rb], cst[3 * KSA + kl]));
          }
        }
        cm = halves_max(cm);
        if constexpr (MODE == 2 || MODE == 3) {
          M[rb] = fmaxf(M[rb], cm);
          continue;
        }
        const float Mn = fmaxf(M[rb], cm);
        float s = Sl[rb] * __builtin_amdgcn_exp2f(M[rb] - Mn);
#pragma unroll
        for (int v = 0; v < 16; ++v) s += __builtin_amdgcn_exp2f(acc[rb][v] - Mn);
        Sl[rb] = s;
        M[rb] = Mn;
      }
    }
    if constexpr (KLB) {
      // lane group 2 (lane / 32) + j of row rb 32 + lane % 32: entry 2 (lane / 32) + j of (row, slice)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int64_t row = t * PT + rb * 32 + (lane & 31);
        if (row < nrows)
          *reinterpret_cast<float2*>(reinterpret_cast<float*>(A.lmx) + ((size_t)row * A.S + slice) * 4 + 2 * hl) =
              float2{Lb[rb][0], Lb[rb][1]};
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float S = FUSED ? 0.f : halves_sum(Sl[rb]);
      const int64_t row = t * PT + rb * 32 + lane;
      if (lane < 32 && row < nrows) {
        if constexpr (MARK) {
          // this slice's below-band mass (mode 5: its maximum) and its 8
          // candidate words of the row
          const uint32_t* src = wbuf + (rb * 32 + lane) * NCH;
          if constexpr (FUSED) {
            A.P[(size_t)row * A.S + slice] = float2{M[rb], 0.f};
          } else {
            float Sb = S;
            if constexpr (MODE == 1) {
              int nc = 0;
#pragma unroll
              for (int c = 0; c < NCH; ++c) nc += __popc(src[c]);
              Sb = fmaxf(S - (float)nc * __builtin_amdgcn_exp2f(thr[rb] - mr[rb]), 0.f);
            }
            A.prem[(size_t)row * A.S + slice] = Sb;
          }
          uint4* dst = reinterpret_cast<uint4*>(A.cmask + (size_t)row * (A.KP / 32) + slice * NCH);
          dst[0] = uint4{src[0], src[1], src[2], src[3]};
          dst[1] = uint4{src[4], src[5], src[6], src[7]};
        } else {
          A.P[(size_t)row * A.S + slice] = float2{M[rb], (MODE == 2 || MODE == 3) ? 1.f : S};
        }
      }
    }
  }
  };
  if (any_sharp) rows_loop(std::true_type{});
  else rows_loop(std::false_type{});
}

// 32-row blocks per tile of the barrier-free pass A: every weight fragment
// read from LDS feeds kPassARB MFMAs
constexpr int kPassARB = 2;

size_t largek_pass_a_lds_bytes(int mode) {
  const bool mark = mode == 1 || mode == 4 || mode == 5;
  return (size_t)(KSA / 32) * (2 * (128 / 16) + 1) * 64 * 16 + ((mark || mode == 3) ? 4 : 2) * KSA * sizeof(float) +
         (mark ? (size_t)LNW * 32 * kPassARB * (KSA / 32) * sizeof(uint32_t) : 0);
}

// Pass B: per row, combine the slices' (max, sum) into the LSE (log2 units);
// each workgroup also sums its rows' LSE (natural log) into its LL partial.
// The rows from N up to the next multiple of the row tile get LSE = +inf, so
// that pass C reads a tile's LSE values unguarded and gets r = 0 for them.
__global__ void __launch_bounds__(256) largek_lse_kernel(LargeKArgs A) {
  constexpr double LN2 = 0.69314718055994530942;
  __shared__ double red[256];
  double ll = 0.0;
  const int64_t npad = (A.N + LT - 1) / LT * LT;
  for (int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; row < npad;
       row += (int64_t)gridDim.x * blockDim.x) {
    if (row >= A.N) {
      A.lse[row] = INFINITY;
      if (A.ext) reinterpret_cast<u16x8*>(A.ext)[row] = u16x8{(unsigned short)0x3F80, 0, 0, 0, 0, 0, 0, 0};
      continue;
    }
    if (A.ext) {
      // the statistics features of pass C: 1 and |x|^2 as five bf16 terms,
      // each the bf16 rounding of the float64 remainder so far (every
      // remainder exact in float64; 40 bits, as many as |x|^2 of a bf16 row
      // can need), so that N_k and sum r |x|^2 come out of both magnitude
      // classes like sum r x, and a component collapsed onto one row gets
      // them exactly
      u16x8 ext = u16x8{(unsigned short)0x3F80, 0, 0, 0, 0, 0, 0, 0};
      double q = A.xsq[row];
#pragma unroll
      for (int e = 1; e <= 5; ++e) {
        const __bf16 h = (__bf16)(float)q;
        ext[e] = __builtin_bit_cast(unsigned short, h);
        q -= (double)(float)h;
      }
      reinterpret_cast<u16x8*>(A.ext)[row] = ext;
    }
    const float2* P = A.P + (size_t)row * A.S;
    float M = P[0].x;
    for (int s = 1; s < A.S; ++s) M = fmaxf(M, P[s].x);
    double S = 0.0;
    for (int s = 0; s < A.S; ++s) S += (double)P[s].y * exp2((double)P[s].x - (double)M);
    const double l2 = (double)M + log2(S);
    A.lse[row] = (float)l2;
    ll += l2 * LN2;
    if (A.topm) A.mrow[row] = M;
    if (A.topk) {
      // the m-th largest of the 4 S lane-group maxima of score - error bound:
      // m different components reach it, so it bounds the row's m-th best true
      // score from below (never below the dead-component floor, so padding
      // never becomes a candidate); without them every live component is one
      float top[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) top[j] = kDead;
      if (A.lmx) {
        const float* lv = reinterpret_cast<const float*>(A.lmx + (size_t)row * A.S);
        for (int i = 0; i < 4 * A.S; ++i) {
          float v = lv[i];
#pragma unroll
          for (int j = 0; j < 16; ++j) {  // insert into the descending list
            const float hi = fmaxf(top[j], v), lo = fminf(top[j], v);
            top[j] = hi;
            v = lo;
          }
        }
      }
      float th = kDead;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j == A.m - 1) th = top[j];
      A.kthr[row] = fmaxf(th, 0.5f * kDead);
    }
  }
  red[threadIdx.x] = ll;
  __syncthreads();
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int i = 0; i < (int)blockDim.x; ++i) s += red[i];
    A.llpart[blockIdx.x] = (A.accumulate ? A.llpart[blockIdx.x] : 0.0) + s;
  }
}

// Prologue: weights w = lambda mu log2(e) split into bf16 hi + lo in the
// B-fragment order of v_mfma_f32_16x16x32_bf16 (16-component tiles) and in
// the A-operand order of v_mfma_f32_32x32x16_bf16 (32-component tiles), the
// constants c, a, c0, lambda (float64) and the sharp-component error bounds.
// grid: KP blocks of 64 threads.
__global__ void __launch_bounds__(64) largek_prologue_kernel(int D, int K, int DP, const float* __restrict__ w,
                                                             const float* __restrict__ mu,
                                                             const float* __restrict__ cv, __bf16* __restrict__ W,
                                                             __bf16* __restrict__ W32, __bf16* __restrict__ W32C,
                                                             double* __restrict__ c, double* __restrict__ a,
                                                             double* __restrict__ c0, double* __restrict__ lamk,
                                                             float* __restrict__ esh, float* __restrict__ eall,
                                                             double* __restrict__ mmk, double2* __restrict__ kconst) {
  constexpr double kLog2e = 1.4426950408889634074;
  constexpr double kLog2Pi = 1.8378770664093454836;
  const int k = blockIdx.x, tid = threadIdx.x;
  const int KSTEP = DP / 32;
  const int kt = k / 16, col = k % 16;
  const bool live = k < K;
  const double var = live ? (double)cv[k] : 1.0;
  const bool ok = live && var > 0.0 && !isinf(var);
  const double lam = 1.0 / var;
  for (int f = tid; f < DP; f += blockDim.x) {
    const double val = (ok && f < D) ? lam * (double)mu[(size_t)k * D + f] * kLog2e : 0.0;
    const __bf16 hi = (__bf16)val;
    const __bf16 lo = (__bf16)(val - (double)(float)hi);
    const int ks = f / 32, j = f % 32, grp = j / 8, e = j % 8;
    const int lane = grp * 16 + col;
    for (int h = 0; h < 2; ++h) {
      const size_t idx = ((size_t)kt * 2 + h) * KSTEP + ks;
      W[(idx * 64 + lane) * 8 + e] = h == 0 ? hi : lo;
    }
    // the 32x32x16 operand order: lane 32 (j / 8) + k % 32 of 16-dim step
    // f / 16 holds dims 16 (f / 16) + 8 (j / 8) .. +7, j = f % 16
    const int ks2 = f / 16, j2 = f % 16;
    const int lane2 = (j2 / 8) * 32 + k % 32;
    for (int h = 0; h < 2; ++h) {
      const size_t idx = ((size_t)(k / 32) * 2 + h) * (DP / 16) + ks2;
      W32[(idx * 64 + lane2) * 8 + j2 % 8] = h == 0 ? hi : lo;
    }
  }
  __shared__ double ca[2];  // c and a of the component, for the constant step below
  if (tid == 0 && !ok) {
    c[k] = c0[k] = kDead;
    a[k] = lamk[k] = 0.0;
    esh[2 * k] = esh[2 * k + 1] = 0.f;
    eall[2 * k] = eall[2 * k + 1] = 0.f;
    mmk[k] = 0.0;
    kconst[k] = double2{(double)kDead, 0.0};
    ca[0] = kDead;
    ca[1] = 0.0;
  } else if (tid == 0) {
    double mm = 0.0;
    for (int d = 0; d < D; ++d) mm += (double)mu[(size_t)k * D + d] * (double)mu[(size_t)k * D + d];
    c0[k] = (log((double)w[k]) - 0.5 * (D * kLog2Pi + D * log(var))) * kLog2e;
    c[k] = c0[k] - 0.5 * lam * mm * kLog2e;
    a[k] = -0.5 * lam * kLog2e;
    lamk[k] = lam;
    // the expanded score's terms reach lambda (|mu|^2 + |x|^2) log2(e); the
    // bf16 split of the weights and the float32 sums leave an error below
    // 2^-14 of that.  Components whose terms exceed kSharpLowp are rescored.
    const bool sharp = lam * (mm + D * var) > kSharpLowp;
    const double ea = ldexp(lam * kLog2e, -14);
    const double eb = sharp ? ea : 0.0;
    esh[2 * k] = (float)eb;
    esh[2 * k + 1] = (float)(eb * mm);
    eall[2 * k] = (float)ea;
    eall[2 * k + 1] = (float)(ea * mm);
    mmk[k] = mm;
    kconst[k] = double2{c0[k] - 0.5 * lam * mm * kLog2e, lam * kLog2e};
    ca[0] = c[k];
    ca[1] = a[k];
  }
  __syncthreads();
  // pass A's c + a |x|^2 as one more 32x32x16 MFMA step (A operand, the
  // 32-component tile's order): slots (c1, c2, c3, a1, a1, a1, a2, a2 | a3,
  // 0, ...) against the row's (1, 1, 1, x1, x2, x3, x1, x2 | x1, 0, ...), c and a
  // split into three bf16 terms each (successive remainders), every product
  // exact in the float32 accumulation
  if (tid < 16) {
    __bf16 ct[3], at[3];
    double cr = ca[0], ar = ca[1];
    for (int i = 0; i < 3; ++i) {
      ct[i] = (__bf16)cr;
      cr -= (double)(float)ct[i];
      at[i] = (__bf16)ar;
      ar -= (double)(float)at[i];
    }
    const int j = tid;
    __bf16 val = (__bf16)0.f;
    if (j < 3) val = ct[j];
    else if (j < 6) val = at[0];
    else if (j < 8) val = at[1];
    else if (j == 8) val = at[2];
    W32C[(((size_t)(k / 32)) * 64 + (j / 8) * 32 + k % 32) * 8 + j % 8] = val;
  }
}

hipError_t launch_largek(const Plan& p, const LargeKArgs& a0, const float* w, const float* mu, const float* cv,
                         hipStream_t s) {
  LargeKArgs a = a0;
  hipLaunchKernelGGL(largek_prologue_kernel, dim3((unsigned)p.KP), dim3(64), 0, s, (int)p.D, (int)p.K, p.DP, w, mu,
                     cv, reinterpret_cast<__bf16*>(const_cast<void*>(a.W)),
                     reinterpret_cast<__bf16*>(const_cast<void*>(a.W32)),
                     reinterpret_cast<__bf16*>(const_cast<void*>(a.W32C)), const_cast<double*>(a.c),
                     const_cast<double*>(a.a), const_cast<double*>(a.c0), const_cast<double*>(a.lam),
                     const_cast<float*>(a.esh), const_cast<float*>(a.eall),
                     const_cast<double*>(a.mmk), const_cast<double2*>(a.kconst));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto kA = largek_kernel<128, 0>;
  auto kC = p.D == 128 ? largek_kernel<128, 2, true> : largek_kernel<128, 2, false>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)kA, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    (void)hipFuncSetAttribute((const void*)largek_kernel<128, 2, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytes);
    (void)hipFuncSetAttribute((const void*)largek_kernel<128, 2, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytes);
    (void)hipFuncSetAttribute((const void*)largek_pass_a_kernel<kPassARB, 0>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytes);
    attr_set = true;
  }
  const int64_t N = a.N;
  const unsigned char* x0 = reinterpret_cast<const unsigned char*>(a.x);
  for (int64_t r0 = 0, chunk = 0; r0 < N || (N == 0 && chunk == 0); r0 += p.chunk_rows, ++chunk) {
    LargeKArgs ac = a;
    ac.N = std::min<int64_t>(p.chunk_rows, N - r0);
    ac.x = x0 + (size_t)r0 * p.ld_x * 2;
    ac.accumulate = chunk > 0;
    if (ac.N > 0) {
      ac.G = p.GbA;
      if (p.D == 128 && ac.vec16)
        hipLaunchKernelGGL((largek_pass_a_kernel<kPassARB, 0>), dim3((unsigned)(p.S * p.GbA)), dim3(64 * LNW),
                           largek_pass_a_lds_bytes(0), s, ac);
      else
        hipLaunchKernelGGL(kA, dim3((unsigned)(p.S * p.GbA)), dim3(64 * LNW), p.lds_a, s, ac);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(largek_lse_kernel, dim3((unsigned)p.lse_blocks), dim3(256), 0, s, ac);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    ac.G = p.Gb;
    hipLaunchKernelGGL(kC, dim3((unsigned)(p.SC * p.Gb)), dim3(64 * LNW), p.lds_c, s, ac);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (N == 0) break;
  }
  return hipSuccess;
}


// Top-m, last step: one wave per row.  The row's candidates (the set bits of
// its mask, in increasing component order) are scored in batches, 16 lanes to
// a candidate (lane i of a group holds dims 8i..8i+7 of the row), sixteen at a
// time, exactly in float64: c0 - (lambda/2) log2(e) (|x|^2 - 2 x . mu +
// |mu|^2), every product of a bf16 x and a float32 mu being exact in float64,
// so the expanded form loses nothing at float64 precision.  The scores go to
// LDS; each batch updates the row's running (max, sum) and its best m (kept
// in LDS ahead of the next batch's scores), chosen by m rounds of a
// wave-wide best.  The LSE adds pass T's below-band mass.  Rank 1 is always
// kept, ranks 2..m while r >= thr.  Every step runs in a fixed order.
constexpr int kTopmMaxM = 16;
constexpr int kBatch = 256;                       // scores per batch
constexpr int kSlots = kTopmMaxM + kBatch;        // running best m, then the batch
constexpr int kPer = (kSlots + 63) / 64;          // slots per lane in the selection
constexpr int kMaskSlots = kLargeKMaxK / 32 / 64;  // mask words per lane at the largest K
// rows (one wave each) per workgroup of the rescoring kernel: one, so that a
// row with many candidates holds no other row's slot on the CU (4 rows per
// workgroup: 141.6 ms per IVF top-m pass; 1 row: 121.0 ms; 1 row at four
// waves per SIMD, registers capped at 128: 117.7 ms)
constexpr int kFinalRows = 1;

// 2^d for d <= 0 to about 1e-7 relative: float exp2 of the float part and a
// first-order correction for the rest of d
__device__ __forceinline__ double exp2_acc(double d) {
  const float h = (float)d;
  const double l = d - (double)h;
  return (double)__builtin_amdgcn_exp2f(h) * (1.0 + l * 0.69314718055994530942);
}

__device__ __forceinline__ int wave_excl_scan(int v, int lane, int& total) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  total = __shfl(x, 63, 64);
  return x - v;
}

// One row by the whole wave (any number of candidates): L, KK (kSlots each)
// and LST (kBatch) are the wave's LDS areas.
__device__ __forceinline__ void topm_row_wave(const LargeKArgs& A, int64_t row, double* L, int* KK,
                                           unsigned short* LST) {
  constexpr double LN2 = 0.69314718055994530942;
  const int lane = threadIdx.x & 63;
  const int grp = lane >> 4, li = lane & 15;
  const int m = A.m;
  const int D = (int)A.D;
  const int nwords = A.KP / 32;
  // this lane's words of the row's candidate mask: lanes cover words lane*wpl .. +wpl-1
  const int wpl = (nwords + 63) / 64;
  // one-pass marking (best component alone): the row maximum over the slice
  // maxima and the slices that can hold the best component (as in
  // largek_topm_final4_kernel); no mass outside the candidates
  uint64_t qm = ~0ull;
  double mref = 0.0, remf = 0.0;
  if (A.fused_t) {
    const float ms = lane < A.S ? A.P[(size_t)row * A.S + lane].x : kDead;
    const float mx = (float)wave_max((double)ms);
    const float bq = 34.f * fmaf(A.egb[0], (float)A.xsq[row], A.egb[1]);
    qm = __builtin_amdgcn_ballot_w64(lane < A.S && ms >= mx - bq);
    mref = mx;
  }
  uint32_t mw[kMaskSlots];
  int mycount = 0;
#pragma unroll
  for (int t = 0; t < kMaskSlots; ++t) {
    const int wi = lane * wpl + t;
    uint32_t wd = (t < wpl && wi < nwords) ? A.cmask[(size_t)row * nwords + wi] : 0u;
    if (wi * 32 + 32 > A.K) wd &= wi * 32 >= A.K ? 0u : (1u << (A.K - wi * 32)) - 1u;  // padding is never a candidate
    if (!((qm >> ((wi * 32) / KSA)) & 1ull)) wd = 0u;  // a far slice
    mw[t] = wd;
    mycount += __popc(mw[t]);
  }
  int total;
  const int mybase = wave_excl_scan(mycount, lane, total);
  // this lane's 8 dims of the row
  const unsigned short* xr = reinterpret_cast<const unsigned short*>(A.x) + row * A.ld_x;
  double xv[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * li + e;
    xv[e] = d < D ? (double)__uint_as_float((unsigned)xr[d] << 16) : 0.0;
  }
  const bool vec = (D & 7) == 0 && ((uintptr_t)A.mu & 15) == 0;
  const int doff = vec ? min(8 * li, D - 8) : 0;
  const double xsq = A.xsq[row];
  if (lane < kTopmMaxM) {
    L[lane] = -INFINITY;
    KK[lane] = 0x7fffffff;
  }
  double Mrun = -INFINITY, Srun = 0.0;
  for (int b0 = 0; b0 < total; b0 += kBatch) {
    const int nb = min(kBatch, total - b0);
    // the batch's component list, in increasing component order
    {
      int r = mybase;
#pragma unroll
      for (int t = 0; t < kMaskSlots; ++t) {
        uint32_t w = mw[t];
        const int kbase = (lane * wpl + t) * 32;
        while (w) {
          const int bit = __builtin_ctz(w);
          w &= w - 1;
          if (r >= b0 && r < b0 + nb) LST[r - b0] = (unsigned short)(kbase + bit);
          ++r;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 8 candidates per step (two per 16-lane group), their loads issued
    // together (indices past the batch repeat its last entry; lanes past D
    // read inside the row and hold x = 0)
    constexpr int U = 2;
    for (int i0 = 0; i0 < nb; i0 += 4 * U) {
      int ku[U];
#pragma unroll
      for (int u = 0; u < U; ++u) ku[u] = LST[min(i0 + 4 * u + grp, nb - 1)];
      double2 cu[U];
      float4 m0[U], m1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cu[u] = A.kconst[ku[u]];
        const float* mu = A.mu + (size_t)ku[u] * D;
        if (vec) {
          m0[u] = *reinterpret_cast<const float4*>(mu + doff);
          m1[u] = *reinterpret_cast<const float4*>(mu + doff + 4);
        } else {
          float t[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = (8 * li + e < D) ? mu[8 * li + e] : 0.f;
          m0[u] = float4{t[0], t[1], t[2], t[3]};
          m1[u] = float4{t[4], t[5], t[6], t[7]};
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        double dot = xv[0] * (double)m0[u].x + xv[1] * (double)m0[u].y + xv[2] * (double)m0[u].z +
                     xv[3] * (double)m0[u].w + xv[4] * (double)m1[u].x + xv[5] * (double)m1[u].y +
                     xv[6] * (double)m1[u].z + xv[7] * (double)m1[u].w;
        dot = row16_sum_f64(dot);
        const int i = i0 + 4 * u + grp;
        if (li == 0 && i < nb) {
          // score = (c0 - lambda log2(e) |mu|^2 / 2) + lambda log2(e) (x . mu - |x|^2 / 2)
          L[kTopmMaxM + i] = cu[u].x + cu[u].y * (dot - 0.5 * xsq);
          KK[kTopmMaxM + i] = ku[u];
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // this batch's slots (and the running best m) into registers; only the
    // first tcnt of each lane's kPer slots can hold entries
    const int tcnt = (kTopmMaxM + nb + 63) / 64;
    double vl[kPer];
    int vk[kPer];
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      vl[t] = -INFINITY;
      vk[t] = 0x7fffffff;
      if (t < tcnt) {
        const int j = lane + 64 * t;
        if (j < kTopmMaxM + nb) {
          vl[t] = L[j];
          vk[t] = KK[j];
        }
      }
    }
    // running max and sum over the batch's scores
    double lmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < kPer; ++t)
      if (t < tcnt && lane + 64 * t >= kTopmMaxM) lmax = fmax(lmax, vl[t]);
    const double Mb = wave_max(lmax);
    double ssum = 0.0;
#pragma unroll
    for (int t = 0; t < kPer; ++t)
      if (t < tcnt && lane + 64 * t >= kTopmMaxM && vl[t] > -INFINITY) ssum += exp2_acc(vl[t] - Mb);
    const double Sb = wave_sum(ssum);
    const double Mn = fmax(Mrun, Mb);
    Srun = (Mrun > -INFINITY ? Srun * exp2(Mrun - Mn) : 0.0) + Sb * exp2(Mb - Mn);
    Mrun = Mn;
    // the best m of the running list and the batch
    double rl = -INFINITY;
    int rk = 0x7fffffff;
    for (int j = 0; j < m; ++j) {
      double bl = -INFINITY;
      int bk = 0x7fffffff;
      int bt = -1;
#pragma unroll
      for (int t = 0; t < kPer; ++t)
        if (t < tcnt && before(vl[t], vk[t], bl, bk)) {
          bl = vl[t];
          bk = vk[t];
          bt = t;
        }
      double wl = bl;
      int wk = bk;
      wave_best(wl, wk);
#pragma unroll
      for (int t = 0; t < kPer; ++t)
        if (t < tcnt && bt == t && bk == wk && bl == wl) vl[t] = -INFINITY, vk[t] = 0x7fffffff;
      if (lane == j) {
        rl = wl;
        rk = wk;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (lane < kTopmMaxM) {
      L[lane] = rl;
      KK[lane] = rk;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  double lse;
  if (A.topk) {
    // top-k: the log-sum-exp of the kept m (the best first)
    double S = 0.0;
    for (int j = 0; j < m; ++j)
      if (KK[j] < A.K) S += exp2(L[j] - L[0]);
    lse = L[0] + log2(S);
  } else {
    // below-band mass of every slice, relative to the expanded-form maximum
    const double rem = A.fused_t ? remf : wave_sum(lane < A.S ? (double)A.prem[(size_t)row * A.S + lane] : 0.0);
    const double S = Srun + rem * exp2((A.fused_t ? mref : (double)A.mrow[row]) - Mrun);
    lse = Mrun + log2(S);
  }
  if (lane == 0) {
    int c = 0;
    for (int j = 0; j < m; ++j) {
      const double bl = L[j];
      const int bk = KK[j];
      const double r = bk < A.K ? exp2(bl - lse) : 0.0;
      const bool keep = bk < A.K && (A.topk || j == 0 || r >= (double)A.thr) && c == j;
      A.idx[row * m + j] = keep ? bk : -1;
      A.resp[row * m + j] = keep ? (float)r : 0.f;
      if (keep) ++c;
    }
    if (A.count) A.count[row] = c;
    if (A.logp) A.logp[row] = (float)(lse * LN2);
  }
}

// The rescoring kernel: one wave per four rows, 16 lanes (a DPP row) per row.
// A group counts its row's candidates (16-lane scan of the mask words'
// popcounts); a row with at most kLight of them is scored by the group alone
// (each candidate's 128-term float64 dot product split over the 16 lanes,
// two candidates' loads in flight), its best m picked by m rounds of a
// 16-lane best, LSE and outputs as in topm_row_wave.  Four independent rows per wave keep four chains of
// dependent loads in flight where one row per wave kept one.
constexpr int kLight = 32;

__global__ void __launch_bounds__(64) largek_topm_final4_kernel(LargeKArgs A) {
  constexpr double LN2 = 0.69314718055994530942;
  __shared__ unsigned short light[4][kLight];
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, li = lane & 15;
  const int64_t row = (int64_t)blockIdx.x * 4 + g;
  const bool live = row < A.N;
  const int m = A.m;
  const int D = (int)A.D;
  const int K = A.K;
  const int nwords = A.KP / 32;
  const int64_t rc = live ? row : A.N - 1;
  // ---- one-pass marking (best component alone): the row maximum over the
  // slice maxima and the slices that can hold the best component (slice bits
  // qm; the others' candidates are dropped); no mass outside the candidates
  uint64_t qm = ~0ull;
  float mref = 0.f;
  const double remf = 0.0;
  if (A.fused_t) {
    float ms[4];
    float mx = kDead;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = li + 16 * j;
      ms[j] = sl < A.S ? A.P[(size_t)rc * A.S + sl].x : kDead;
      mx = fmaxf(mx, ms[j]);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
    const float bq = 34.f * fmaf(A.egb[0], (float)A.xsq[rc], A.egb[1]);
    qm = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool q = li + 16 * j < A.S && ms[j] >= mx - bq;
      const uint64_t b = __builtin_amdgcn_ballot_w64(q);
      qm |= ((b >> (16 * g)) & 0xFFFFull) << (16 * j);
    }
    mref = mx;
  }
  // ---- candidates of the group's row: words li, li + 16, ... (coalesced per group)
  auto word_at = [&](int wi) -> uint32_t {
    uint32_t wd = A.cmask[(size_t)rc * nwords + wi];
    if (wi * 32 + 32 > K) wd &= wi * 32 >= K ? 0u : (1u << (K - wi * 32)) - 1u;  // padding is never a candidate
    if (!((qm >> ((wi * 32) / KSA)) & 1ull)) wd = 0u;  // a far slice
    return wd;
  };
  int mycount = 0;
  for (int wi = li; wi < nwords; wi += 16) mycount += __popc(word_at(wi));
  int x = mycount;  // 16-lane inclusive scan
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    const int y = __shfl_up(x, off, 16);
    if (li >= off) x += y;
  }
  const int total = live ? __shfl(x, 15, 16) : 0;
  const int mybase = x - mycount;
  const bool is_light = total <= kLight;
  if (is_light && live) {
    int r = mybase;
    for (int wi = li; wi < nwords; wi += 16) {
      uint32_t wd = word_at(wi);
      while (wd) {
        const int bit = __builtin_ctz(wd);
        wd &= wd - 1;
        light[g][r++] = (unsigned short)(wi * 32 + bit);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (is_light && live) {
    // this lane's 8 dims of the row
    const unsigned short* xr = reinterpret_cast<const unsigned short*>(A.x) + row * A.ld_x;
    double xv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * li + e;
      xv[e] = d < D ? (double)__uint_as_float((unsigned)xr[d] << 16) : 0.0;
    }
    const bool vec = (D & 7) == 0 && ((uintptr_t)A.mu & 15) == 0;
    const int doff = vec ? min(8 * li, D - 8) : 0;
    const double xsq = A.xsq[row];
    // candidate c's score ends in lane c % 16, slot c / 16
    constexpr int NS = kLight / 16;
    double sc[NS];
    int kc[NS];
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      sc[t] = -INFINITY;
      kc[t] = 0x7fffffff;
    }
    constexpr int U = 2;
    for (int c0 = 0; c0 < total; c0 += U) {
      int ku[U];
      double2 cu[U];
      float4 m0[U], m1[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        ku[u] = light[g][min(c0 + u, total - 1)];
        cu[u] = A.kconst[ku[u]];
        const float* mu = A.mu + (size_t)ku[u] * D;
        if (vec) {
          m0[u] = *reinterpret_cast<const float4*>(mu + doff);
          m1[u] = *reinterpret_cast<const float4*>(mu + doff + 4);
        } else {
          float t[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) t[e] = (8 * li + e < D) ? mu[8 * li + e] : 0.f;
          m0[u] = float4{t[0], t[1], t[2], t[3]};
          m1[u] = float4{t[4], t[5], t[6], t[7]};
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        double dot = xv[0] * (double)m0[u].x + xv[1] * (double)m0[u].y + xv[2] * (double)m0[u].z +
                     xv[3] * (double)m0[u].w + xv[4] * (double)m1[u].x + xv[5] * (double)m1[u].y +
                     xv[6] * (double)m1[u].z + xv[7] * (double)m1[u].w;
        dot = row16_sum_f64(dot);
        const int c = c0 + u;
        const double v = cu[u].x + cu[u].y * (dot - 0.5 * xsq);
#pragma unroll
        for (int t = 0; t < NS; ++t)
          if (c < total && li == (c & 15) && t == (c >> 4)) {
            // score = (c0 - lambda log2(e) |mu|^2 / 2) + lambda log2(e) (x . mu - |x|^2 / 2)
            sc[t] = v;
            kc[t] = ku[u];
          }
      }
    }
    // top-m: the LSE over every candidate plus the slices' below-band mass
    double Mx = sc[0];
#pragma unroll
    for (int t = 1; t < NS; ++t) Mx = fmax(Mx, sc[t]);
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) Mx = fmax(Mx, __shfl_xor(Mx, off, 16));
    double lse = 0.0;
    if (!A.topk) {
      double ssum = 0.0;
#pragma unroll
      for (int t = 0; t < NS; ++t)
        if (sc[t] > -INFINITY) ssum += exp2_acc(sc[t] - Mx);
      double rem = remf;
      if (!A.fused_t)
        for (int s = li; s < A.S; s += 16) rem += (double)A.prem[(size_t)row * A.S + s];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        ssum += __shfl_xor(ssum, off, 16);
        rem += __shfl_xor(rem, off, 16);
      }
      const double mb = A.fused_t ? (double)mref : (double)A.mrow[row];
      lse = Mx + log2(ssum + rem * exp2(mb - Mx));
    }
    // the best m, one per round; lane j of the group keeps round j's
    double rl = -INFINITY;
    int rk = 0x7fffffff;
    for (int j = 0; j < m; ++j) {
      double bl = sc[0];
      int bk = kc[0];
#pragma unroll
      for (int t = 1; t < NS; ++t)
        if (before(sc[t], kc[t], bl, bk)) { bl = sc[t]; bk = kc[t]; }
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) {
        const double l2 = __shfl_xor(bl, off, 16);
        const int k2 = __shfl_xor(bk, off, 16);
        if (before(l2, k2, bl, bk)) { bl = l2; bk = k2; }
      }
#pragma unroll
      for (int u = 0; u < NS; ++u)
        if (kc[u] == bk && bk != 0x7fffffff) { sc[u] = -INFINITY; kc[u] = 0x7fffffff; }  // taken
      if (li == j) {
        rl = bl;
        rk = bk;
      }
    }
    if (A.topk) {
      // top-k: the log-sum-exp of the kept m (round 0 holds the best)
      double s = (li < m && rk < K) ? exp2(rl - Mx) : 0.0;
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) s += __shfl_xor(s, off, 16);
      lse = Mx + log2(s);
    }
    const double r = rk < K ? exp2(rl - lse) : 0.0;
    const bool ok = li < m && rk < K && (A.topk || li == 0 || r >= (double)A.thr);
    const unsigned okb = (unsigned)((__builtin_amdgcn_ballot_w64(ok) >> (16 * g)) & 0xFFFFu);
    const int c = __builtin_ctz(~okb);  // the kept ranks are a prefix
    if (li < m) {
      A.idx[row * m + li] = li < c ? rk : -1;
      A.resp[row * m + li] = li < c ? (float)r : 0.f;
    }
    if (li == 0) {
      if (A.count) A.count[row] = c;
      if (A.logp) A.logp[row] = (float)(lse * LN2);
    }
  }
  // ---- rows past kLight candidates: flagged for the heavy kernel
  const uint64_t heavy = __builtin_amdgcn_ballot_w64(live && !is_light && li == 0);  // bits 0, 16, 32, 48
  if (lane == 0)
    A.hv[blockIdx.x] = (unsigned char)((heavy & 1u) | ((heavy >> 15) & 2u) | ((heavy >> 30) & 4u) | ((heavy >> 45) & 8u));
}

// Rows flagged by largek_topm_final4_kernel, a whole wave each: waves stride
// over the flag bytes (one per four rows).
// Four waves per SIMD (registers capped at 128; a few spill): the rows are
// chains of dependent loads, and more of them in flight beat the spills
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4)))
largek_topm_heavy_kernel(LargeKArgs A, int64_t nflags) {
  __shared__ double sl[kSlots];
  __shared__ int skk[kSlots];
  __shared__ unsigned short slist[kBatch];
  for (int64_t b = blockIdx.x; b < nflags; b += gridDim.x) {
    const unsigned f = A.hv[b];  // uniform across the wave
    for (int q = 0; q < 4; ++q)
      if ((f >> q) & 1u) topm_row_wave(A, b * 4 + q, sl, skk, slist);
  }
}

hipError_t launch_largek_topm(const Plan& p, const LargeKArgs& a0, const float* w, const float* mu, const float* cv,
                              hipStream_t s) {
  LargeKArgs a = a0;
  hipLaunchKernelGGL(largek_prologue_kernel, dim3((unsigned)p.KP), dim3(64), 0, s, (int)p.D, (int)p.K, p.DP, w, mu,
                     cv, reinterpret_cast<__bf16*>(const_cast<void*>(a.W)),
                     reinterpret_cast<__bf16*>(const_cast<void*>(a.W32)),
                     reinterpret_cast<__bf16*>(const_cast<void*>(a.W32C)), const_cast<double*>(a.c),
                     const_cast<double*>(a.a), const_cast<double*>(a.c0), const_cast<double*>(a.lam),
                     const_cast<float*>(a.esh), const_cast<float*>(a.eall),
                     const_cast<double*>(a.mmk), const_cast<double2*>(a.kconst));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto kA = largek_kernel<128, 0>;
  auto kT = largek_kernel<128, 1>;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)kA, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    (void)hipFuncSetAttribute((const void*)kT, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    (void)hipFuncSetAttribute((const void*)largek_pass_a_kernel<kPassARB, 2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytes);
    (void)hipFuncSetAttribute((const void*)largek_pass_a_kernel<kPassARB, 1>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytes);
    (void)hipFuncSetAttribute((const void*)largek_pass_a_kernel<kPassARB, 3>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytes);
    (void)hipFuncSetAttribute((const void*)largek_pass_a_kernel<kPassARB, 4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytes);
    (void)hipFuncSetAttribute((const void*)largek_pass_a_kernel<kPassARB, 5>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)kLdsBytes);
    attr_set = true;
  }
  const int64_t N = a.N;
  const unsigned char* x0 = reinterpret_cast<const unsigned char*>(a.x);
  for (int64_t r0 = 0; r0 < N; r0 += p.chunk_rows) {
    LargeKArgs ac = a;
    ac.N = std::min<int64_t>(p.chunk_rows, N - r0);
    ac.x = x0 + (size_t)r0 * p.ld_x * 2;
    ac.idx = a.idx + r0 * a.m;
    ac.resp = a.resp + r0 * a.m;
    ac.count = a.count ? a.count + r0 : nullptr;
    ac.logp = a.logp ? a.logp + r0 : nullptr;
    ac.G = p.GbA;
    // the barrier-free passes (rows of 128 bf16, 16-byte aligned); the top-k
    // threshold needs their lane-group maxima, without them every live
    // component of a row is a top-k candidate
    const bool bf = p.D == 128 && ac.vec16;
    if (!bf) ac.lmx = nullptr;
    // the one-pass marking keeps the best component alone: a row's label, no
    // responsibilities, counts or log-likelihoods
    ac.fused_t = a0.fused_t && bf && !ac.topk && ac.m == 1 && !ac.count && !ac.logp;
    if (ac.fused_t) {
      // top-m over full-width rows: one marking pass, then the rescoring
      hipLaunchKernelGGL((largek_pass_a_kernel<kPassARB, 5>), dim3((unsigned)(p.S * p.GbA)), dim3(64 * LNW),
                         largek_pass_a_lds_bytes(5), s, ac);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
    if (bf && ac.topk)
      hipLaunchKernelGGL((largek_pass_a_kernel<kPassARB, 3>), dim3((unsigned)(p.S * p.GbA)), dim3(64 * LNW),
                         largek_pass_a_lds_bytes(3), s, ac);
    else if (bf)
      hipLaunchKernelGGL((largek_pass_a_kernel<kPassARB, 2>), dim3((unsigned)(p.S * p.GbA)), dim3(64 * LNW),
                         largek_pass_a_lds_bytes(2), s, ac);
    else
      hipLaunchKernelGGL(kA, dim3((unsigned)(p.S * p.GbA)), dim3(64 * LNW), p.lds_a, s, ac);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(largek_lse_kernel, dim3((unsigned)p.lse_blocks), dim3(256), 0, s, ac);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (bf && ac.topk)
      hipLaunchKernelGGL((largek_pass_a_kernel<kPassARB, 4>), dim3((unsigned)(p.S * p.GbA)), dim3(64 * LNW),
                         largek_pass_a_lds_bytes(4), s, ac);
    else if (bf)
      hipLaunchKernelGGL((largek_pass_a_kernel<kPassARB, 1>), dim3((unsigned)(p.S * p.GbA)), dim3(64 * LNW),
                         largek_pass_a_lds_bytes(1), s, ac);
    else
      hipLaunchKernelGGL(kT, dim3((unsigned)(p.S * p.GbA)), dim3(64 * LNW), p.lds_t, s, ac);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t nflags = (ac.N + 3) / 4;
    hipLaunchKernelGGL(largek_topm_final4_kernel, dim3((unsigned)nflags), dim3(64), 0, s, ac);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(largek_topm_heavy_kernel, dim3((unsigned)std::min<int64_t>(nflags, 16384)), dim3(64), 0, s, ac,
                       nflags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gmm
