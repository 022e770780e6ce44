// gmm_ivf.hip -- inverted lists (IVF posting lists) from a soft multi-assignment.
//
// What it builds ("Flash-GMM: A Memory-Efficient Kernel for Scalable Soft
// Clustering", Section 4 -- the GMM as the IVF coarse quantizer with the
// multi-assignment scheme of Section 4.3 -- and Conclusion: boundary vectors
// are stored in several posting lists): for each component k of a problem, the
// rows whose multi-assignment kept k, in increasing row order, as CSR -- list
// offsets, then the rows and, optionally, their responsibilities.
//
// How (deterministic, no atomics).  Rows are cut into blocks of kIvfBlock rows,
// one wave per block:
//   1. walk (count): the wave reads its block in 64-row chunks, one row per
//      lane, and keeps per-component entry counts of the block in LDS;
//   2. per (problem, component): the block counts become exclusive prefixes
//      over the blocks, and their total is the list size;
//   3. per problem: list sizes -> offsets (exclusive scan over components);
//   4. walk (scatter): the same walk, its LDS counters starting at
//      offsets[k] + (entries of k in earlier blocks); an entry of component k
//      lands at that counter + (entries of k in earlier rows of this chunk),
//      so placing an entry reads LDS only.  Positions fit in int32 (N m < 2^31).
// The rank inside a chunk: for each slot of the other rows, one ballot per bit
// of the component index gives, per lane, the mask of lanes holding this
// lane's component; a popcount below the lane counts the earlier rows.
#include "gmm_internal.h"

#include <hip/hip_runtime.h>

#include <algorithm>

namespace gmm {

namespace {

// Walk over one block: SCATTER = false counts, true places the entries.
// M: a compile-time bound on m (slots past m are empty).
template <int M, bool SCATTER>
__global__ void __launch_bounds__(64) ivf_walk_kernel(IvfArgs A) {
  // K counters: count -- entries of each component so far in this block;
  // scatter -- the position of its next entry in the problem's lists
  extern __shared__ int run[];
  const int lane = threadIdx.x;
  const int b = blockIdx.x / A.nblk, blk = blockIdx.x % A.nblk;
  const int32_t* before_blocks = A.cnt + ((size_t)b * A.nblk + blk) * A.K;
  const int64_t* offb = A.offsets + (size_t)b * (A.K + 1);
  for (int k = lane; k < A.K; k += 64) run[k] = SCATTER ? (int)(offb[k] + before_blocks[k]) : 0;
  const int64_t r0 = (int64_t)blk * kIvfBlock;
  const int64_t r1 = std::min<int64_t>(A.N, r0 + kIvfBlock);
  const int32_t* idxb = A.idx + (size_t)b * A.N * A.m;
  const float* respb = A.resp ? A.resp + (size_t)b * A.N * A.m : nullptr;
  int32_t* rowsb = A.rows + (size_t)b * A.N * A.m;
  float* lrb = A.lresp ? A.lresp + (size_t)b * A.N * A.m : nullptr;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes under this one

  // a chunk's raw slots (and, when placing, their responsibilities) are loaded
  // one chunk ahead, so the walk does not wait on memory at each chunk
  int nraw[M];
  float nresp[M];
  auto load = [&](int64_t c0) {
    const int64_t row = c0 + lane;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      nraw[j] = (row < r1 && j < A.m) ? idxb[row * A.m + j] : -1;
      if constexpr (SCATTER) nresp[j] = (lrb && row < r1 && j < A.m) ? respb[row * A.m + j] : 0.f;
    }
  };
  load(r0);
  for (int64_t c0 = r0; c0 < r1; c0 += 64) {
    const int64_t row = c0 + lane;
    int raw[M];
    float rsp[M];
#pragma unroll
    for (int j = 0; j < M; ++j) {
      raw[j] = nraw[j];
      rsp[j] = nresp[j];
    }
    if (c0 + 64 < r1) load(c0 + 64);
    // this row's entries: its leading components in [0, K); -1 past them
    int key[M];
    bool live = row < r1;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      int k = live ? raw[j] : -1;
      if (k < 0 || k >= A.K) {
        live = false;
        k = -1;
      }
      key[j] = k;
    }
    // rank[j]: entries of key[j] in earlier rows of the chunk (and in earlier
    // slots of this row); tot[j]: entries of key[j] in the chunk
    int rank[M], tot[M];
#pragma unroll
    for (int j = 0; j < M; ++j) rank[j] = tot[j] = 0;
#pragma unroll
    for (int jp = 0; jp < M; ++jp) {
      const uint64_t act = __builtin_amdgcn_ballot_w64(key[jp] >= 0);
      if (act == 0) continue;  // the same for every lane
      uint64_t msk[M];
#pragma unroll
      for (int j = 0; j < M; ++j) msk[j] = act;
      for (int bit = 0; bit < A.KB; ++bit) {
        const uint64_t set = __builtin_amdgcn_ballot_w64(((key[jp] >> bit) & 1) != 0);
#pragma unroll
        for (int j = 0; j < M; ++j) msk[j] &= ((key[j] >> bit) & 1) ? set : ~set;
      }
#pragma unroll
      for (int j = 0; j < M; ++j) {
        if (key[j] < 0) continue;
        rank[j] += __builtin_popcountll(msk[j] & below) + ((jp < j && key[jp] == key[j]) ? 1 : 0);
        tot[j] += __builtin_popcountll(msk[j]);
      }
    }
    // every lane reads the running counts before any lane updates them; the
    // last entry of each component in the chunk advances its count
    int seen[M];
#pragma unroll
    for (int j = 0; j < M; ++j) seen[j] = key[j] >= 0 ? run[key[j]] : 0;
    if constexpr (SCATTER) {
#pragma unroll
      for (int j = 0; j < M; ++j) {
        if (key[j] < 0) continue;
        const int pos = seen[j] + rank[j];
        rowsb[pos] = (int32_t)row;
        if (lrb) lrb[pos] = rsp[j];
      }
    }
#pragma unroll
    for (int j = 0; j < M; ++j)
      if (key[j] >= 0 && rank[j] == tot[j] - 1) run[key[j]] = seen[j] + tot[j];
  }
  if constexpr (!SCATTER) {
    int32_t* out = A.cnt + ((size_t)b * A.nblk + blk) * A.K;
    for (int k = lane; k < A.K; k += 64) out[k] = run[k];
  }
}

// Per (problem, component): block counts -> exclusive prefixes over the
// blocks; the total (the list size) goes to offsets[b][k].
__global__ void __launch_bounds__(256) ivf_blocks_kernel(IvfArgs A) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)A.B * A.K) return;
  const int b = (int)(t / A.K), k = (int)(t % A.K);
  int32_t* c = A.cnt + (size_t)b * A.nblk * A.K + k;
  int64_t s = 0;
  constexpr int U = 16;  // loads in flight per thread
  int blk = 0;
  for (; blk + U <= A.nblk; blk += U) {
    int32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = c[(size_t)(blk + u) * A.K];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      c[(size_t)(blk + u) * A.K] = (int32_t)s;
      s += v[u];
    }
  }
  for (; blk < A.nblk; ++blk) {
    const int32_t v = c[(size_t)blk * A.K];
    c[(size_t)blk * A.K] = (int32_t)s;
    s += v;
  }
  A.offsets[(size_t)b * (A.K + 1) + k] = s;
}

// Per problem (one workgroup of 1024 threads): list sizes in offsets[b][0..K)
// -> offsets[b][0..K] (exclusive scan; offsets[b][K] = entries of the problem).
__global__ void __launch_bounds__(1024) ivf_offsets_kernel(IvfArgs A) {
  __shared__ int64_t part[1024];
  const int b = blockIdx.x, t = threadIdx.x, nt = blockDim.x;
  int64_t* o = A.offsets + (size_t)b * (A.K + 1);
  const int per = (A.K + nt - 1) / nt;
  const int k0 = std::min(A.K, t * per), k1 = std::min(A.K, k0 + per);
  int64_t s = 0;
  for (int k = k0; k < k1; ++k) s += o[k];
  part[t] = s;
  __syncthreads();
  if (t == 0) {
    int64_t run = 0;
    for (int i = 0; i < nt; ++i) {
      const int64_t v = part[i];
      part[i] = run;
      run += v;
    }
    o[A.K] = run;
  }
  __syncthreads();
  s = part[t];
  for (int k = k0; k < k1; ++k) {
    const int64_t v = o[k];
    o[k] = s;
    s += v;
  }
}

template <int M, bool SCATTER>
void allow_lds() {
  static bool set = false;  // the counters take up to 64 KB at K = kIvfMaxK
  if (!set) {
    (void)hipFuncSetAttribute((const void*)ivf_walk_kernel<M, SCATTER>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(sizeof(int) * kIvfMaxK));
    set = true;
  }
}

template <bool SCATTER>
hipError_t launch_walk(const IvfArgs& A, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)A.B * A.nblk)), block(64);
  const size_t lds = sizeof(int) * (size_t)A.K;
  allow_lds<1, SCATTER>();
  allow_lds<2, SCATTER>();
  allow_lds<4, SCATTER>();
  allow_lds<8, SCATTER>();
  allow_lds<16, SCATTER>();
  if (A.m <= 1) hipLaunchKernelGGL((ivf_walk_kernel<1, SCATTER>), grid, block, lds, s, A);
  else if (A.m <= 2) hipLaunchKernelGGL((ivf_walk_kernel<2, SCATTER>), grid, block, lds, s, A);
  else if (A.m <= 4) hipLaunchKernelGGL((ivf_walk_kernel<4, SCATTER>), grid, block, lds, s, A);
  else if (A.m <= 8) hipLaunchKernelGGL((ivf_walk_kernel<8, SCATTER>), grid, block, lds, s, A);
  else hipLaunchKernelGGL((ivf_walk_kernel<16, SCATTER>), grid, block, lds, s, A);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ivf_lists(const IvfArgs& A, hipStream_t s) {
  hipError_t e;
  if (A.nblk > 0 && (e = launch_walk<false>(A, s)) != hipSuccess) return e;
  const int64_t nk = (int64_t)A.B * A.K;
  hipLaunchKernelGGL(ivf_blocks_kernel, dim3((unsigned)((nk + 255) / 256)), dim3(256), 0, s, A);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(ivf_offsets_kernel, dim3((unsigned)A.B), dim3(1024), 0, s, A);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (A.nblk > 0 && (e = launch_walk<true>(A, s)) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace gmm
