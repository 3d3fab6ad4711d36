// Token-to-expert permutation with capacity dropping, and the device-side
// tile schedule of the grouped expert GEMMs.
//
// Pages: "MoE Model Architectures", Mixtral "Sparse MoE Block" (each expert
// gathers its tokens in token order; experts without tokens are skipped);
// Switch Transformers "Top-1 Routing" (an expert takes at most its capacity);
// "Current Bug: CuTeDSLMoERunner produces wrong output" (expert offsets over
// the permuted rows, leading-zero form; padding must never leak into them).
//
// One work-group of 1024 threads walks the assignments a = t*k + j in chunks
// of 1024 in ascending order.  Inside a chunk, lanes of one wave that hold the
// same expert find each other with ballots over the expert-id bits (rank =
// popcount of lower lanes in the match mask); per-wave counts go to LDS and a
// short prefix over the 16 waves plus the running per-expert count gives each
// assignment its rank among all earlier assignments of its expert.  Ranks are
// therefore stable (ascending a) and the result is deterministic with no
// atomics.  A second pass scatters kept assignments to offsets[e] + rank.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

__device__ __forceinline__ void block_exclusive_scan_1024(int* buf, int n, int* total) {
  // Hillis-Steele inclusive scan over buf[0..1024) by 1024 threads, then shift.
  const int tid = threadIdx.x;
  int v = (tid < n) ? buf[tid] : 0;
  __syncthreads();
  for (int off = 1; off < kPermThreads; off <<= 1) {
    buf[tid] = v;
    __syncthreads();
    if (tid >= off) v += buf[tid - off];
    __syncthreads();
  }
  buf[tid] = v;                     // inclusive
  __syncthreads();
  int ex = (tid == 0) ? 0 : buf[tid - 1];
  int tot = buf[kPermThreads - 1];
  __syncthreads();
  buf[tid] = ex;
  if (total && tid == 0) *total = tot;
  __syncthreads();
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ idx, int n, int E, int cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ n_dropped, int32_t* __restrict__ rank_ws) {
  __shared__ int run[kMaxExperts];
  __shared__ int wcnt[kPermWaves][kMaxExperts];
  __shared__ int scan[kPermThreads];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;

  for (int e = tid; e < E; e += kPermThreads) run[e] = 0;
  __syncthreads();

  for (int base = 0; base < n; base += kPermThreads) {
    const int a = base + tid;
    const bool valid = a < n;
    const int e = valid ? idx[a] : 0;
    // lanes of this wave holding the same expert
    uint64_t m = ballot64(valid);
    for (int b = 0; b < nbits; ++b) {
      bool bit = (e >> b) & 1;
      uint64_t bb = ballot64(bit);
      m &= bit ? bb : ~bb;
    }
    const int rank_w = __popcll(m & lanemask_lt());
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i / E][i % E] = 0;
    __syncthreads();
    if (valid && rank_w == 0) wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (valid) {
      int r = run[e] + rank_w;
      for (int w = 0; w < wave; ++w) r += wcnt[w][e];
      rank_ws[a] = r;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kPermThreads) {
      int s = 0;
      for (int w = 0; w < kPermWaves; ++w) s += wcnt[w][ee];
      run[ee] += s;
    }
    __syncthreads();
  }
  // kept counts and exclusive offsets
  int kept = 0, dropped_local = 0;
  if (tid < E) {
    int c = run[tid];
    kept = (cap >= 0 && c > cap) ? cap : c;
    dropped_local = c - kept;
    counts[tid] = kept;
  }
  scan[tid] = kept;
  __syncthreads();
  block_exclusive_scan_1024(scan, E, &s_total);
  if (tid < E) offsets[tid] = scan[tid];
  if (tid == 0) offsets[E] = s_total;
  // dropped total
  scan[tid] = dropped_local;
  __syncthreads();
  block_exclusive_scan_1024(scan, kPermThreads, &s_total);
  if (tid == 0) *n_dropped = s_total;
  // offsets back into LDS for the scatter
  for (int e = tid; e < E; e += kPermThreads) run[e] = offsets[e];
  __syncthreads();
  const int total_kept = offsets[E];
  for (int a = tid; a < n; a += kPermThreads) {
    int e = idx[a];
    int r = rank_ws[a];
    if (cap < 0 || r < cap) {
      int pos = run[e] + r;
      sorted_assign[pos] = a;
      inv_perm[a] = pos;
    } else {
      inv_perm[a] = -1;
    }
  }
  for (int p = total_kept + tid; p < n; p += kPermThreads) sorted_assign[p] = -1;
}

// ---------------------------------------------------------------------------
// Tile schedule of the grouped GEMMs.  From the expert offsets, list the
// row tiles (expert, first row, rows) of every expert with rows, experts in
// ascending order, plus the shared expert (group index E, rows T*k .. T*k+T-1)
// when present.  Layout (int32):
//   sched[0]                    number of row tiles Q
//   sched[1 + 4q .. 4q + 4]     tile q: group, row0, rows, first tile of group
//   group g's row-tile count is stored in sched[1 + 4*maxQ + g]
// ---------------------------------------------------------------------------
// Row tiles of every group (expert, or the shared expert as group E), in two
// segments: "heavy" tiles with more than BM / 2 rows (all full tiles and a
// large last tile) and "light" tiles with at most BM / 2 rows (a group's
// small last tile).  The GEMMs run light tiles with a cheaper body and spread
// each segment evenly over the XCDs.  Layout (ints):
//   [0] QH, [1] QL,
//   heavy tile q:  [kSchedHead + 4 q + {0: group, 1: row0, 2: rows, 3: first heavy tile of the group}]
//   heavy count g: [kSchedHead + 4 maxQ + g]
//   light tile p:  [kSchedHead + 4 maxQ + maxG + 3 p + {0: group, 1: row0, 2: rows}]
__global__ __launch_bounds__(kPermThreads) void tile_schedule_kernel(const int32_t* __restrict__ offsets, int E,
                                                                     int BM, int shared_rows, int shared_row0,
                                                                     int maxQ, int32_t* __restrict__ sched) {
  __shared__ int scan_h[kPermThreads];
  __shared__ int scan_l[kPermThreads];
  __shared__ int s_qh, s_ql;
  const int tid = threadIdx.x;
  const int G = E + (shared_rows > 0 ? 1 : 0);
  const int maxG = E + 1;
  int rows = 0, row0 = 0;
  if (tid < E) {
    row0 = offsets[tid];
    rows = offsets[tid + 1] - row0;
  } else if (tid == E && shared_rows > 0) {
    row0 = shared_row0;
    rows = shared_rows;
  }
  const int full = rows / BM, rem = rows - full * BM;
  const int nh = full + (rem > BM / 2 ? 1 : 0);
  const int nl = (rem > 0 && rem <= BM / 2) ? 1 : 0;
  scan_h[tid] = nh;
  scan_l[tid] = nl;
  __syncthreads();
  block_exclusive_scan_1024(scan_h, G, &s_qh);
  block_exclusive_scan_1024(scan_l, G, &s_ql);
  if (tid < G) {
    const int first = scan_h[tid];
    int32_t* hs = sched + kSchedHead;
    hs[4 * maxQ + tid] = nh;
    for (int i = 0; i < nh; ++i) {
      const int q = first + i;
      hs[4 * q + 0] = tid;
      hs[4 * q + 1] = row0 + i * BM;
      hs[4 * q + 2] = min(BM, rows - i * BM);
      hs[4 * q + 3] = first;
    }
    if (nl) {
      int32_t* ls = hs + 4 * maxQ + maxG + 3 * scan_l[tid];
      ls[0] = tid;
      ls[1] = row0 + full * BM;
      ls[2] = rem;
    }
  }
  if (tid == 0) {
    sched[0] = s_qh;
    sched[1] = s_ql;
  }
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  permute_kernel<<<1, kPermThreads, 0, s>>>(a.idx, a.n, a.E, a.cap, a.counts, a.offsets, a.sorted_assign,
                                            a.inv_perm, a.n_dropped, a.rank_ws);
  return hipGetLastError();
}

hipError_t launch_tile_schedule(const int32_t* offsets, int E, int BM, int shared_rows, int shared_row0, int maxQ,
                                int32_t* sched, hipStream_t s) {
  tile_schedule_kernel<<<1, kPermThreads, 0, s>>>(offsets, E, BM, shared_rows, shared_row0, maxQ, sched);
  return hipGetLastError();
}

}  // namespace moe
