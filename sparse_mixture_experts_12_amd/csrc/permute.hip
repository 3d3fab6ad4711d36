// Token-to-expert permutation with capacity dropping, and the device-side
// tile schedule of the grouped expert GEMMs.
//
// Pages: "MoE Model Architectures", Mixtral "Sparse MoE Block" (each expert
// gathers its tokens in token order; experts without tokens are skipped);
// Switch Transformers "Top-1 Routing" (an expert takes at most its capacity);
// "Current Bug: CuTeDSLMoERunner produces wrong output" (expert offsets over
// the permuted rows, leading-zero form; padding must never leak into them).
//
// Ranks: inside a block of 1024 assignments a = t*k + j, lanes of one wave
// that hold the same expert find each other with ballots over the expert-id
// bits (rank = popcount of lower lanes in the match mask); per-wave counts go
// to LDS and a prefix over the 16 waves gives each assignment its rank among
// the block's earlier assignments of its expert.  Ranks are therefore stable
// (ascending a) and deterministic, with no atomics.
//   Up to kPermSingleMax assignments: one work-group; each wave ranks its own
//   contiguous range with a running count per expert, a prefix over the
//   waves completes the ranks, then the scatter.
//   Beyond: three launches over all blocks -- per-block histograms and local
//   ranks; per expert, an exclusive scan of its counts over the blocks; the
//   expert offsets (a scan over experts, repeated by every block) and the
//   scatter of each kept assignment to offsets[e] + block base + local rank.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
// Largest assignment count the single-work-group permutation takes.
constexpr int kPermSingleMax = 4096;
// Multi-block permutations of at most this many blocks sum the per-block
// counts inside the scatter launch (each block reads E x nb counts).
constexpr int kPermFusedScanBlocks = 64;

// Inclusive scan of one int per lane over a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive scan of one value per thread over a work-group of NT threads (a
// multiple of 64): wave scans, then one wave scans the wave totals.  Two
// barriers; s_wave holds NT / 64 + 1 ints.  Returns the exclusive prefix;
// *total (optional) receives the sum in every thread.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* s_wave, int* total = nullptr) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < NW ? s_wave[lane] : 0;
    const int wi = wave_inclusive_scan(w);
    if (lane < NW) s_wave[lane] = wi - w;
    if (lane == NW - 1) s_wave[NW] = wi;
  }
  __syncthreads();
  const int ex = inc - v + s_wave[wave];
  if (total) *total = s_wave[NW];
  __syncthreads();                  // s_wave may be reused right after
  return ex;
}

// The grouped GEMMs' tile schedule (defined with tile_schedule_kernel below).
__device__ void write_tile_schedule(int row0, int rows, int E, int G, const SchedSpec& sp, int* s_wave);

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ idx, int n, int E, int cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ n_dropped, SchedSpec sp) {
  // wave w takes assignments [w * npw, (w + 1) * npw), 64 at a time in order
  // (npw: n spread evenly, in multiples of 64), keeping its own running count
  // per expert in its row of wcnt (no barrier inside that loop); an exclusive
  // prefix over the waves per expert then turns the in-wave ranks into ranks
  // over all earlier assignments.
  constexpr int NIT = kPermSingleMax / kPermThreads;    // most assignments per lane
  const int nit = (n + kPermThreads - 1) / kPermThreads;
  const int npw = nit * 64;
  __shared__ int run[kMaxExperts];
  __shared__ int wcnt[kPermWaves][kMaxExperts];
  __shared__ int scan[kPermWaves + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  int ev[NIT], rv[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {                    // all loads in flight together
    const int a = wave * npw + it * 64 + lane;
    ev[it] = (it < nit && a < n) ? idx[a] : 0;
    rv[it] = 0;
  }
  for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i / E][i % E] = 0;
  __syncthreads();
  int* mine = wcnt[wave];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    if (it >= nit) break;
    const bool valid = wave * npw + it * 64 + lane < n;
    const int e = ev[it];
    uint64_t m = ballot64(valid);                       // lanes of this wave holding the same expert
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = ballot64(bit);
      m &= bit ? bb : ~bb;
    }
    const int rank_w = __popcll(m & lanemask_lt());
    const int before = valid ? mine[e] : 0;             // this wave's earlier assignments of e
    rv[it] = before + rank_w;
    __builtin_amdgcn_wave_barrier();
    if (valid && rank_w == 0) mine[e] = before + __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  if (tid < E) {                                        // per expert: exclusive prefix over the waves
    int acc = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) {
      const int t = wcnt[w][tid];
      wcnt[w][tid] = acc;
      acc += t;
    }
    run[tid] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < NIT; ++it)
    if (it < nit && wave * npw + it * 64 + lane < n) rv[it] += mine[ev[it]];
  // kept counts and exclusive offsets
  int kept = 0, dropped_local = 0;
  if (tid < E) {
    int c = run[tid];
    kept = (cap >= 0 && c > cap) ? cap : c;
    dropped_local = c - kept;
    counts[tid] = kept;
  }
  int total_kept = 0, total_dropped = 0;
  const int off = block_exclusive_scan<kPermThreads>(kept, scan, &total_kept);
  block_exclusive_scan<kPermThreads>(dropped_local, scan, &total_dropped);
  if (tid < E) {
    offsets[tid] = off;
    run[tid] = off;                 // offsets for the scatter
  }
  if (tid == 0) {
    offsets[E] = total_kept;
    *n_dropped = total_dropped;
  }
  if (sp.sched) {                   // the grouped GEMMs' tile schedule, from the same offsets
    const bool sh = tid == E && sp.shared_rows > 0;
    write_tile_schedule(sh ? sp.shared_row0 : off, sh ? sp.shared_rows : kept, E, E + (sp.shared_rows > 0 ? 1 : 0),
                        sp, scan);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int a = wave * npw + it * 64 + lane;
    if (it < nit && a < n) {
      const int e = ev[it], r = rv[it];
      if (cap < 0 || r < cap) {
        const int pos = run[e] + r;
        sorted_assign[pos] = a;
        inv_perm[a] = pos;
      } else {
        inv_perm[a] = -1;
      }
      if (a >= total_kept) sorted_assign[a] = -1;
    }
  }
}

// ---------------------------------------------------------------------------
// Multi-block permutation (more than kPermSingleMax assignments).
// ---------------------------------------------------------------------------
// Stable rank of this thread's assignment among the block's earlier
// assignments of the same expert, and (through wcnt) the block's per-wave
// counts.  valid: the thread holds an assignment; e: its expert.
__device__ __forceinline__ int block_local_rank(bool valid, int e, int nbits, int E,
                                                int (*wcnt)[kMaxExperts]) {
  const int tid = threadIdx.x, wave = tid >> 6;
  uint64_t m = ballot64(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = ballot64(bit);
    m &= bit ? bb : ~bb;
  }
  const int rank_w = __popcll(m & lanemask_lt());
  for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i / E][i % E] = 0;
  __syncthreads();
  if (valid && rank_w == 0) wcnt[wave][e] = __popcll(m);
  __syncthreads();
  int r = rank_w;
  if (valid)
    for (int w = 0; w < wave; ++w) r += wcnt[w][e];
  return r;
}

// Launch 1: block b's count per expert -> hist[e * nb + b]; local ranks.
__global__ __launch_bounds__(kPermThreads) void perm_count_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                                  int nb, int32_t* __restrict__ hist,
                                                                  int32_t* __restrict__ rank_ws) {
  __shared__ int wcnt[kPermWaves][kMaxExperts];
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int a = blockIdx.x * kPermThreads + threadIdx.x;
  const bool valid = a < n;
  const int e = valid ? idx[a] : 0;
  const int r = block_local_rank(valid, e, nbits, E, wcnt);
  if (valid) rank_ws[a] = r;
  for (int ee = threadIdx.x; ee < E; ee += kPermThreads) {
    int c = 0;
    for (int w = 0; w < kPermWaves; ++w) c += wcnt[w][ee];
    hist[(size_t)ee * nb + blockIdx.x] = c;
  }
}

// Launch 2 (one work-group per expert): exclusive scan of the expert's block
// counts in place; its total, kept count (capacity) -> totals[e], counts[e].
__global__ __launch_bounds__(256) void perm_scan_kernel(int nb, int cap, int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ totals, int32_t* __restrict__ counts) {
  __shared__ int s_wave[256 / 64 + 1];
  int32_t* h = hist + (size_t)blockIdx.x * nb;
  int carry = 0;
  for (int b0 = 0; b0 < nb; b0 += 256) {
    const int b = b0 + threadIdx.x;
    const int v = b < nb ? h[b] : 0;
    int tot = 0;
    const int ex = block_exclusive_scan<256>(v, s_wave, &tot);
    if (b < nb) h[b] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) {
    totals[blockIdx.x] = carry;
    counts[blockIdx.x] = (cap >= 0 && carry > cap) ? cap : carry;
  }
}

// Launch 3: expert offsets (every block scans the kept counts; block 0 also
// writes offsets and the dropped total), then the scatter of the block's
// assignments and the -1 fill of unused sorted_assign entries in its range.
__global__ __launch_bounds__(kPermThreads) void perm_scatter_kernel(
    const int32_t* __restrict__ idx, int n, int E, int nb, int cap, const int32_t* __restrict__ hist,
    const int32_t* __restrict__ totals, const int32_t* __restrict__ counts, const int32_t* __restrict__ rank_ws,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ n_dropped, SchedSpec sp, int32_t* __restrict__ counts_out) {
  __shared__ int off[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int s_wave[kPermWaves + 1];
  const int tid = threadIdx.x;
  int kept, dropped;
  if (counts_out) {
    // few blocks: this block's base per expert (its counts in the blocks
    // before it) and the totals straight from the raw block counts, summed
    // in block order, instead of a separate scan launch
    int b4 = 0, tot = 0;
    if (tid < E) {
      const int32_t* h = hist + (size_t)tid * nb;
      for (int b = 0; b < nb; ++b) {
        if (b == (int)blockIdx.x) b4 = tot;
        tot += h[b];
      }
      base[tid] = b4;
    }
    kept = (cap >= 0 && tot > cap) ? cap : tot;
    dropped = tot - kept;
    if (blockIdx.x == 0 && tid < E) counts_out[tid] = kept;
  } else {
    kept = tid < E ? counts[tid] : 0;
    dropped = tid < E ? totals[tid] - kept : 0;
  }
  int total_kept = 0, total_dropped = 0;
  const int ex = block_exclusive_scan<kPermThreads>(kept, s_wave, &total_kept);
  block_exclusive_scan<kPermThreads>(dropped, s_wave, &total_dropped);
  if (tid < E) off[tid] = ex;
  if (blockIdx.x == 0) {
    if (tid < E) offsets[tid] = ex;
    if (tid == 0) {
      offsets[E] = total_kept;
      *n_dropped = total_dropped;
    }
    if (sp.sched) {                 // the grouped GEMMs' tile schedule, from the same offsets
      const bool sh = tid == E && sp.shared_rows > 0;
      write_tile_schedule(sh ? sp.shared_row0 : ex, sh ? sp.shared_rows : kept, E,
                          E + (sp.shared_rows > 0 ? 1 : 0), sp, s_wave);
    }
  }
  __syncthreads();
  const int a = blockIdx.x * kPermThreads + tid;
  if (a < n) {
    const int e = idx[a];
    const int r = (counts_out ? base[e] : hist[(size_t)e * nb + blockIdx.x]) + rank_ws[a];
    if (cap < 0 || r < cap) {
      const int pos = off[e] + r;
      sorted_assign[pos] = a;
      inv_perm[a] = pos;
    } else {
      inv_perm[a] = -1;
    }
    if (a >= total_kept) sorted_assign[a] = -1;
  }
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
// segments: "heavy" tiles with more than light_max rows (all full tiles and a
// large last tile) and "light" tiles with at most light_max rows (a group's
// small last tile; light_max is BM / 2 unless the caller sets it).  The GEMMs run light tiles with a cheaper body and spread
// each segment evenly over the XCDs.  Layout (ints):
//   [0] QH, [1] QL,
//   heavy tile q:  [kSchedHead + 4 q + {0: group, 1: row0, 2: rows, 3: first heavy tile of the group}]
//   heavy count g: [kSchedHead + 4 maxQ + g]
//   light tile p:  [kSchedHead + 4 maxQ + maxG + 3 p + {0: group, 1: row0, 2: rows}]
// Called by every thread of a kPermThreads work-group: thread g < G gives
// group g's first permuted row and row count (routed experts g < E, the
// shared expert as group E).  s_wave: kPermWaves + 1 ints of LDS.
__device__ void write_tile_schedule(int row0, int rows, int E, int G, const SchedSpec& sp, int* s_wave) {
  const int tid = threadIdx.x;
  const int BM = sp.BM, maxQ = sp.maxQ, maxG = E + 1;
  const int LM = sp.light_max > 0 ? sp.light_max : BM / 2;
  if (tid >= G) rows = 0;
  const int full = rows / BM, rem = rows - full * BM;
  const int nh = full + (rem > LM ? 1 : 0);
  const int nl = (rem > 0 && rem <= LM) ? 1 : 0;
  int qh = 0, ql = 0;
  const int first = block_exclusive_scan<kPermThreads>(nh, s_wave, &qh);
  const int lfirst = block_exclusive_scan<kPermThreads>(nl, s_wave, &ql);
  int32_t* hs = sp.sched + kSchedHead;
  if (tid < G) {
    hs[4 * maxQ + tid] = nh;
    for (int i = 0; i < nh; ++i) {
      const int q = first + i;
      hs[4 * q + 0] = tid;
      hs[4 * q + 1] = row0 + i * BM;
      hs[4 * q + 2] = min(BM, rows - i * BM);
      hs[4 * q + 3] = first;
    }
    if (nl) {
      int32_t* ls = hs + 4 * maxQ + maxG + 3 * lfirst;
      ls[0] = tid;
      ls[1] = row0 + full * BM;
      ls[2] = rem;
    }
  }
  if (tid == 0) {
    sp.sched[0] = qh;
    sp.sched[1] = ql;
  }
}

__global__ __launch_bounds__(kPermThreads) void tile_schedule_kernel(const int32_t* __restrict__ offsets, int E,
                                                                     SchedSpec sp) {
  __shared__ int s_wave[kPermWaves + 1];
  const int tid = threadIdx.x;
  int rows = 0, row0 = 0;
  if (tid < E) {
    row0 = offsets[tid];
    rows = offsets[tid + 1] - row0;
  } else if (tid == E && sp.shared_rows > 0) {
    row0 = sp.shared_row0;
    rows = sp.shared_rows;
  }
  write_tile_schedule(row0, rows, E, E + (sp.shared_rows > 0 ? 1 : 0), sp, s_wave);
}

static int perm_blocks(int n) { return (n + kPermThreads - 1) / kPermThreads; }

size_t permute_ws_bytes(int n, int E) {
  if (n <= kPermSingleMax) return 0;                   // ranks stay in registers
  return ((size_t)n + (size_t)E * perm_blocks(n) + E) * sizeof(int32_t);   // ranks, block counts, totals
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  if (a.n <= kPermSingleMax) {
    permute_kernel<<<1, kPermThreads, 0, s>>>(a.idx, a.n, a.E, a.cap, a.counts, a.offsets, a.sorted_assign,
                                              a.inv_perm, a.n_dropped, a.sched);
    return hipGetLastError();
  }
  const int nb = perm_blocks(a.n);
  int32_t* hist = a.rank_ws + a.n;
  int32_t* totals = hist + (size_t)a.E * nb;
  perm_count_kernel<<<nb, kPermThreads, 0, s>>>(a.idx, a.n, a.E, nb, hist, a.rank_ws);
  // up to kPermFusedScanBlocks blocks the scatter launch sums the block counts itself
  const bool fused = nb <= kPermFusedScanBlocks;
  if (!fused) perm_scan_kernel<<<a.E, 256, 0, s>>>(nb, a.cap, hist, totals, a.counts);
  perm_scatter_kernel<<<nb, kPermThreads, 0, s>>>(a.idx, a.n, a.E, nb, a.cap, hist, totals, a.counts, a.rank_ws,
                                                  a.offsets, a.sorted_assign, a.inv_perm, a.n_dropped, a.sched,
                                                  fused ? a.counts : nullptr);
  return hipGetLastError();
}

hipError_t launch_tile_schedule(const int32_t* offsets, int E, int BM, int shared_rows, int shared_row0, int maxQ,
                                int32_t* sched, hipStream_t s, int light_max) {
  SchedSpec sp{sched, BM, shared_rows, shared_row0, maxQ, light_max};
  tile_schedule_kernel<<<1, kPermThreads, 0, s>>>(offsets, E, sp);
  return hipGetLastError();
}

}  // namespace moe
