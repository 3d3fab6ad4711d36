// Router of the MoE layer on gfx950: logits = fp32(fp64 sum of x W_g (+ b)),
// softmax over experts, top-k (ties -> lower expert index), optional
// renormalisation of the chosen weights.
//
// Pages: "MoE Model Architectures", Mixtral "Sparse MoE Block" (gate, softmax,
// topk, divide by the top-k sum); DeepSeek-V3 "Auxiliary-Loss-Free Load
// Balancing" (router bias inside the linear map); "perf(moe): route
// granite-4.0-h single-token MoE through the fused kernel" (fp32 scores).
//
// The logits are accumulated in fp64 so that every summation order rounds to
// the same fp32 value except in vanishingly rare cases; selection is done on
// those fp32 values and is therefore reproducible against an fp64 reference.
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router logits for T > 8 as fp64 partial sums over slices of the hidden
// dimension (split-K), finished by the top-k kernel, which adds the slices in
// a fixed order:
//   part[z][t][e] = sum over rows r of slice z of x[t, r] * W_g[r, e]   (fp64)
//
// Partial logits on the fp64 matrix cores (v_mfma_f64_16x16x4f64).  The
// products of bf16 or fp32 inputs are exact in fp64, so these partial sums
// differ from a sequential fp64 sum only in the order of the additions.
// Operand layout (checked on gfx950): A lane l = A[l % 16][l / 16],
// B lane l = B[l / 16][l % 16], result lane l, register v = D[l / 16 + 4 v][l % 16].
// Large layers (router_partial_lds): work-group tile BT tokens x BE experts
// (64 x 64, or 256 x 16 for few experts), K step 16, operands staged in LDS as
// fp32 (exact) with padded rows so that the 4 K-rows read by one fragment load
// fall in distinct banks, each step's loads issued two steps ahead; each
// operand value is read from L2 by E / BE or T / BT work-groups.
// ---------------------------------------------------------------------------
template <typename TIn, int BE>
__global__ __launch_bounds__(256) void router_partial_lds(const TIn* __restrict__ x, const TIn* __restrict__ W,
                                                           double* __restrict__ part, int T, int d, int E,
                                                           int dsplit) {
  typedef double f64x4_t __attribute__((ext_vector_type(4)));
  constexpr int BT = (BE == 64) ? 64 : 256;
  constexpr int WM = (BE == 64) ? 2 : 4, WN = 4 / WM;   // wave grid
  constexpr int MT = BT / WM / 16, NT = BE / WN / 16;    // 16 x 16 MFMA tiles per wave
  constexpr int BK = 16;
  constexpr int XP = BT + 16, WP = BE + 16;
  constexpr int XE = BT * BK / 256;                      // x elements per thread per step (4 or 16)
  constexpr int TPT = BK / XE;                           // threads per token row
  constexpr int WE = BE * BK / 256;                      // W elements per thread per step (4 or 1)
  __shared__ float xs[2][BK][XP];
  __shared__ float ws[2][BK][WP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE, z = blockIdx.z;
  const int r_begin = z * dsplit;
  const int r_end = min(d, r_begin + dsplit);            // r_end - r_begin is a multiple of BK
  const int xt_l = tid / TPT, xk_l = (tid % TPT) * XE;
  const bool xt_ok = t0 + xt_l < T;
  const TIn* xrow = x + (size_t)(xt_ok ? t0 + xt_l : T - 1) * d + xk_l;
  const int wk_l = tid / (BE / WE), we_l = (tid % (BE / WE)) * WE;
  // two register sets: the loads of step j go to set j % 2, two steps ahead of
  // the MFMAs that use them (stored to LDS at the end of step j - 1)
  float xr[2][XE], wr[2][WE];
  // loads of the step at k0 (always a valid step; rows past T and experts past
  // E read clamped addresses and are zeroed)
  auto load = [&](int k0, auto SET) {
    constexpr int q = decltype(SET)::value;
#pragma unroll
    for (int i = 0; i < XE; ++i) {
      const float v = ActTraits<TIn>::load(xrow, k0 + i);
      xr[q][i] = xt_ok ? v : 0.f;
    }
#pragma unroll
    for (int j = 0; j < WE; ++j) {
      const int e = e0 + we_l + j;
      const float v = ActTraits<TIn>::load(W, (size_t)(k0 + wk_l) * E + (e < E ? e : 0));
      wr[q][j] = e < E ? v : 0.f;
    }
  };
  auto store = [&](int buf, auto SET) {
    constexpr int q = decltype(SET)::value;
#pragma unroll
    for (int i = 0; i < XE; ++i) xs[buf][xk_l + i][xt_l] = xr[q][i];
#pragma unroll
    for (int j = 0; j < WE; ++j) ws[buf][wk_l][we_l + j] = wr[q][j];
  };
  f64x4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = (f64x4_t){0.0, 0.0, 0.0, 0.0};
  const int fr = lane & 15, fk = lane >> 4;
  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < BK / 4; ++ks) {
      double a[MT], b[NT];
#pragma unroll
      for (int i = 0; i < MT; ++i) a[i] = (double)xs[buf][ks * 4 + fk][wm * (BT / WM) + i * 16 + fr];
#pragma unroll
      for (int j = 0; j < NT; ++j) b[j] = (double)ws[buf][ks * 4 + fk][wn * (BE / WN) + j * 16 + fr];
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int nk = (r_end - r_begin) / BK;                 // >= 1
  // clamped step index: steps past the end reload the last step (unused)
  const auto kof = [&](int j) { return r_begin + min(j, nk - 1) * BK; };
  load(kof(0), S0{});
  load(kof(1), S1{});
  store(0, S0{});
  __syncthreads();
  // step j: issue step j + 2's loads into set j % 2, compute from LDS buffer
  // j % 2, then store step j + 1 (set (j + 1) % 2) into the other buffer
  for (int j = 0; j < nk; j += 2) {
    load(kof(j + 2), S0{});
    compute(0);
    store(1, S1{});
    __syncthreads();
    if (j + 1 < nk) {
      load(kof(j + 3), S1{});
      compute(1);
      store(0, S0{});
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + wm * (BT / WM) + i * 16 + fk + 4 * v;
        const int e = e0 + wn * (BE / WN) + j * 16 + fr;
        if (t < T && e < E) part[((size_t)z * T + t) * E + e] = acc[i][j][v];
      }
}

// ---------------------------------------------------------------------------
// Small layers (router_partial_tile, at most 256 tiles of 16 x 16):
// one work-group computes 16 tokens x 16 experts over its K slice; the slice
// is dealt to the four waves in 32-wide chunks (chunk c to wave c mod 4) and
// the waves' sums are added in wave order through LDS.  In MFMA step s of the
// chunk at k0, lane l supplies A = x[t0 + l % 16][k0 + 8 (l / 16) + s] and
// B = W_g[k0 + 8 (l / 16) + s][e0 + l % 16]; both operands index K the same
// way, so the eight steps add the chunk's 32 products of every (token,
// expert) pair.  A lane's eight x values are one contiguous 16-byte (bf16) or
// 32-byte (fp32) load; the next two chunks' loads are in flight during a
// chunk's MFMAs.  No LDS staging and four waves per 256 outputs: more
// work-groups than the 64 x 64 tiles give when T x E is small, at the price
// of 4x (16 / 64) more L2 reads per operand, which is why large layers keep
// the LDS-staged tiles.  Measured on MI355X, partial + top-k kernels: tiny
// fp32 layer (T 64, E 8) 15.0 -> 8.6 us, fp8 layer (T 512, E 128) 23.9 ->
// 19.7 us, Mixtral prefill (T 4096, E 8) 36.3 -> 30.6 us; the fine-grained
// layer (T 2048, E 256, 2048 tiles) was slower with these tiles (190 -> 210 us).
// ---------------------------------------------------------------------------
template <typename TIn>
__device__ __forceinline__ void load_x8(const TIn* p, float* v) {
  if constexpr (sizeof(TIn) == 2) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16lo(w[i]);
      v[2 * i + 1] = bf16hi(w[i]);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <typename TIn>
__global__ __launch_bounds__(256) void router_partial_tile(const TIn* __restrict__ x, const TIn* __restrict__ W,
                                                           double* __restrict__ part, int T, int d, int E,
                                                           int dsplit) {
  typedef double f64x4_t __attribute__((ext_vector_type(4)));
  __shared__ double red[3][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * 16, e0 = blockIdx.y * 16, z = blockIdx.z;
  const int r_begin = z * dsplit;
  const int r_end = min(d, r_begin + dsplit);            // r_end - r_begin is a multiple of 32
  const int m = lane & 15, kg = lane >> 4;
  // rows past T and experts past E read clamped addresses; they only reach
  // output rows / columns that are never stored
  const TIn* xrow = x + (size_t)min(t0 + m, T - 1) * d + 8 * kg;
  const TIn* wcol = W + min(e0 + m, E - 1) + (size_t)(8 * kg) * E;
  auto load = [&](int k0, float* xv, float* wv) {
    load_x8<TIn>(xrow + k0, xv);
#pragma unroll
    for (int s = 0; s < 8; ++s) wv[s] = ActTraits<TIn>::load(wcol, (size_t)(k0 + s) * E);
  };
  f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
  auto mfmas = [&](const float* xv, const float* wv) {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xv[s], (double)wv[s], acc, 0, 0, 0);
  };
  // this wave's chunks start at k_i = r_begin + 32 wave + 128 i; two buffers,
  // each refilled right after its MFMAs, so two chunks' loads are in flight
  // while a chunk's MFMAs run
  const int kw = r_begin + 32 * wave;
  const int n = kw < r_end ? (r_end - kw + 127) / 128 : 0;
  float x0[8], w0[8], x1[8], w1[8];
  if (n > 0) load(kw, x0, w0);
  if (n > 1) load(kw + 128, x1, w1);
  for (int i = 0; i < n; i += 2) {
    mfmas(x0, w0);
    if (i + 2 < n) load(kw + 128 * (i + 2), x0, w0);
    if (i + 1 < n) {
      mfmas(x1, w1);
      if (i + 3 < n) load(kw + 128 * (i + 3), x1, w1);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave - 1][v][lane] = acc[v];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const double sum = ((acc[v] + red[0][v][lane]) + red[1][v][lane]) + red[2][v][lane];
      const int t = t0 + kg + 4 * v;
      const int e = e0 + m;
      if (t < T && e < E) part[((size_t)z * T + t) * E + e] = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k of one token held by one wave: values are spread over the lanes
// (lane l owns experts l, l + 64, ...).  Selection order: larger logit first,
// equal logits -> lower index.  Weights: fp64 softmax rounded to fp32.
// ---------------------------------------------------------------------------
constexpr int kMaxEPerLane = 16;   // E <= 1024

__device__ void wave_topk(const float* lg /* logits of the token, any memory */, int E, int k,
                          int renormalize, int32_t* out_idx, float* out_w) {
  const int lane = lane_id();
  float v[kMaxEPerLane];
  bool used[kMaxEPerLane];
#pragma unroll
  for (int i = 0; i < kMaxEPerLane; ++i) {
    int e = lane + i * 64;
    v[i] = (e < E) ? lg[e] : -INFINITY;
    used[i] = (e >= E);
  }
  // running maximum (the first selected logit) for the softmax shift
  float m = -INFINITY;
  double chosen_sum = 0.0;
  int sel_idx = -1;          // lane j < k keeps slot j's expert
  float sel_logit = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kMaxEPerLane; ++i) {
      int e = lane + i * 64;
      if (!used[i] && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    // every lane now holds the winner
#pragma unroll
    for (int i = 0; i < kMaxEPerLane; ++i)
      if (lane + i * 64 == bi) used[i] = true;
    if (j == 0) m = bv;
    if (lane == j) { sel_idx = bi; sel_logit = bv; }
  }
  double den;
  if (renormalize) {
    // sum over the chosen experts in slot order (lane order 0..k-1)
    double p = (lane < k) ? exp((double)sel_logit - (double)m) : 0.0;
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += __shfl(p, j);
    den = s;
    chosen_sum = p;
  } else {
    // full softmax denominator: per-lane sum in index order, then a fixed
    // butterfly across lanes
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < kMaxEPerLane; ++i) {
      int e = lane + i * 64;
      if (e < E) s += exp((double)v[i] - (double)m);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    den = s;
    chosen_sum = (lane < k) ? exp((double)sel_logit - (double)m) : 0.0;
  }
  if (lane < k) {
    out_idx[lane] = sel_idx;
    out_w[lane] = (float)(chosen_sum / den);
  }
}

// ---------------------------------------------------------------------------
// Small-T router (T <= 8) in one work-group of 512 threads: logits for every
// token, top-k, and the decode plan used by the fused decode path:
//   plan[0]            n_used: number of distinct experts with a kept assignment
//   plan[1 .. E]       used expert ids, ascending (first n_used valid)
//   plan[1 + E + a]    for assignment a = t*k + j: index into the used list, or -1
//                      if the assignment is dropped by the capacity rule.
// Each thread owns one chunk of 8 experts and a strided set of rows of W_g
// (one 16-byte load per row for bf16), all issued before use; per-thread fp64
// sums are combined by a fixed butterfly inside the wave and a fixed-order sum
// over the waves.  When W_g is large, the same kernel first runs as S
// work-groups that each write one slice of rows' fp64 partial logits, and the
// one-work-group call adds the S slices in slice order.  Top-k is rank based:
// every logit's rank is the count of logits that precede it (larger, or equal
// with a lower index), so no serial cross-lane selection loop is needed.
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 512;
constexpr int kSmallWaves = kSmallThreads / 64;

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* __restrict__ W, size_t off, int nvalid, bool vec, double* w) {
  if (vec && nvalid == 8 && sizeof(TIn) == 2) {
    const uint4 v = *reinterpret_cast<const uint4*>(W + off);
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[2 * i] = (double)bf16lo(q[i]);
      w[2 * i + 1] = (double)bf16hi(q[i]);
    }
  } else if (vec && nvalid == 8) {
    const float4 a = *reinterpret_cast<const float4*>((const float*)W + off);
    const float4 b = *reinterpret_cast<const float4*>((const float*)W + off + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (i < nvalid) ? (double)ActTraits<TIn>::load(W, off + i) : 0.0;
  }
}

// Rank-based top-k of one token (E <= 256) by one wave; lg in LDS.
// SL = logit slots per lane (E <= 64 * SL): the code a single call runs
// shrinks with E, which matters for the one-work-group decode router.
template <int SL>
__device__ void wave_topk_rank_sl(const float* lg, int E, int k, int renormalize, int32_t* sel /* LDS [k] */,
                                  double* ps /* LDS [max(E,k)] */, int32_t* out_idx, float* out_w) {
  const int lane = lane_id();
  float v[SL];
  int rank[SL];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    v[i] = (lane + 64 * i < E) ? lg[lane + 64 * i] : -INFINITY;
    rank[i] = 0;
  }
  // slots start at a valid expert (a NaN logit compares with nothing)
  if (lane < k) sel[lane] = 0;
  // every other logit comes from a register of the wave (readlane) rather
  // than from LDS, which would cost one LDS round trip per compared logit.
  // Padding slots hold -inf at indexes >= E and never precede a real expert.
#pragma unroll
  for (int i2 = 0; i2 < SL; ++i2) {
    if (64 * i2 >= E) break;
#pragma unroll
    for (int l = 0; l < 64; ++l) {
      const int e2 = 64 * i2 + l;
      const float u = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i2]), l));
      m = fmaxf(m, u);
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        const int e = lane + 64 * i;
        rank[i] += (u > v[i] || (u == v[i] && e2 < e)) ? 1 : 0;
      }
    }
  }
  double p[SL];
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const int e = lane + 64 * i;
    p[i] = (e < E) ? exp((double)v[i] - (double)m) : 0.0;
    if (e < E && rank[i] < k) {
      sel[rank[i]] = e;
      if (renormalize) ps[rank[i]] = p[i];
    }
    if (!renormalize && e < E) ps[e] = p[i];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0);
  double den = 0.0;
  const int nden = renormalize ? k : E;   // slot order, or expert index order
  for (int j = 0; j < nden; ++j) den += ps[j];
  if (lane < k) {
    const int e = sel[lane];
    out_idx[lane] = e;
    out_w[lane] = (float)((renormalize ? ps[lane] : ps[e]) / den);
  }
}

__device__ void wave_topk_rank(const float* lg, int E, int k, int renormalize, int32_t* sel, double* ps,
                               int32_t* out_idx, float* out_w) {
  if (E <= 64) wave_topk_rank_sl<1>(lg, E, k, renormalize, sel, ps, out_idx, out_w);
  else if (E <= 128) wave_topk_rank_sl<2>(lg, E, k, renormalize, sel, ps, out_idx, out_w);
  else wave_topk_rank_sl<4>(lg, E, k, renormalize, sel, ps, out_idx, out_w);
}

constexpr int kSmallMaxS = 32;   // d slices of a split small-T router

template <typename TIn, int MT>
__global__ __launch_bounds__(kSmallThreads) void route_small_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ W, const float* __restrict__ bias, int T, int d,
    int E, int k, int renormalize, int cap, float* __restrict__ logits_out, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, int32_t* __restrict__ plan, const double* __restrict__ part, int S,
    double* __restrict__ part_out, int dsplit) {
  __shared__ double wpart[kSmallThreads][8];
  __shared__ float lg[MT * 1024];
  __shared__ int32_t sidx[MT * 32];
  __shared__ double ps[MT][256];
  __shared__ double psel[MT][32];
  __shared__ int32_t flag[1024];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // slots start at a valid expert, so a logit that compares with nothing
  // (NaN) cannot leave an index for the plan to follow
  for (int a = tid; a < T * k; a += kSmallThreads) sidx[a] = 0;
  const bool vec_ok = (E % 8) == 0;    // rows of W_g are 16-byte aligned only then
  // split mode (part_out set): work-group z sums rows z * dsplit .. + dsplit - 1
  // of x W_g in fp64 and writes them as slice z's partial logits, nothing else
  const int r_lo = part_out ? (int)blockIdx.x * dsplit : 0;
  const int r_hi = part_out ? min(d, r_lo + dsplit) : d;
  if (part) {
    // wide routers: the S fp64 partial sums over slices of d (split-K kernel)
    // are added in slice order
    for (int i = tid; i < T * E; i += kSmallThreads) {
      const int t = i / E, e = i % E;
      double v[kSmallMaxS];   // all loads in flight before the first add; past S: repeats, not added
#pragma unroll
      for (int z = 0; z < kSmallMaxS; ++z) v[z] = part[((size_t)min(z, S - 1) * T + t) * E + e];
      double sum = 0.0;
#pragma unroll
      for (int z = 0; z < kSmallMaxS; ++z)
        if (z < S) sum += v[z];
      if (bias) sum += (double)bias[e];
      const float lv = (float)sum;
      lg[t * 1024 + e] = lv;
      if (logits_out) logits_out[(size_t)t * E + e] = lv;
    }
    __syncthreads();
  }
  for (int e0 = 0; e0 < (part ? 0 : E); e0 += 512) {
    const int ne = min(E - e0, 512);
    const int nchunk = (ne + 7) / 8;
    int ecp = 1;
    while (ecp < nchunk) ecp <<= 1;          // chunks per wave row, power of two <= 64
    const int ec = lane & (ecp - 1);
    const int rows_per_wave = 64 / ecp;
    const int rg = wave * rows_per_wave + lane / ecp;
    const int RG = kSmallWaves * rows_per_wave;
    const int nvalid = (ec < nchunk) ? min(8, ne - ec * 8) : 0;
    double acc[MT][8];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[t][j] = 0.0;
    constexpr int RB = (MT <= 2) ? 8 : 4;     // rows whose loads are issued together
    if (vec_ok) {
      // Branch-free: out-of-range rows and padding chunks load a valid address
      // and contribute zero, so all loads of a batch are in flight together.
      const int ecl = min(ec, nchunk - 1);
      const TIn* wbase = W + e0 + ecl * 8;
      for (int r0 = r_lo + rg; r0 < r_hi; r0 += RB * RG) {
        uint4 raw[RB][sizeof(TIn) == 2 ? 1 : 2];
        TIn xr[RB][MT];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const int rc = min(r0 + b * RG, r_hi - 1);
          const uint4* src = reinterpret_cast<const uint4*>(wbase + (size_t)rc * E);
          raw[b][0] = src[0];
          if (sizeof(TIn) == 4) raw[b][sizeof(TIn) == 2 ? 0 : 1] = src[1];
#pragma unroll
          for (int t = 0; t < MT; ++t) xr[b][t] = x[(size_t)min(t, T - 1) * d + rc];
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const bool live = (r0 + b * RG) < r_hi;
          double wv[8];
          if (sizeof(TIn) == 2) {
            const uint32_t q[4] = {raw[b][0].x, raw[b][0].y, raw[b][0].z, raw[b][0].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              wv[2 * i] = (double)bf16lo(q[i]);
              wv[2 * i + 1] = (double)bf16hi(q[i]);
            }
          } else {
            const uint32_t q[8] = {raw[b][0].x, raw[b][0].y, raw[b][0].z, raw[b][0].w,
                                   raw[b][sizeof(TIn) == 2 ? 0 : 1].x, raw[b][sizeof(TIn) == 2 ? 0 : 1].y,
                                   raw[b][sizeof(TIn) == 2 ? 0 : 1].z, raw[b][sizeof(TIn) == 2 ? 0 : 1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) wv[i] = (double)__uint_as_float(q[i]);
          }
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const double xv = (live && t < T) ? (double)ActTraits<TIn>::load(&xr[b][t], 0) : 0.0;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[t][j] = __fma_rn(xv, wv[j], acc[t][j]);
          }
        }
      }
    } else if (nvalid > 0) {
      // E not a multiple of 8: element loads (rare shapes, not latency tuned)
      for (int r = r_lo + rg; r < r_hi; r += RG) {
        double wv[8];
        load8<TIn>(W, (size_t)r * E + e0 + ec * 8, nvalid, false, wv);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const double xv = (t < T) ? (double)ActTraits<TIn>::load(x, (size_t)t * d + r) : 0.0;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[t][j] = __fma_rn(xv, wv[j], acc[t][j]);
        }
      }
    }
    // Reduction over the row groups, one token at a time: every thread stores
    // its 8 sums in LDS; output (chunk c, column j) is then added by L lanes
    // (each over a fixed stride of row groups) and a fixed butterfly across
    // those L lanes of one wave.
    const int nout = nchunk * 8;
    int L = 1;
    while (L * nout * 2 <= kSmallThreads && L < 64) L <<= 1;
    const int o = tid / L, l = tid % L;
    const int oc = o >> 3, oj = o & 7;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t >= T) break;
#pragma unroll
      for (int j = 0; j < 8; ++j) wpart[tid][j] = acc[t][j];
      __syncthreads();
      double sum = 0.0;
      if (o < nout) {
        // thread (rg, ec) stored its sums at index rg_wave * 64 + lane; row
        // group r of chunk c lives at thread r * ecp + c (waves hold
        // rows_per_wave row groups each)
        for (int r = l; r < RG; r += L) sum += wpart[r * ecp + oc][oj];
      }
      for (int off = 1; off < L; off <<= 1) sum += __shfl_xor(sum, off);
      if (o < nout && l == 0 && oc * 8 + oj < ne && part_out) {
        part_out[((size_t)blockIdx.x * T + t) * E + e0 + oc * 8 + oj] = sum;
      } else if (o < nout && l == 0 && oc * 8 + oj < ne) {
        const int e = e0 + oc * 8 + oj;
        if (bias) sum += (double)bias[e];
        const float lv = (float)sum;
        lg[t * 1024 + e] = lv;
        if (logits_out) logits_out[(size_t)t * E + e] = lv;
      }
      __syncthreads();
    }
  }
  if (part_out) return;
  if (E <= 256) {
    // Rank-based top-k over the whole work-group: R adjacent lanes share one
    // (token, expert) logit, each counts the logits that precede it (larger,
    // or equal with a lower index) over a contiguous 1/R of the token's
    // experts and takes their maximum; a butterfly over the R lanes adds the
    // counts and the maxima.  One wave per token left the other waves idle
    // and made this the router's longest step at T = 1, E = 128.
    int R = 1;
    while (R < 64 && 2 * R * T * E <= kSmallThreads && 16 * R <= E) R <<= 1;
    const int chunk = (E + R - 1) / R;
    for (int i0 = tid; i0 < T * E * R; i0 += kSmallThreads) {
      const int item = i0 / R, q = i0 - item * R;
      const int t = item / E, e = item - t * E;
      const float* l = lg + t * 1024;
      const float v = l[e];
      const int lo = q * chunk, hi = min(E, lo + chunk);
      int r = 0;
      float m = -INFINITY;
#pragma unroll 8
      for (int e2 = lo; e2 < hi; ++e2) {
        const float u = l[e2];
        m = fmaxf(m, u);
        r += (u > v || (u == v && e2 < e)) ? 1 : 0;
      }
      for (int off = 1; off < R; off <<= 1) {   // the R lanes of an item are active together
        r += __shfl_xor(r, off);
        m = fmaxf(m, __shfl_xor(m, off));
      }
      if (q == 0) {
        const double pv = exp((double)v - (double)m);
        if (r < k) {
          sidx[t * k + r] = e;
          psel[t][r] = pv;
        }
        if (!renormalize) ps[t][e] = pv;
      }
    }
    __syncthreads();
    // weights: the chosen experts (slot order) or all experts (index order)
    // form the denominator
    for (int a = tid; a < T * k; a += kSmallThreads) {
      const int t = a / k, j = a - t * k;
      double den = 0.0;
      if (renormalize) {
        for (int q = 0; q < k; ++q) den += psel[t][q];
      } else {
        for (int q = 0; q < E; ++q) den += ps[t][q];
      }
      idx_out[a] = sidx[a];
      w_out[a] = (float)(psel[t][j] / den);
    }
  } else if (wave < T) {
    wave_topk(lg + wave * 1024, E, k, renormalize, sidx + wave * k, w_out + (size_t)wave * k);
  }
  __syncthreads();
  const int n = T * k;
  if (E > 256)
    for (int a = tid; a < n; a += kSmallThreads) idx_out[a] = sidx[a];
  if (!plan) return;
  for (int e = tid; e < E; e += kSmallThreads) flag[e] = 0;
  __syncthreads();
  int keep = 0;   // n <= 8 * 32 = 256: at most one assignment per thread
  if (tid < n) {
    const int e = sidx[tid];
    int r = 0;
    if (cap >= 0) {
#pragma unroll 8
      for (int b = 0; b < tid; ++b) r += (sidx[b] == e);
    }
    keep = (cap < 0 || r < cap);
    if (keep) flag[e] = 1;     // benign: all writers store 1
  }
  __syncthreads();
  // wave 0: exclusive scan of the flags with ballots, 64 experts at a time
  if (wave == 0) {
    int run = 0;
    for (int c0 = 0; c0 < E; c0 += 64) {
      const int e = c0 + lane;
      const bool f = (e < E) && flag[e];
      const uint64_t m = ballot64(f);
      const int pos = run + __popcll(m & lanemask_lt());
      if (e < E) flag[e] = f ? pos : -1;
      if (f) plan[1 + pos] = e;
      run += __popcll(m);
    }
    if (lane == 0) plan[0] = run;
  }
  __syncthreads();
  if (tid < n) plan[1 + E + tid] = keep ? flag[sidx[tid]] : -1;
}

// One wave per token: add the S fp64 partial sums of each logit in slice
// order, add the bias, round once to fp32, then top-k and weights.
// ZB slices' loads are in flight together (4 for S <= 4, else 32).
template <int ZB>
__global__ __launch_bounds__(256) void topk_finalize_kernel(const double* __restrict__ part, int S,
                                                            const float* __restrict__ bias, int T, int E, int k,
                                                            int renormalize, float* __restrict__ logits,
                                                            int32_t* __restrict__ idx, float* __restrict__ w) {
  __shared__ float lg[4][1024];
  __shared__ int32_t sel[4][32];
  __shared__ double ps[4][256];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;     // whole wave leaves together; no block barrier follows
  // the slices of up to two experts per lane are loaded together (one memory
  // round trip for S <= ZB, padding loads repeat a valid address) and added
  // in slice order
  for (int e0 = lane; e0 < E; e0 += 128) {
    const int e1 = e0 + 64;
    const int e1c = e1 < E ? e1 : e0;
    double s0 = 0.0, s1 = 0.0;
    for (int z = 0; z < S; z += ZB) {
      double v0[ZB], v1[ZB];
#pragma unroll
      for (int i = 0; i < ZB; ++i) {
        const size_t row = ((size_t)min(z + i, S - 1) * T + t) * E;
        v0[i] = part[row + e0];
        v1[i] = part[row + e1c];
      }
#pragma unroll
      for (int i = 0; i < ZB; ++i)
        if (z + i < S) {
          s0 += v0[i];
          s1 += v1[i];
        }
    }
    if (bias) {
      s0 += (double)bias[e0];
      s1 += (double)bias[e1c];
    }
    const float l0 = (float)s0, l1 = (float)s1;
    lg[wv][e0] = l0;
    if (logits) logits[(size_t)t * E + e0] = l0;
    if (e1 < E) {
      lg[wv][e1] = l1;
      if (logits) logits[(size_t)t * E + e1] = l1;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0);
  // rank-based selection (every lane counts the logits that precede its own:
  // E / 64 slots x 64 comparisons per lane, a short critical path) for the
  // latency-bound launches of few tokens and E <= 128; k rounds of a wave
  // argmax otherwise (fewer instructions when many waves share the SIMDs or E
  // is large).  Measured on MI355X: fine-grained (T 2048, E 256, k 8) 27-30
  // -> 16.5 us, Mixtral prefill (T 4096, E 8) 11.0 -> 7.8 us; fp8 layer
  // (T 512, E 128, k 8) 9.1 us rank-based against 12.3 us.
  if (E <= 128 && T < 1024)
    wave_topk_rank(lg[wv], E, k, renormalize, sel[wv], ps[wv], idx + (size_t)t * k, w + (size_t)t * k);
  else
    wave_topk(lg[wv], E, k, renormalize, idx + (size_t)t * k, w + (size_t)t * k);
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
// Layers of at most this many 16 x 16 tiles run the small-layer partial kernel.
constexpr long kTileRouterMaxTiles = 256;

static bool tile_router(int T, int E) { return (long)((T + 15) / 16) * ((E + 15) / 16) <= kTileRouterMaxTiles; }

// K split of the partial-logit kernels.  LDS-staged tiles: enough work-groups
// (>= 512) to fill the chip, each K range a multiple of 16 and at least 64
// long.  16 x 16 tiles: about 1024 work-groups (four waves per SIMD), each
// slice at least 256 long (two 32-wide chunks per wave) and a multiple of 32.
static void router_split(int T, int d, int E, int* S, int* dsplit) {
  const bool tile = tile_router(T, E);
  const int bt = tile ? 16 : (E <= 16 ? 256 : 64), be = tile ? 16 : (E <= 16 ? 16 : 64);
  const long target = tile ? 1024 : 512, minlen = tile ? 256 : 64, align = tile ? 32 : 16;
  const long nblk = (long)((T + bt - 1) / bt) * ((E + be - 1) / be);
  long s = (target + nblk - 1) / nblk;
  const long smax = d / minlen > 0 ? d / minlen : 1;
  s = s < 1 ? 1 : (s > smax ? smax : s);
  const int ds = (int)((d + s - 1) / s);
  *dsplit = (int)((ds + align - 1) / align * align);
  *S = (d + *dsplit - 1) / *dsplit;
}

// Small T: one work-group reads all of W_g, which at d * E > 64 K weights
// takes longer than spreading the dot products over split-K work-groups.
static bool small_t_split(int d, int E) { return (long)d * E > 65536; }

// Small T, split: slices of at least 64 rows and about 16 K weights of W_g
// each (one batch of loads per thread of the 512-thread work-group), at most
// kSmallMaxS slices (the top-k kernel adds them with all loads in flight).
static void router_split_small(int d, int E, int* S, int* dsplit) {
  int ds = 16384 / (E > 0 ? E : 1);
  ds = ds < 64 ? 64 : ds;
  if ((d + ds - 1) / ds > kSmallMaxS) ds = (d + kSmallMaxS - 1) / kSmallMaxS;
  *dsplit = (ds + 15) / 16 * 16;
  *S = (d + *dsplit - 1) / *dsplit;
}

size_t router_partial_bytes(int T, int d, int E) {
  int S, ds;
  if (T <= kDecodeMaxT) {
    if (!small_t_split(d, E)) return 0;
    router_split_small(d, E, &S, &ds);
  } else {
    router_split(T, d, E, &S, &ds);
  }
  return (size_t)S * T * E * sizeof(double);
}

template <typename TIn>
static hipError_t launch_partials(const void* x, const void* W, double* part, int T, int d, int E, int S, int ds,
                                  hipStream_t s) {
  const TIn* xp = (const TIn*)x;
  const TIn* wp = (const TIn*)W;
  if (tile_router(T, E))
    router_partial_tile<TIn><<<dim3((T + 15) / 16, (E + 15) / 16, S), 256, 0, s>>>(xp, wp, part, T, d, E, ds);
  else if (E <= 16)
    router_partial_lds<TIn, 16><<<dim3((T + 255) / 256, (E + 15) / 16, S), 256, 0, s>>>(xp, wp, part, T, d, E, ds);
  else
    router_partial_lds<TIn, 64><<<dim3((T + 63) / 64, (E + 63) / 64, S), 256, 0, s>>>(xp, wp, part, T, d, E, ds);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T <= kDecodeMaxT) {
    const int mt = a.T <= 1 ? 1 : a.T <= 2 ? 2 : a.T <= 4 ? 4 : 8;
    // split: S work-groups write the slices' partial logits, then one
    // work-group adds them and selects
    int S = 0, ds = 0;
    if (a.part && small_t_split(a.d, a.E)) router_split_small(a.d, a.E, &S, &ds);
    const double* part = S ? a.part : nullptr;
#define MOE_ROUTE_SMALL(TY, MTV)                                                                               \
  do {                                                                                                         \
    if (S)                                                                                                     \
      route_small_kernel<TY, MTV><<<S, kSmallThreads, 0, s>>>((const TY*)a.x, (const TY*)a.W_g, nullptr, a.T,  \
                                                              a.d, a.E, a.k, a.renormalize, a.cap, nullptr,    \
                                                              nullptr, nullptr, nullptr, nullptr, 0, a.part, ds); \
    route_small_kernel<TY, MTV><<<1, kSmallThreads, 0, s>>>((const TY*)a.x, (const TY*)a.W_g, a.bias, a.T, a.d,  \
                                                            a.E, a.k, a.renormalize, a.cap, a.logits, a.idx, a.w,  \
                                                            a.plan, part, S, nullptr, 0);                     \
  } while (0)
    if (a.act_f32) {
      if (mt == 1) MOE_ROUTE_SMALL(float, 1); else if (mt == 2) MOE_ROUTE_SMALL(float, 2);
      else if (mt == 4) MOE_ROUTE_SMALL(float, 4); else MOE_ROUTE_SMALL(float, 8);
    } else {
      if (mt == 1) MOE_ROUTE_SMALL(bf16_t, 1); else if (mt == 2) MOE_ROUTE_SMALL(bf16_t, 2);
      else if (mt == 4) MOE_ROUTE_SMALL(bf16_t, 4); else MOE_ROUTE_SMALL(bf16_t, 8);
    }
#undef MOE_ROUTE_SMALL
    return hipGetLastError();
  }
  int S, ds;
  router_split(a.T, a.d, a.E, &S, &ds);
  hipError_t err = a.act_f32 ? launch_partials<float>(a.x, a.W_g, a.part, a.T, a.d, a.E, S, ds, s)
                             : launch_partials<bf16_t>(a.x, a.W_g, a.part, a.T, a.d, a.E, S, ds, s);
  if (err != hipSuccess) return err;
  if (S <= 4)
    topk_finalize_kernel<4><<<(a.T + 3) / 4, 256, 0, s>>>(a.part, S, a.bias, a.T, a.E, a.k, a.renormalize, a.logits,
                                                          a.idx, a.w);
  else
    topk_finalize_kernel<32><<<(a.T + 3) / 4, 256, 0, s>>>(a.part, S, a.bias, a.T, a.E, a.k, a.renormalize,
                                                           a.logits, a.idx, a.w);
  return hipGetLastError();
}

}  // namespace moe
