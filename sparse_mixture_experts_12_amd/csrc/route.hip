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
// Large-T logits: BT x BE tile per work-group, fp64 FMA, LDS staged.
// 256 threads; each thread owns TM tokens x TN experts.
// ---------------------------------------------------------------------------
template <typename TIn, int BT, int BE, int TM, int TN>
__global__ __launch_bounds__(256) void router_logits_tiled(
    const TIn* __restrict__ x, const TIn* __restrict__ W, const float* __restrict__ bias,
    float* __restrict__ logits, int T, int d, int E) {
  constexpr int BK = 16;
  static_assert((BT / TM) * (BE / TN) == 256, "thread tile");
  __shared__ double xs[BK][BT + 1];
  __shared__ double ws[BK][BE + 1];
  const int tid = threadIdx.x;
  const int tx = tid % (BE / TN);   // expert group
  const int ty = tid / (BE / TN);   // token group
  const int t0 = blockIdx.x * BT;
  const int e0 = blockIdx.y * BE;
  double acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.0;

  for (int k0 = 0; k0 < d; k0 += BK) {
    for (int i = tid; i < BT * BK; i += 256) {
      int tt = i / BK, kk = i % BK;
      int t = t0 + tt;
      xs[kk][tt] = (t < T) ? (double)ActTraits<TIn>::load(x, (size_t)t * d + k0 + kk) : 0.0;
    }
    for (int i = tid; i < BK * BE; i += 256) {
      int kk = i / BE, ee = i % BE;
      int e = e0 + ee;
      ws[kk][ee] = (e < E) ? (double)ActTraits<TIn>::load(W, (size_t)(k0 + kk) * E + e) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      double a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = xs[kk][ty * TM + i];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = ws[kk][tx * TN + j];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __fma_rn(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int t = t0 + ty * TM + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int e = e0 + tx * TN + j;
      if (e >= E) continue;
      double s = acc[i][j];
      if (bias) s += (double)bias[e];
      logits[(size_t)t * E + e] = (float)s;
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

__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int T, int E,
                                                           int k, int renormalize, int32_t* __restrict__ idx,
                                                           float* __restrict__ w) {
  int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  wave_topk(logits + (size_t)t * E, E, k, renormalize, idx + (size_t)t * k, w + (size_t)t * k);
}

// ---------------------------------------------------------------------------
// Small-T router (T <= 8) in one work-group: logits for every token, top-k,
// and the decode plan used by the fused decode path:
//   plan[0]            n_used: number of distinct experts with a kept assignment
//   plan[1 .. E]       used expert ids, ascending (first n_used valid)
//   plan[1 + E + a]    for assignment a = t*k + j: index into the used list, or -1
//                      if the assignment is dropped by the capacity rule.
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void route_small_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ W, const float* __restrict__ bias, int T, int d,
    int E, int k, int renormalize, int cap, float* __restrict__ logits_out, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, int32_t* __restrict__ plan) {
  __shared__ double red[256 * kDecodeMaxT];
  __shared__ float lg[kDecodeMaxT * 1024];
  __shared__ int32_t sidx[kDecodeMaxT * 32];
  __shared__ int32_t flag[1024 + 1];
  const int tid = threadIdx.x;
  for (int e0 = 0; e0 < E; e0 += 256) {
    const int ecols = min(E - e0, 256);
    const int rgroups = 256 / ecols;
    const int ec = tid % ecols;
    const int rg = tid / ecols;
    double acc[kDecodeMaxT];
#pragma unroll
    for (int t = 0; t < kDecodeMaxT; ++t) acc[t] = 0.0;
    if (rg < rgroups) {
      for (int r = rg; r < d; r += rgroups) {
        double wv = (double)ActTraits<TIn>::load(W, (size_t)r * E + e0 + ec);
#pragma unroll
        for (int t = 0; t < kDecodeMaxT; ++t)
          if (t < T) acc[t] = __fma_rn((double)ActTraits<TIn>::load(x, (size_t)t * d + r), wv, acc[t]);
      }
#pragma unroll
      for (int t = 0; t < kDecodeMaxT; ++t) red[(rg * ecols + ec) * kDecodeMaxT + t] = acc[t];
    }
    __syncthreads();
    for (int i = tid; i < ecols * T; i += 256) {
      int e = i % ecols, t = i / ecols;
      double s = 0.0;
      for (int g = 0; g < rgroups; ++g) s += red[(g * ecols + e) * kDecodeMaxT + t];
      if (bias) s += (double)bias[e0 + e];
      float l = (float)s;
      lg[t * 1024 + e0 + e] = l;
      if (logits_out) logits_out[(size_t)t * E + e0 + e] = l;
    }
    __syncthreads();
  }
  // top-k: wave w handles tokens w, w + 4
  const int wv = tid >> 6;
  for (int t = wv; t < T; t += 4) {
    wave_topk(lg + t * 1024, E, k, renormalize, sidx + t * k, w_out + (size_t)t * k);
  }
  __syncthreads();
  const int n = T * k;
  for (int a = tid; a < n; a += 256) idx_out[a] = sidx[a];
  if (!plan) return;
  // capacity: rank of a among earlier assignments to the same expert
  for (int e = tid; e <= E; e += 256) flag[e] = 0;
  __syncthreads();
  int keep = 0;   // n <= 8 * 32 = 256 -> at most one assignment per thread
  if (tid < n) {
    int e = sidx[tid];
    int r = 0;
    for (int b = 0; b < tid; ++b) r += (sidx[b] == e);
    keep = (cap < 0 || r < cap);
    if (keep) flag[e] = 1;     // benign: all writers store 1
  }
  __syncthreads();
  // exclusive scan of flags over experts (serial per 256-chunk is fine: E <= 1024)
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      int f = flag[e];
      flag[e] = f ? run : -1;
      if (f) plan[1 + run] = e;
      run += f;
    }
    plan[0] = run;
  }
  __syncthreads();
  if (tid < n) plan[1 + E + tid] = keep ? flag[sidx[tid]] : -1;
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <typename TIn>
static hipError_t launch_logits(const void* x, const void* W, const float* bias, float* logits, int T, int d,
                                int E, hipStream_t s) {
  const TIn* xp = (const TIn*)x;
  const TIn* wp = (const TIn*)W;
  if (E <= 8) {
    dim3 g((T + 255) / 256, (E + 7) / 8);
    router_logits_tiled<TIn, 256, 8, 4, 2><<<g, 256, 0, s>>>(xp, wp, bias, logits, T, d, E);
  } else if (E <= 32) {
    dim3 g((T + 127) / 128, (E + 31) / 32);
    router_logits_tiled<TIn, 128, 32, 4, 4><<<g, 256, 0, s>>>(xp, wp, bias, logits, T, d, E);
  } else {
    dim3 g((T + 31) / 32, (E + 63) / 64);
    router_logits_tiled<TIn, 32, 64, 2, 4><<<g, 256, 0, s>>>(xp, wp, bias, logits, T, d, E);
  }
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T <= kDecodeMaxT) {
    if (a.act_f32)
      route_small_kernel<float><<<1, 256, 0, s>>>((const float*)a.x, (const float*)a.W_g, a.bias, a.T, a.d, a.E,
                                                   a.k, a.renormalize, a.cap, a.logits, a.idx, a.w, a.plan);
    else
      route_small_kernel<bf16_t><<<1, 256, 0, s>>>((const bf16_t*)a.x, (const bf16_t*)a.W_g, a.bias, a.T, a.d,
                                                    a.E, a.k, a.renormalize, a.cap, a.logits, a.idx, a.w,
                                                    a.plan);
    return hipGetLastError();
  }
  hipError_t err = a.act_f32 ? launch_logits<float>(a.x, a.W_g, a.bias, a.logits, a.T, a.d, a.E, s)
                             : launch_logits<bf16_t>(a.x, a.W_g, a.bias, a.logits, a.T, a.d, a.E, s);
  if (err != hipSuccess) return err;
  topk_softmax_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a.logits, a.T, a.E, a.k, a.renormalize, a.idx, a.w);
  return hipGetLastError();
}

}  // namespace moe
