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
// Small-T router (T <= 8) in one work-group of 1024 threads: logits for every
// token, top-k, and the decode plan used by the fused decode path:
//   plan[0]            n_used: number of distinct experts with a kept assignment
//   plan[1 .. E]       used expert ids, ascending (first n_used valid)
//   plan[1 + E + a]    for assignment a = t*k + j: index into the used list, or -1
//                      if the assignment is dropped by the capacity rule.
// Each thread owns one chunk of 8 experts and a strided set of rows of W_g
// (one 16-byte load per row for bf16), all issued before use; per-thread fp64
// sums are combined by a fixed butterfly inside the wave and a fixed-order sum
// over the 16 waves.  Top-k is rank based: every lane counts the logits that
// precede its own (larger, or equal with a lower index), so no serial
// cross-lane selection loop is needed.
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
__device__ void wave_topk_rank(const float* lg, int E, int k, int renormalize, int32_t* sel /* LDS [k] */,
                               double* ps /* LDS [max(E,k)] */, int32_t* out_idx, float* out_w) {
  const int lane = lane_id();
  float v[4];
  int rank[4];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (lane + 64 * i < E) ? lg[lane + 64 * i] : -INFINITY;
    rank[i] = 0;
  }
  for (int e2 = 0; e2 < E; ++e2) {
    const float u = lg[e2];
    m = fmaxf(m, u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      rank[i] += (u > v[i] || (u == v[i] && e2 < e)) ? 1 : 0;
    }
  }
  double p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
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
    const double pe = exp((double)lg[e] - (double)m);
    out_w[lane] = (float)(pe / den);
  }
}

template <typename TIn, int MT>
__global__ __launch_bounds__(kSmallThreads) void route_small_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ W, const float* __restrict__ bias, int T, int d,
    int E, int k, int renormalize, int cap, float* __restrict__ logits_out, int32_t* __restrict__ idx_out,
    float* __restrict__ w_out, int32_t* __restrict__ plan) {
  __shared__ double wpart[kSmallWaves][64][8];
  __shared__ float lg[MT * 1024];
  __shared__ int32_t sidx[MT * 32];
  __shared__ double ps[MT][256];
  __shared__ int32_t flag[1024];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const bool vec_ok = (E % 8) == 0;    // rows of W_g are 16-byte aligned only then
  for (int e0 = 0; e0 < E; e0 += 512) {
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
      for (int r0 = rg; r0 < d; r0 += RB * RG) {
        uint4 raw[RB][sizeof(TIn) == 2 ? 1 : 2];
        TIn xr[RB][MT];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const int rc = min(r0 + b * RG, d - 1);
          const uint4* src = reinterpret_cast<const uint4*>(wbase + (size_t)rc * E);
          raw[b][0] = src[0];
          if (sizeof(TIn) == 4) raw[b][sizeof(TIn) == 2 ? 0 : 1] = src[1];
#pragma unroll
          for (int t = 0; t < MT; ++t) xr[b][t] = x[(size_t)min(t, T - 1) * d + rc];
        }
#pragma unroll
        for (int b = 0; b < RB; ++b) {
          const bool live = (r0 + b * RG) < d;
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
      for (int r = rg; r < d; r += RG) {
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
    // butterfly over the lanes that share a chunk (fixed order)
    for (int off = ecp; off < 64; off <<= 1) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[t][j] += __shfl_xor(acc[t][j], off);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t >= T) break;
      if (lane < ecp) {
#pragma unroll
        for (int j = 0; j < 8; ++j) wpart[wave][lane][j] = acc[t][j];
      }
      __syncthreads();
      if (tid < nchunk * 8) {
        const int c = tid >> 3, j = tid & 7;
        if (c * 8 + j < ne) {
          double s = 0.0;
#pragma unroll
          for (int w = 0; w < kSmallWaves; ++w) s += wpart[w][c][j];
          const int e = e0 + c * 8 + j;
          if (bias) s += (double)bias[e];
          const float l = (float)s;
          lg[t * 1024 + e] = l;
          if (logits_out) logits_out[(size_t)t * E + e] = l;
        }
      }
      __syncthreads();
    }
  }
  // top-k: wave w handles token w
  if (wave < T) {
    if (E <= 256)
      wave_topk_rank(lg + wave * 1024, E, k, renormalize, sidx + wave * k, ps[wave], idx_out + (size_t)wave * k,
                     w_out + (size_t)wave * k);
    else
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
    const int mt = a.T <= 1 ? 1 : a.T <= 2 ? 2 : a.T <= 4 ? 4 : 8;
#define MOE_ROUTE_SMALL(TY, MTV)                                                                          \
  route_small_kernel<TY, MTV><<<1, kSmallThreads, 0, s>>>((const TY*)a.x, (const TY*)a.W_g, a.bias, a.T, a.d, a.E, a.k, \
                                                a.renormalize, a.cap, a.logits, a.idx, a.w, a.plan)
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
  hipError_t err = a.act_f32 ? launch_logits<float>(a.x, a.W_g, a.bias, a.logits, a.T, a.d, a.E, s)
                             : launch_logits<bf16_t>(a.x, a.W_g, a.bias, a.logits, a.T, a.d, a.E, s);
  if (err != hipSuccess) return err;
  topk_softmax_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a.logits, a.T, a.E, a.k, a.renormalize, a.idx, a.w);
  return hipGetLastError();
}

}  // namespace moe
