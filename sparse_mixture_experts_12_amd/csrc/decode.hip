// Fused decode path of the MoE layer (T <= 8 tokens) on gfx950.
//
// Pages: "perf(moe): route granite-4.0-h single-token MoE through the fused
// kernel" (a fused single-token kernel computes the chosen experts' SwiGLU
// and their weighted sum; the gather path is the fallback); "Faster writing:
// run only the chosen experts; uncap the large profile" (decode is bound by
// the weight bytes read, so only the chosen experts' weights are touched).
//
// At decode sizes the whole cost is streaming the chosen experts' weights
// from HBM once.  Work unit = (used expert u, slice s of FS intermediate
// columns); one work-group per unit:
//   phase 1: stream W_gate[:, slice] and W_up[:, slice] (d rows of FS
//            columns each), dot with the T token rows (x staged in LDS),
//            reduce over row groups in a fixed order -> h[t, slice] =
//            silu(g) * u (fp32, kept in LDS);
//   phase 2: stream the contiguous block W_down[slice, :] (FS rows of d) and
//            write the partial product h[t, slice] . W_down[slice, :] (fp32).
// No phase needs a grid-wide barrier.  A small second kernel sums the slices
// of each used expert in a fixed order, applies the routing weights in slot
// order (+ the shared expert with weight 1) and rounds once to bf16.
// No atomics: results are bitwise reproducible.
#include <hip/hip_ext.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace moe {

struct DecodeParams {
  const bf16_t* x;
  const int32_t* plan;
  ExpertWeights w;
  int T, d, E, k, f, maxU, has_shared;
  float* partial;        // [units][n_slices][T][d]
};

template <int WK, int MT, int FS>
__global__ __launch_bounds__(256) void decode_ffn_kernel(DecodeParams p) {
  constexpr int ES = (WK == W_FP8) ? 1 : 2;
  constexpr int CPL = 16 / ES;                 // weight columns per 16-byte load
  constexpr int CH = FS / CPL;                 // chunks per slice row per matrix
  constexpr int TPR = 2 * CH;                  // threads per row (gate + up)
  constexpr int RG = 256 / TPR;                // row groups
  constexpr int U = 8;                         // loads in flight per thread
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int s = blockIdx.x;
  const int unit = blockIdx.y;
  const int n_slices = p.f / FS;
  int e;
  const bool shared = (unit == p.maxU);
  if (!shared) {
    if (unit >= p.plan[0]) return;
    e = p.plan[1 + unit];
  } else {
    e = -1;
  }
  const int tid = threadIdx.x;
  const int d = p.d;
  const int T = p.T;

  // ---- stage x (bf16) as xs[r][MT] ----
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem);
  for (int i = tid; i < d * MT; i += 256) {
    const int r = i / MT, t = i % MT;
    xs[i] = (t < T) ? p.x[(size_t)t * d + r] : (bf16_t)0;
  }
  __syncthreads();

  const size_t mstride = (size_t)d * p.f;
  const unsigned char* Wg;
  const unsigned char* Wu;
  const unsigned char* Wd;
  if (shared) {
    Wg = (const unsigned char*)p.w.Wsg; Wu = (const unsigned char*)p.w.Wsu; Wd = (const unsigned char*)p.w.Wsd;
  } else {
    Wg = (const unsigned char*)p.w.Wg + (size_t)e * mstride * ES;
    Wu = (const unsigned char*)p.w.Wu + (size_t)e * mstride * ES;
    Wd = (const unsigned char*)p.w.Wd + (size_t)e * mstride * ES;
  }

  // ---- phase 1 ----
  const int m = (tid % TPR) / CH;        // 0 gate, 1 up
  const int c = tid % CH;
  const int rg = tid / TPR;
  const unsigned char* Wm = (m == 0 ? Wg : Wu) + ((size_t)s * FS + c * CPL) * ES;
  const size_t rstride = (size_t)p.f * ES;
  float acc[MT][CPL];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < CPL; ++j) acc[t][j] = 0.f;

  auto fma_row = [&](const u32x4_t& wv, int r) {
    float xv[MT];
    if (MT == 1) {
      xv[0] = bf16_to_f32(xs[r]);
    } else {
#pragma unroll
      for (int t = 0; t < MT; ++t) xv[t] = bf16_to_f32(xs[r * MT + t]);
    }
    float wf[CPL];
    const uint32_t* ww = reinterpret_cast<const uint32_t*>(&wv);
    if (WK == W_FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) fp8x4_to_f32(ww[q], wf + 4 * q);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) { wf[2 * q] = bf16lo(ww[q]); wf[2 * q + 1] = bf16hi(ww[q]); }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < CPL; ++j) acc[t][j] = __fmaf_rn(xv[t], wf[j], acc[t][j]);
  };

  int r = rg;
  for (; r + (U - 1) * RG < d; r += U * RG) {
    u32x4_t wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) wv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Wm + (size_t)(r + u * RG) * rstride));
#pragma unroll
    for (int u = 0; u < U; ++u) fma_row(wv[u], r + u * RG);
  }
  for (; r < d; r += RG) {
    u32x4_t wv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Wm + (size_t)r * rstride));
    fma_row(wv, r);
  }
  __syncthreads();   // xs no longer needed: reuse LDS for the reduction

  float* red = reinterpret_cast<float*>(smem);       // [RG][2][MT][FS]
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < CPL; ++j) red[((rg * 2 + m) * MT + t) * FS + c * CPL + j] = acc[t][j];
  __syncthreads();
  float* hs = red + RG * 2 * MT * FS;                // [MT][FS]
  for (int i = tid; i < MT * FS; i += 256) {
    const int t = i / FS, col = i % FS;
    float g = 0.f, u = 0.f;
    for (int q = 0; q < RG; ++q) {
      g += red[((q * 2 + 0) * MT + t) * FS + col];
      u += red[((q * 2 + 1) * MT + t) * FS + col];
    }
    if (WK == W_FP8) {
      const int fc = s * FS + col;
      g *= shared ? p.w.ssg[fc] : p.w.sg[(size_t)e * p.f + fc];
      u *= shared ? p.w.ssu[fc] : p.w.su[(size_t)e * p.f + fc];
    }
    hs[i] = silu_f(g) * u;
  }
  __syncthreads();

  // ---- phase 2: W_down[slice, :] is FS contiguous rows of d ----
  const unsigned char* Wds = Wd + (size_t)s * FS * d * ES;
  const int nchunks = d / CPL;
  float* out = p.partial + ((size_t)unit * n_slices + s) * T * d;
  for (int ch = tid; ch < nchunks; ch += 256) {
    float a2[MT][CPL];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < CPL; ++j) a2[t][j] = 0.f;
    const unsigned char* base = Wds + (size_t)ch * 16;
#pragma unroll 1
    for (int r0 = 0; r0 < FS; r0 += U) {
      u32x4_t wv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) wv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + (size_t)(r0 + u) * d * ES));
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float wf[CPL];
        const uint32_t* ww = reinterpret_cast<const uint32_t*>(&wv[u]);
        if (WK == W_FP8) {
#pragma unroll
          for (int q = 0; q < 4; ++q) fp8x4_to_f32(ww[q], wf + 4 * q);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) { wf[2 * q] = bf16lo(ww[q]); wf[2 * q + 1] = bf16hi(ww[q]); }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const float hv = hs[t * FS + r0 + u];
#pragma unroll
          for (int j = 0; j < CPL; ++j) a2[t][j] = __fmaf_rn(hv, wf[j], a2[t][j]);
        }
      }
    }
    const int col0 = ch * CPL;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t >= T) break;
      float* o = out + (size_t)t * d + col0;
#pragma unroll
      for (int j = 0; j < CPL; j += 4) {
        float4 v = make_float4(a2[t][j], a2[t][j + 1], a2[t][j + 2], a2[t][j + 3]);
        if (WK == W_FP8) {
          const float* sc = shared ? p.w.ssd + col0 + j : p.w.sd + (size_t)e * d + col0 + j;
          v.x *= sc[0]; v.y *= sc[1]; v.z *= sc[2]; v.w *= sc[3];
        }
        *reinterpret_cast<float4*>(o + j) = v;
      }
    }
  }
}

// Sum the slice partials of the used experts for 16 columns of one token:
// out = sum_j w[t,j] * partial[unit(t,j)][s] (+ shared partials).  Thread
// (slice lane sl, column quad cq) accumulates s = sl, sl + 64, ... unit-major
// in a fixed order; the 64 slice lanes are then added by a fixed LDS tree and
// the result is rounded once to bf16.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ partial,
                                                            const int32_t* __restrict__ plan,
                                                            const float* __restrict__ topk_w, int T, int d, int E,
                                                            int k, int n_slices, int maxU, int has_shared,
                                                            bf16_t* __restrict__ out) {
  __shared__ float4 red[64][4];
  const int t = blockIdx.y;
  const int cq = threadIdx.x & 3;
  const int sl = threadIdx.x >> 2;
  const int col = blockIdx.x * 16 + cq * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int nunits = k + (has_shared ? 1 : 0);
  for (int j = 0; j < nunits; ++j) {
    int unit;
    float wgt;
    if (j < k) {
      unit = plan[1 + E + t * k + j];
      wgt = topk_w[t * k + j];
      if (unit < 0) continue;    // dropped by the capacity rule
    } else {
      unit = maxU;
      wgt = 1.f;
    }
    const float* base = partial + ((size_t)unit * n_slices * T + t) * d + col;
#pragma unroll 4
    for (int s = sl; s < n_slices; s += 64) {
      const float4 v = *reinterpret_cast<const float4*>(base + (size_t)s * T * d);
      acc.x = __fmaf_rn(wgt, v.x, acc.x);
      acc.y = __fmaf_rn(wgt, v.y, acc.y);
      acc.z = __fmaf_rn(wgt, v.z, acc.z);
      acc.w = __fmaf_rn(wgt, v.w, acc.w);
    }
  }
  red[sl][cq] = acc;
  __syncthreads();
  for (int half = 32; half >= 1; half >>= 1) {
    if (sl < half) {
      const float4 o = red[sl + half][cq];
      float4 v = red[sl][cq];
      v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
      red[sl][cq] = v;
    }
    __syncthreads();
  }
  if (sl == 0) {
    const float4 tot = red[0][cq];
    uint2 o;
    o.x = pack_bf16x2(tot.x, tot.y);
    o.y = pack_bf16x2(tot.z, tot.w);
    *reinterpret_cast<uint2*>(out + (size_t)t * d + col) = o;
  }
}

static int pick_mt(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8; }

// Slice width: the widest slice (longest contiguous row segment of W_gate /
// W_up, at most 512 bytes) that still gives every CU at least one work unit.
static int pick_fs(int units, int f, int es) {
  static int forced = -1;
  if (forced < 0) {
    const char* e = getenv("MOE_DECODE_FS");
    forced = e ? atoi(e) : 0;
  }
  if ((forced == 64 || forced == 128 || forced == 256) && f % forced == 0) return forced;
  const int cands[3] = {256, 128, 64};
  for (int c : cands) {
    if (f % c) continue;
    if (c * es > 512) continue;
    if (units * (f / c) >= 200) return c;
  }
  return 64;
}

static int decode_max_used(int T, int k, int E) { return (T * k < E) ? T * k : E; }

size_t decode_partial_bytes(int T, int d, int E, int k, int f, int has_shared, int wkind) {
  (void)wkind;
  const int units = decode_max_used(T, k, E) + (has_shared ? 1 : 0);
  return (size_t)units * (size_t)(f / 64) * T * d * sizeof(float);
}

template <int WK, int MT, int FS>
static hipError_t launch_decode_t(const DecodeParams& p, int units, hipStream_t s, hipEvent_t ev_begin,
                                  hipEvent_t ev_end) {
  constexpr int ES = (WK == W_FP8) ? 1 : 2;
  constexpr int CH = FS / (16 / ES);
  constexpr int RG = 256 / (2 * CH);
  size_t xs_bytes = (size_t)p.d * MT * sizeof(bf16_t);
  size_t red_bytes = (size_t)(RG * 2 * MT * FS + MT * FS) * sizeof(float);
  size_t lds = xs_bytes > red_bytes ? xs_bytes : red_bytes;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_ffn_kernel<WK, MT, FS>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(p.f / FS, units);
  if (ev_begin || ev_end)
    hipExtLaunchKernelGGL(decode_ffn_kernel<WK, MT, FS>, grid, dim3(256), (uint32_t)lds, s, ev_begin, ev_end, 0, p);
  else
    decode_ffn_kernel<WK, MT, FS><<<grid, 256, lds, s>>>(p);
  return hipGetLastError();
}

template <int WK, int MT>
static hipError_t launch_decode_fs(const DecodeParams& p, int units, int fs, hipStream_t s, hipEvent_t b,
                                   hipEvent_t e) {
  if (fs == 256) return launch_decode_t<WK, MT, 256>(p, units, s, b, e);
  if (fs == 128) return launch_decode_t<WK, MT, 128>(p, units, s, b, e);
  return launch_decode_t<WK, MT, 64>(p, units, s, b, e);
}

template <int WK>
static hipError_t launch_decode_mt(const DecodeParams& p, int units, int fs, hipStream_t s, hipEvent_t b,
                                   hipEvent_t e) {
  switch (pick_mt(p.T)) {
    case 1: return launch_decode_fs<WK, 1>(p, units, fs, s, b, e);
    case 2: return launch_decode_fs<WK, 2>(p, units, fs, s, b, e);
    case 4: return launch_decode_fs<WK, 4>(p, units, fs, s, b, e);
    default: return launch_decode_fs<WK, 8>(p, units, fs, s, b, e);
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  DecodeParams p{};
  p.x = (const bf16_t*)a.x;
  p.plan = a.plan;
  p.w = a.w;
  p.T = a.T; p.d = a.d; p.E = a.E; p.k = a.k; p.f = a.f;
  p.maxU = decode_max_used(a.T, a.k, a.E);
  p.has_shared = a.has_shared;
  p.partial = a.partial;
  const int units = p.maxU + (a.has_shared ? 1 : 0);
  const int fs = pick_fs(units, a.f, a.wkind == W_FP8 ? 1 : 2);
  hipError_t err = (a.wkind == W_FP8) ? launch_decode_mt<W_FP8>(p, units, fs, s, a.ev_begin, a.ev_end)
                                      : launch_decode_mt<W_BF16>(p, units, fs, s, a.ev_begin, a.ev_end);
  if (err != hipSuccess) return err;
  dim3 g2(a.d / 16, a.T);
  decode_reduce_kernel<<<g2, 256, 0, s>>>(a.partial, a.plan, a.topk_w, a.T, a.d, a.E, a.k, a.f / fs, p.maxU,
                                          a.has_shared, (bf16_t*)a.out);
  return hipGetLastError();
}

}  // namespace moe
