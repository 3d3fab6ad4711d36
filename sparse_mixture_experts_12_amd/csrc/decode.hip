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
//
// Layers whose used experts are small (many experts of a short f, e.g. 8 of
// 128 experts with f = 768) give the fused kernel too few work-groups to keep
// HBM busy.  They run split: phase 1 additionally splits the d rows over DS
// work-groups, each writing its fp32 (gate, up) sums; a down kernel adds the
// DS parts in order, forms h and streams a block of FS2 rows x DW columns of
// W_down per work-group; the same reduce kernel finishes.
#include <hip/hip_ext.h>
#include <map>
#include <mutex>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace moe {

struct DecodeParams {
  const bf16_t* x;
  const int32_t* plan;
  ExpertWeights w;
  int T, d, E, k, f, maxU, has_shared;
  float* partial;        // [units][n_slices][T][d]
  float* gu;             // split layers: [units][DS][2][T][f] (gate, up) row-split sums
};

// SPLIT: phase 1 only, over rows [z dr, (z + 1) dr) of d, z = blockIdx.z,
// dr = d / gridDim.z; writes the (gate, up) sums of its slice to p.gu.
template <int WK, int MT, int FS, bool SPLIT = false>
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

  const int DS = SPLIT ? (int)gridDim.z : 1;
  const int r_lo = SPLIT ? (int)blockIdx.z * (d / DS) : 0;
  const int r_hi = SPLIT ? r_lo + d / DS : d;

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

  // split layers: this thread's first rows (usually all of them) are loaded
  // before x is staged, so the two memory latencies overlap.  Loads past the
  // thread's rows repeat its last row (no load sits behind a branch, which
  // would make the compiler wait for each one in turn).
  constexpr int UP = SPLIT ? (ES == 1 ? 8 : 16) : 1;   // = rows per thread at 256-column slices, 64-row parts
  u32x4_t wpre[UP];
  if constexpr (SPLIT) {
    const int last = r_lo + rg + ((r_hi - 1 - r_lo - rg) / RG) * RG;
#pragma unroll
    for (int i = 0; i < UP; ++i) {
      const int rr = min(r_lo + rg + i * RG, last);
      wpre[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Wm + (size_t)rr * rstride));
    }
  }

  // ---- stage x rows r_lo .. r_hi - 1 (bf16) as xs[r - r_lo][MT] ----
  // 16-byte chunks c = (row block of 8, token), four per thread in flight;
  // clamped indexes keep every load unconditional, tokens past T stage zeros
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem);
  {
    const int nchunk = (r_hi - r_lo) / 8 * MT;
    for (int c0 = tid; c0 < nchunk; c0 += 4 * 256) {
      u32x4_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = min(c0 + 256 * q, nchunk - 1);
        const int t = c % MT, rb = c / MT;
        v[q] = *reinterpret_cast<const u32x4_t*>(p.x + (size_t)min(t, T - 1) * d + r_lo + rb * 8);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + 256 * q;
        if (c >= nchunk) break;
        const int t = c % MT, rb = c / MT;
        if (t >= T) v[q] = u32x4_t{0u, 0u, 0u, 0u};
        if constexpr (MT == 1) {
          *reinterpret_cast<u32x4_t*>(xs + rb * 8) = v[q];
        } else {
          const unsigned short* hv = reinterpret_cast<const unsigned short*>(&v[q]);
          unsigned short* xw = reinterpret_cast<unsigned short*>(xs);
#pragma unroll
          for (int j = 0; j < 8; ++j) xw[(rb * 8 + j) * MT + t] = hv[j];
        }
      }
    }
  }
  __syncthreads();

  auto fma_row = [&](const u32x4_t& wv, int r) {
    float xv[MT];
    if (MT == 1) {
      xv[0] = bf16_to_f32(xs[r - r_lo]);
    } else {
#pragma unroll
      for (int t = 0; t < MT; ++t) xv[t] = bf16_to_f32(xs[(r - r_lo) * MT + t]);
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

  int r = r_lo + rg;
  if constexpr (SPLIT) {
#pragma unroll
    for (int i = 0; i < UP; ++i)
      if (r + i * RG < r_hi) fma_row(wpre[i], r + i * RG);
    r += UP * RG;
  }
  for (; r + (U - 1) * RG < r_hi; r += U * RG) {
    u32x4_t wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) wv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(Wm + (size_t)(r + u * RG) * rstride));
#pragma unroll
    for (int u = 0; u < U; ++u) fma_row(wv[u], r + u * RG);
  }
  for (; r < r_hi; r += RG) {
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
  if constexpr (SPLIT) {
    // (gate, up) sums of this row part; the scales apply after the parts add
    float* gu = p.gu + ((size_t)unit * DS + blockIdx.z) * 2 * T * p.f;
    for (int i = tid; i < T * FS; i += 256) {
      const int t = i / FS, col = i % FS;
      float g = 0.f, u = 0.f;
      for (int q = 0; q < RG; ++q) {
        g += red[((q * 2 + 0) * MT + t) * FS + col];
        u += red[((q * 2 + 1) * MT + t) * FS + col];
      }
      gu[(size_t)t * p.f + s * FS + col] = g;
      gu[(size_t)(T + t) * p.f + s * FS + col] = u;
    }
    return;
  }
  float* hs = red + RG * 2 * MT * FS;                // [FS][MT]: a row's MT values are contiguous
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
    hs[col * MT + t] = silu_f(g) * u;
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
        float hv[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) hv[t] = hs[(r0 + u) * MT + t];
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int j = 0; j < CPL; ++j) a2[t][j] = __fmaf_rn(hv[t], wf[j], a2[t][j]);
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

constexpr int kMaxDS = 32;   // d-row parts of a split layer's phase 1
constexpr int kMaxDecodeSlots = 33;           // slots of one token: top_k <= 32, + the shared expert

// Split layers, phase 2: work-group (s2, unit, c) adds the DS row parts of
// (gate, up) for intermediate rows s2 * 64 .. +63 in order, forms
// h = silu(g) * u, and streams W_down[those rows, c * DW .. +DW - 1].  Thread
// (row group rg, chunk ch) covers rows rg, rg + RG2, ... of one 16-byte column
// chunk; the RG2 row groups are added in LDS in a fixed order.
template <int WK, int MT, int DW>
__global__ __launch_bounds__(256) void decode_down_kernel(DecodeParams p, int DS) {
  constexpr int ES = (WK == W_FP8) ? 1 : 2;
  constexpr int CPL = 16 / ES;
  constexpr int FS2 = 64;                      // W_down rows per work-group
  constexpr int CW = DW / CPL;                 // 16-byte chunks per row
  constexpr int RG2 = 256 / CW;                // row groups
  constexpr int NR = FS2 / RG2;                // rows per thread (all loads in flight)
  static_assert(CW * RG2 == 256 && NR >= 1 && NR * RG2 == FS2, "down tile shape");
  __shared__ __attribute__((aligned(16))) float hs[FS2][MT];
  __shared__ float red[RG2][DW];
  const int s2 = blockIdx.x;
  const int unit = blockIdx.y;
  const int c0 = blockIdx.z * DW;
  const bool shared = (unit == p.maxU);
  int e = -1;
  if (!shared) {
    if (unit >= p.plan[0]) return;
    e = p.plan[1 + unit];
  }
  const int tid = threadIdx.x;
  const int T = p.T, d = p.d, f = p.f;
  // the W_down block does not depend on h: its loads go out first
  const unsigned char* Wd = shared ? (const unsigned char*)p.w.Wsd
                                   : (const unsigned char*)p.w.Wd + (size_t)e * f * d * ES;
  const int ch = tid % CW, rg = tid / CW;
  const unsigned char* base = Wd + ((size_t)(s2 * FS2 + rg) * d + c0 + ch * CPL) * ES;
  u32x4_t wv[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i)
    wv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + (size_t)i * RG2 * d * ES));
  constexpr int CPT = (DW + 255) / 256;        // output columns per thread in the final sum
  float dsc[CPT];                              // their fp8 column scales, loaded early too
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int col = tid + 256 * i;
    dsc[i] = 1.f;
    if (WK == W_FP8 && col < DW) dsc[i] = shared ? p.w.ssd[c0 + col] : p.w.sd[(size_t)e * d + c0 + col];
  }
  for (int i = tid; i < MT * FS2; i += 256) {
    const int t = i / FS2, j = i % FS2, fc = s2 * FS2 + j;
    float hv = 0.f;
    if (t < T) {
      // all parts' loads are issued before the first add (one memory latency);
      // indexes past DS repeat the last part and are not added
      float gv[kMaxDS], uv[kMaxDS];
      const float* gu = p.gu + (size_t)unit * DS * 2 * T * f + (size_t)t * f + fc;
#pragma unroll
      for (int z = 0; z < kMaxDS; ++z) {
        const size_t zo = (size_t)min(z, DS - 1) * 2 * T * f;
        gv[z] = gu[zo];
        uv[z] = gu[zo + (size_t)T * f];
      }
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int z = 0; z < kMaxDS; ++z) {
        if (z < DS) {
          g += gv[z];
          u += uv[z];
        }
      }
      if (WK == W_FP8) {
        g *= shared ? p.w.ssg[fc] : p.w.sg[(size_t)e * f + fc];
        u *= shared ? p.w.ssu[fc] : p.w.su[(size_t)e * f + fc];
      }
      hv = silu_f(g) * u;
    }
    hs[j][t] = hv;
  }
  __syncthreads();
  float a2[MT][CPL];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int j = 0; j < CPL; ++j) a2[t][j] = 0.f;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    float wf[CPL];
    const uint32_t* ww = reinterpret_cast<const uint32_t*>(&wv[i]);
    if (WK == W_FP8) {
#pragma unroll
      for (int q = 0; q < 4; ++q) fp8x4_to_f32(ww[q], wf + 4 * q);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) { wf[2 * q] = bf16lo(ww[q]); wf[2 * q + 1] = bf16hi(ww[q]); }
    }
    float hv[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) hv[t] = hs[rg + i * RG2][t];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int j = 0; j < CPL; ++j) a2[t][j] = __fmaf_rn(hv[t], wf[j], a2[t][j]);
  }
  const int n_slices = f / FS2;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t >= T) break;
#pragma unroll
    for (int j = 0; j < CPL; ++j) red[rg][ch * CPL + j] = a2[t][j];
    __syncthreads();
    float* out = p.partial + (((size_t)unit * n_slices + s2) * T + t) * d + c0;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int col = tid + 256 * i;
      if (col >= DW) break;
      float v = 0.f;
      for (int q = 0; q < RG2; ++q) v += red[q][col];
      out[col] = WK == W_FP8 ? v * dsc[i] : v;
    }
    __syncthreads();
  }
}

// Sum the slice partials of the used experts for 16 columns of one token:
// out = sum_j w[t,j] * partial[unit(t,j)][s] (+ shared partials).  The
// (slot j, slice s) pairs are numbered slot-major; thread (slice lane sl,
// column quad cq) accumulates pairs sl, sl + 64, ... in that fixed order (the
// slots' units and weights are read once into LDS, so the partial loads of
// consecutive pairs are independent and overlap); the 64 slice lanes are then
// added by a fixed LDS tree and the result is rounded once to bf16.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ partial,
                                                            const int32_t* __restrict__ plan,
                                                            const float* __restrict__ topk_w, int T, int d, int E,
                                                            int k, int n_slices, int maxU, int has_shared,
                                                            bf16_t* __restrict__ out) {
  __shared__ float4 red[64][4];
  __shared__ int s_unit[kMaxDecodeSlots];
  __shared__ float s_w[kMaxDecodeSlots];
  const int t = blockIdx.y;
  const int cq = threadIdx.x & 3;
  const int sl = threadIdx.x >> 2;
  const int col = blockIdx.x * 16 + cq * 4;
  const int nunits = k + (has_shared ? 1 : 0);
  for (int j = threadIdx.x; j < nunits; j += 256) {
    if (j < k) {
      s_unit[j] = plan[1 + E + t * k + j];    // -1: dropped by the capacity rule
      s_w[j] = topk_w[t * k + j];
    } else {
      s_unit[j] = maxU;                       // the shared expert, weight 1
      s_w[j] = 1.f;
    }
  }
  __syncthreads();
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int npairs = nunits * n_slices;
  // RB pairs per batch, all loads issued before the first add: pairs past
  // the end and dropped slots load a valid partial (unit 0, or the last
  // pair) and are not added, so no load waits behind a branch
  constexpr int RB = 4;
  for (int i0 = sl; i0 < npairs; i0 += 64 * RB) {
    float4 v[RB];
    float wgt[RB];
    bool live[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int i = i0 + 64 * b;
      const int ic = i < npairs ? i : npairs - 1;
      const int j = ic / n_slices, s = ic - j * n_slices;
      const int unit = s_unit[j];
      live[b] = i < npairs && unit >= 0;
      wgt[b] = s_w[j];
      v[b] = *reinterpret_cast<const float4*>(partial + (((size_t)max(unit, 0) * n_slices + s) * T + t) * d + col);
    }
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      if (!live[b]) continue;
      acc.x = __fmaf_rn(wgt[b], v[b].x, acc.x);
      acc.y = __fmaf_rn(wgt[b], v[b].y, acc.y);
      acc.z = __fmaf_rn(wgt[b], v[b].z, acc.z);
      acc.w = __fmaf_rn(wgt[b], v[b].w, acc.w);
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

// Kernels whose dynamic LDS exceeds the default 64 KB limit need the limit
// raised once per kernel and device; the largest size granted so far is
// remembered, so steady-state calls make no runtime call for it.
static hipError_t allow_dynamic_lds(const void* fn, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, size_t> granted;
  std::lock_guard<std::mutex> lock(mu);
  size_t& have = granted[{fn, dev}];
  if (have >= lds) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) have = lds;
  return e;
}

static int pick_mt(int T) { return T <= 1 ? 1 : T <= 2 ? 2 : T <= 4 ? 4 : 8; }

// Slice width: the widest slice (longest contiguous row segment of W_gate /
// W_up, at most 512 bytes) that still gives every CU at least one work unit.
static int pick_fs(int units, int f, int es) {
  const int cands[3] = {256, 128, 64};
  for (int c : cands) {
    if (f % c) continue;
    if (c * es > 512) continue;
    if (units * (f / c) >= 200) return c;
  }
  return 64;
}

static int decode_max_used(int T, int k, int E) { return (T * k < E) ? T * k : E; }

// Split layout (see the top of the file): chosen when the fused kernel would
// get fewer than 200 work-groups even with 64-column slices.  Phase 1 takes
// the widest slice of at most 512 bytes per row dividing f, and DS <= 32, a
// power of two of d-row parts of at least 64 rows, for at most 1024
// work-groups: three or four per CU, each loading all of its rows at once.
struct DecodeSplit {
  int DS;     // 0: fused kernel
  int FS;     // phase-1 slice width
  int DW;     // phase-2 columns per work-group
};

static DecodeSplit decode_split(int units, int d, int f, int es) {
  DecodeSplit sp{0, 0, 0};
  if (units * (f / 64) >= 200) return sp;
  sp.FS = 64;
  for (int c : {256, 128}) {
    if (f % c == 0 && c * es <= 512) { sp.FS = c; break; }
  }
  const int groups = units * (f / sp.FS);
  sp.DS = 1;
  while (sp.DS * 2 <= kMaxDS && sp.DS * 2 * groups <= 1024 && d % (sp.DS * 16) == 0 && d / (sp.DS * 2) >= 64)
    sp.DS *= 2;                                   // parts stay multiples of 8 rows
  sp.DW = 64;
  for (int c : {512, 256, 128}) {
    if (d % c == 0 && c * es <= 512) { sp.DW = c; break; }
  }
  return sp;
}

size_t decode_partial_bytes(int T, int d, int E, int k, int f, int has_shared, int wkind) {
  const int units = decode_max_used(T, k, E) + (has_shared ? 1 : 0);
  const DecodeSplit sp = decode_split(units, d, f, wkind == W_FP8 ? 1 : 2);
  const size_t partial = (size_t)units * (size_t)(f / 64) * T * d * sizeof(float);
  const size_t gu = (size_t)units * sp.DS * 2 * T * f * sizeof(float);
  return (partial + 255) / 256 * 256 + gu;
}

template <int WK, int MT>
static hipError_t launch_decode_split(const DecodeParams& p, int units, const DecodeSplit& sp, hipStream_t s,
                                      hipEvent_t ev_begin, hipEvent_t ev_end) {
  constexpr int ES = (WK == W_FP8) ? 1 : 2;
  auto phase1 = [&](auto kern, int FS) -> hipError_t {
    const int CH = FS / (16 / ES), RG = 256 / (2 * CH);
    const size_t xs_bytes = (size_t)(p.d / sp.DS) * MT * sizeof(bf16_t);
    const size_t red_bytes = (size_t)(RG * 2 * MT * FS + MT * FS) * sizeof(float);
    const size_t lds = xs_bytes > red_bytes ? xs_bytes : red_bytes;
    if (hipError_t e = allow_dynamic_lds((const void*)kern, lds); e != hipSuccess) return e;
    const dim3 grid(p.f / FS, units, sp.DS);
    if (ev_begin)
      hipExtLaunchKernelGGL(kern, grid, dim3(256), (uint32_t)lds, s, ev_begin, nullptr, 0, p);
    else
      kern<<<grid, 256, lds, s>>>(p);
    return hipGetLastError();
  };
  hipError_t err;
  if (sp.FS == 256) err = phase1(decode_ffn_kernel<WK, MT, 256, true>, 256);
  else if (sp.FS == 128) err = phase1(decode_ffn_kernel<WK, MT, 128, true>, 128);
  else err = phase1(decode_ffn_kernel<WK, MT, 64, true>, 64);
  if (err != hipSuccess) return err;
  auto phase2 = [&](auto kern) -> hipError_t {
    const dim3 grid(p.f / 64, units, p.d / sp.DW);
    if (ev_end)
      hipExtLaunchKernelGGL(kern, grid, dim3(256), 0, s, nullptr, ev_end, 0, p, sp.DS);
    else
      kern<<<grid, 256, 0, s>>>(p, sp.DS);
    return hipGetLastError();
  };
  if (sp.DW == 512) {
    if constexpr (ES == 1) return phase2(decode_down_kernel<WK, MT, 512>);
    return hipErrorInvalidValue;   // 512-column blocks are fp8 only
  }
  if (sp.DW == 256) return phase2(decode_down_kernel<WK, MT, 256>);
  if (sp.DW == 128) return phase2(decode_down_kernel<WK, MT, 128>);
  return phase2(decode_down_kernel<WK, MT, 64>);
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
  if (hipError_t e = allow_dynamic_lds((const void*)decode_ffn_kernel<WK, MT, FS>, lds); e != hipSuccess) return e;
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
static hipError_t launch_decode_mt(const DecodeParams& p, int units, int fs, const DecodeSplit& sp, hipStream_t s,
                                   hipEvent_t b, hipEvent_t e) {
  if (sp.DS) {
    switch (pick_mt(p.T)) {
      case 1: return launch_decode_split<WK, 1>(p, units, sp, s, b, e);
      case 2: return launch_decode_split<WK, 2>(p, units, sp, s, b, e);
      case 4: return launch_decode_split<WK, 4>(p, units, sp, s, b, e);
      default: return launch_decode_split<WK, 8>(p, units, sp, s, b, e);
    }
  }
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
  const int es = a.wkind == W_FP8 ? 1 : 2;
  const DecodeSplit sp = decode_split(units, a.d, a.f, es);
  const size_t partial = (size_t)units * (size_t)(a.f / 64) * a.T * a.d * sizeof(float);
  p.gu = reinterpret_cast<float*>(reinterpret_cast<char*>(a.partial) + (partial + 255) / 256 * 256);
  const int fs = sp.DS ? 64 : pick_fs(units, a.f, es);   // split layers: 64-row W_down slices
  hipError_t err = (a.wkind == W_FP8) ? launch_decode_mt<W_FP8>(p, units, fs, sp, s, a.ev_begin, a.ev_end)
                                      : launch_decode_mt<W_BF16>(p, units, fs, sp, s, a.ev_begin, a.ev_end);
  if (err != hipSuccess) return err;
  dim3 g2(a.d / 16, a.T);
  decode_reduce_kernel<<<g2, 256, 0, s>>>(a.partial, a.plan, a.topk_w, a.T, a.d, a.E, a.k, a.f / fs, p.maxU,
                                          a.has_shared, (bf16_t*)a.out);
  return hipGetLastError();
}

}  // namespace moe
