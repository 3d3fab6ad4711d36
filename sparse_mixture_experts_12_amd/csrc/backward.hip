// Backward of the layer on gfx950: everything around the grouped GEMMs of
// bwd_gemm.hip, for token-choice and expert-choice routing and every layer
// dtype the forward takes.
//
// Pages: "MoE Model Architectures", Mixtral "Sparse MoE Block" (softmax, top-k,
// divide by the top-k sum, weighted sum of the chosen experts: the forward
// these are the derivatives of) and DeepSeek-V3 "DeepSeekMoE Architecture"
// (the shared expert, weight 1); "Testing using claude to graft ETHOS onto
// modded-nanogpt base", "Key Implementation Details" (recompute the forward
// values in the backward; gradients of each expert's weights summed over its
// tokens -- here without atomics); "Faster writing: run only the chosen
// experts; uncap the large profile", "Test plan" (slot gradients of the
// chosen-experts dispatch equal those of running every expert).
//
// With the selection (top-k, capacity) held fixed, for dout = dL/dout:
//   y_r = FFN_e(x_t) of a kept assignment r = (t, j); g_tj = dout_t . y_r
//       = (dout_t W_down^T) . H_r, so no forward down projection is needed
//   dH'_r = dout_t W_down[e]^T;  dG = w_tj dH' * U * silu'(G);  dU = w_tj dH' * silu(G)
//   dW_gate[e] = sum_r x_t^T dG_r, dW_up likewise, dW_down[e] = sum_r (w_tj H_r)^T dout_t
//   dl_t (router): renormalised -> dl_(e_j) = w_j (g_j - sum_i g_i w_i), zero elsewhere;
//                  else         -> dl_e = p_e ([e chosen] g(e) - sum_j g_j p_(e_j))
//   dx_t = sum_j [kept] (dG_r W_gate^T + dU_r W_up^T) + (shared expert's) + dl_t W_g^T
//   dW_g = x^T dl, d_bias = sum_t dl_t
// Expert-choice layers ("MoE Model Architectures", Design Patterns, Pattern 3)
// differ only in where the rows come from: expert e's C rows are the tokens it
// took, a token's slots are the experts that took it (0 to E of them, listed
// in ascending expert order), and the same two router formulas apply over
// that list (renormalised: a softmax over the experts that took the token;
// else the full softmax).
// Weight dtypes: fp8 layers differentiate with respect to the weights' values
// (code x channel scale), MXFP8 / MXFP4 layers likewise, with the forward's
// MXFP8 quantisation of x and H recomputed and passed straight through; both
// run the bf16 GEMMs on a bf16 copy of the values written first.  fp32 layers
// keep every intermediate in fp32 and use the SIMT fp32 GEMMs.
// Every sum runs in a fixed order: the result is bitwise reproducible.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPadRows = 64;   // group row counts are padded to this

// ---------------------------------------------------------------------------
// Padded row space: group g (expert g; the shared expert is group E) owns rows
// [poff[g], poff[g + 1]), its row count rounded up to a multiple of 64.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E, int shared_T,
                                                           int32_t* __restrict__ poff) {
  __shared__ int buf[1024];
  const int tid = threadIdx.x;
  const int G = E + (shared_T > 0 ? 1 : 0);
  int c = 0;
  if (tid < E) c = offsets[tid + 1] - offsets[tid];
  else if (tid == E && shared_T > 0) c = shared_T;
  int v = (tid < G) ? (c + kPadRows - 1) / kPadRows * kPadRows : 0;
  for (int off = 1; off < 1024; off <<= 1) {      // inclusive scan (Hillis-Steele)
    buf[tid] = v;
    __syncthreads();
    if (tid >= off) v += buf[tid - off];
    __syncthreads();
  }
  if (tid < G) poff[tid + 1] = v;
  if (tid == 0) poff[0] = 0;
}

// Per padded row p < pmax: the token whose rows it holds (-1: padding) and its
// combine weight; per assignment a < T k: its padded row (-1: dropped).
__global__ __launch_bounds__(256) void pad_rows_kernel(const int32_t* __restrict__ poff,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ sorted_assign,
                                                       const int32_t* __restrict__ inv_perm,
                                                       const int32_t* __restrict__ topk_idx,
                                                       const float* __restrict__ topk_w, int E, int G, int k, int T,
                                                       int pmax, int32_t* __restrict__ ptok, float* __restrict__ pw,
                                                       int32_t* __restrict__ apos) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p < T * k) {
    const int r = inv_perm[p];
    const int e = topk_idx[p];
    apos[p] = r < 0 ? -1 : poff[e] + (r - offsets[e]);
  }
  if (p >= pmax) return;
  int tok = -1;
  float wt = 0.f;
  if (p < poff[G]) {
    int lo = 0, hi = G;                             // largest g with poff[g] <= p
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (poff[mid] <= p) lo = mid;
      else hi = mid;
    }
    const int local = p - poff[lo];
    if (lo < E) {
      if (local < offsets[lo + 1] - offsets[lo]) {
        const int a = sorted_assign[offsets[lo] + local];
        tok = a / k;
        wt = topk_w[a];
      }
    } else if (local < T) {
      tok = local;
      wt = 1.f;
    }
  }
  ptok[p] = tok;
  pw[p] = wt;
}

// Expert choice: per padded row its token (the expert's row r holds token
// sorted_tokens[r]) and the token's combine weight for that expert (its list
// entry for row r); per token list entry i < ccount[t] (rows crow[t E + i],
// expert crow / C) its padded row, -1 past the list.
__global__ __launch_bounds__(256) void pad_rows_ec_kernel(const int32_t* __restrict__ poff,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted_tokens,
                                                          const int32_t* __restrict__ crow,
                                                          const float* __restrict__ cw,
                                                          const int32_t* __restrict__ ccount, int C, int E, int G,
                                                          int T, int pmax, int32_t* __restrict__ ptok,
                                                          float* __restrict__ pw, int32_t* __restrict__ apos) {
  const long p = (long)blockIdx.x * 256 + threadIdx.x;
  if (p < (long)T * E) {
    const int t = (int)(p / E), i = (int)(p - (long)t * E);
    int v = -1;
    if (i < ccount[t]) {
      const int r = crow[p];
      const int e = r / C;
      v = poff[e] + (r - e * C);
    }
    apos[p] = v;
  }
  if (p >= pmax) return;
  int tok = -1;
  float wt = 0.f;
  if (p < poff[G]) {
    int lo = 0, hi = G;                             // largest g with poff[g] <= p
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (poff[mid] <= p) lo = mid;
      else hi = mid;
    }
    const int local = (int)p - poff[lo];
    if (lo < E) {
      if (local < offsets[lo + 1] - offsets[lo]) {
        const int r = offsets[lo] + local;
        tok = sorted_tokens[r];
        const int n = ccount[tok];
        const size_t b = (size_t)tok * E;
        for (int i = 0; i < n; ++i)
          if (crow[b + i] == r) wt = cw[b + i];
      }
    } else if (local < T) {
      tok = local;
      wt = 1.f;
    }
  }
  ptok[p] = tok;
  pw[p] = wt;
}

// Xp[p] = x[ptok[p]], Dp[p] = dout[ptok[p]] (zero rows for padding); one
// 16-byte chunk per thread (8 bf16 or 4 fp32 values); row_bytes = d * element size.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ dout,
                                                          const int32_t* __restrict__ ptok, int pmax, int row_bytes,
                                                          uint8_t* __restrict__ Xp, uint8_t* __restrict__ Dp) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = row_bytes / 16;
  const long p = i / per_row;
  if (p >= pmax) return;
  const int c = (int)(i - p * per_row) * 16;
  const int t = ptok[p];
  u32x4_t vx = {0u, 0u, 0u, 0u}, vd = {0u, 0u, 0u, 0u};
  if (t >= 0) {
    vx = *reinterpret_cast<const u32x4_t*>(x + (size_t)t * row_bytes + c);
    vd = *reinterpret_cast<const u32x4_t*>(dout + (size_t)t * row_bytes + c);
  }
  *reinterpret_cast<u32x4_t*>(Xp + (size_t)p * row_bytes + c) = vx;
  *reinterpret_cast<u32x4_t*>(Dp + (size_t)p * row_bytes + c) = vd;
}

// One work-group per padded row: SwiGLU backward and the row's slot gradient
//   H = silu(G) U (rounded to bf16 as the bf16 forward rounds it), gsc = dH' . H,
//   dG = w dH' U silu'(G), dU = w dH' silu(G), Hw = w H   (TO: bf16 or fp32 out)
// The dot product: each thread sums its columns in order, then a fixed tree.
// Block-scaled layers (hq set): the down projection saw H quantised to MXFP8
// (codes hq [P, f], scales hs [P, f / 32]), so gsc and Hw take those values;
// dG and dU pass through the quantisation unchanged (straight through).
template <typename TO>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ G, const float* __restrict__ U,
                                                         const float* __restrict__ dH, const float* __restrict__ pw,
                                                         const int32_t* __restrict__ pend, int f,
                                                         TO* __restrict__ dG, TO* __restrict__ dU,
                                                         TO* __restrict__ Hw, float* __restrict__ gsc,
                                                         const uint8_t* __restrict__ hq = nullptr,
                                                         const uint8_t* __restrict__ hs = nullptr) {
  constexpr bool BF = !std::is_same<TO, float>::value;
  __shared__ float red[256];
  const size_t p = blockIdx.x;
  if ((int)p >= *pend) return;                    // past the last group: never read
  const float w = pw[p];
  const size_t base = p * (size_t)f;
  float part = 0.f;
  for (int c = threadIdx.x * 4; c < f; c += 1024) {
    const f32x4_t g4 = *reinterpret_cast<const f32x4_t*>(G + base + c);
    const f32x4_t u4 = *reinterpret_cast<const f32x4_t*>(U + base + c);
    const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(dH + base + c);
    float hqv[4] = {0.f, 0.f, 0.f, 0.f};
    if (hq) {                                     // 4 codes of one 32-column block
      fp8x4_to_f32(*reinterpret_cast<const uint32_t*>(hq + base + c), hqv);
      const int e = (int)hs[p * (size_t)(f >> 5) + (c >> 5)] - 127;
#pragma unroll
      for (int i = 0; i < 4; ++i) hqv[i] = ldexpf(hqv[i], e);
    }
    float og[4], ou[4], oh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = g4[i], u = u4[i], dh = d4[i];
      const float s = 1.f / (1.f + __expf(-g));
      const float si = g * s;
      const float h = hq ? hqv[i] : BF ? bf16_to_f32(f32_to_bf16(si * u)) : si * u;
      part = __fmaf_rn(dh, h, part);
      og[i] = w * dh * u * (s * (1.f + g * (1.f - s)));
      ou[i] = w * dh * si;
      oh[i] = w * h;
    }
    if constexpr (BF) {
      uint2 vg, vu, vh;
      vg.x = pack_bf16x2(og[0], og[1]); vg.y = pack_bf16x2(og[2], og[3]);
      vu.x = pack_bf16x2(ou[0], ou[1]); vu.y = pack_bf16x2(ou[2], ou[3]);
      vh.x = pack_bf16x2(oh[0], oh[1]); vh.y = pack_bf16x2(oh[2], oh[3]);
      *reinterpret_cast<uint2*>(dG + base + c) = vg;
      *reinterpret_cast<uint2*>(dU + base + c) = vu;
      *reinterpret_cast<uint2*>(Hw + base + c) = vh;
    } else {
      *reinterpret_cast<f32x4_t*>(dG + base + c) = f32x4_t{og[0], og[1], og[2], og[3]};
      *reinterpret_cast<f32x4_t*>(dU + base + c) = f32x4_t{ou[0], ou[1], ou[2], ou[3]};
      *reinterpret_cast<f32x4_t*>(Hw + base + c) = f32x4_t{oh[0], oh[1], oh[2], oh[3]};
    }
  }
  red[threadIdx.x] = part;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) gsc[p] = red[0];
}

// One wave per token: dL/dlogits from the slot gradients (see the file comment).
__global__ __launch_bounds__(256) void router_bwd_kernel(const float* __restrict__ logits,
                                                         const int32_t* __restrict__ topk_idx,
                                                         const float* __restrict__ topk_w,
                                                         const int32_t* __restrict__ apos,
                                                         const float* __restrict__ gsc, int T, int E, int k,
                                                         int renorm, float* __restrict__ dl) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  // slot j lives in lane j (k <= 32)
  int ej = -1;
  float gj = 0.f, wj = 0.f;
  if (lane < k) {
    const int a = t * k + lane;
    ej = topk_idx[a];
    wj = topk_w[a];
    const int pp = apos[a];
    gj = pp >= 0 ? gsc[pp] : 0.f;                 // dropped assignments: no gradient
  }
  const float* l = logits + (size_t)t * E;
  if (renorm) {
    float s = gj * wj;
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    s = __shfl(s, 0);
    for (int e = lane; e < E; e += 64) {
      float v = 0.f;
      for (int j = 0; j < k; ++j) {               // the slot (if any) that chose e
        const int ex = __shfl(ej, j);
        const float wx = __shfl(wj, j), gx = __shfl(gj, j);
        if (ex == e) v = wx * (gx - s);
      }
      dl[(size_t)t * E + e] = v;
    }
    return;
  }
  // full softmax p (fp64 inside, as the router computes it)
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, l[e]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  double z = 0.0;
  for (int e = lane; e < E; e += 64) z += exp((double)l[e] - (double)m);
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  z = __shfl(z, 0);
  const float pj = lane < k ? (float)(exp((double)l[ej] - (double)m) / z) : 0.f;
  float s = gj * pj;
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  s = __shfl(s, 0);
  for (int e = lane; e < E; e += 64) {
    const float pe = (float)(exp((double)l[e] - (double)m) / z);
    float ge = 0.f;
    for (int j = 0; j < k; ++j) {                 // the slot (if any) that chose e
      const int ex = __shfl(ej, j);
      const float gx = __shfl(gj, j);
      if (ex == e) ge = gx;
    }
    dl[(size_t)t * E + e] = pe * (ge - s);
  }
}

// Expert choice, one wave per token: s = sum over the token's list (ascending
// experts) of g w, then for every expert e
//   renormalised: dl_e = w_e (g_e - s) if e took the token, else 0
//   otherwise:    dl_e = p_e (g_e - s) with g_e = 0 if e did not take it
// (w_e, the forward's combine weight, is the padded row's pw; p_e the score).
__global__ __launch_bounds__(256) void router_bwd_ec_kernel(const float* __restrict__ scores,
                                                            const int32_t* __restrict__ pos,
                                                            const int32_t* __restrict__ crow,
                                                            const int32_t* __restrict__ ccount,
                                                            const int32_t* __restrict__ poff,
                                                            const float* __restrict__ gsc,
                                                            const float* __restrict__ pw, int T, int E, int C,
                                                            int renorm, float* __restrict__ dl) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const size_t b = (size_t)t * E;
  const int n = ccount[t];
  float s = 0.f;
  for (int i = lane; i < n; i += 64) {
    const int r = crow[b + i];
    const int e = r / C;
    const int pp = poff[e] + (r - e * C);
    s += gsc[pp] * pw[pp];
  }
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  s = __shfl(s, 0);
  for (int e = lane; e < E; e += 64) {
    const int r = pos[b + e];
    float g = 0.f, w = 0.f;
    if (r >= 0) {
      const int pp = poff[e] + (r - e * C);
      g = gsc[pp];
      w = pw[pp];
    }
    float v;
    if (renorm) v = r >= 0 ? w * (g - s) : 0.f;
    else v = scores[(size_t)e * T + t] * (g - s);
    dl[b + e] = v;
  }
}

// Expert choice: dx[t, c] = sum over the token's list of dXp[its padded row, c]
//   + dXp[shared row of t, c] + sum_e dl[t, e] W_g[c, e]   (fp32, in this order;
// renormalised: dl is zero off the token's list, so only the list is summed)
template <bool SPARSE, typename TW>
__global__ __launch_bounds__(256) void dx_ec_kernel(const float* __restrict__ dXp, const int32_t* __restrict__ apos,
                                                    const int32_t* __restrict__ poff, const float* __restrict__ dl,
                                                    const int32_t* __restrict__ crow,
                                                    const int32_t* __restrict__ ccount, int C,
                                                    const TW* __restrict__ Wg, int T, int d, int E,
                                                    int has_shared, float* __restrict__ dx) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  const size_t b = (size_t)t * E;
  const int n = ccount[t];
  float acc = 0.f;
  for (int i = 0; i < n; ++i) acc += dXp[(size_t)apos[b + i] * d + c];
  if (has_shared) acc += dXp[(size_t)(poff[E] + t) * d + c];
  float r = 0.f;
  if (SPARSE) {
    for (int i = 0; i < n; ++i) {
      const int e = crow[b + i] / C;
      r = __fmaf_rn(dl[b + e], ActTraits<TW>::load(Wg, (size_t)c * E + e), r);
    }
  } else {
    for (int e = 0; e < E; ++e) r = __fmaf_rn(dl[b + e], ActTraits<TW>::load(Wg, (size_t)c * E + e), r);
  }
  dx[(size_t)t * d + c] = acc + r;
}

// dx[t, c] = sum_j [kept] dXp[apos[t k + j], c] + dXp[shared row of t, c]
//            + sum_e dl[t, e] W_g[c, e]       (fp32, in this order)
template <bool SPARSE, typename TW>
__global__ __launch_bounds__(256) void dx_kernel(const float* __restrict__ dXp, const int32_t* __restrict__ apos,
                                                 const int32_t* __restrict__ poff, const float* __restrict__ dl,
                                                 const int32_t* __restrict__ topk_idx, const TW* __restrict__ Wg,
                                                 int T, int d, int E, int k, int has_shared, float* __restrict__ dx) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= d) return;
  float acc = 0.f;
  for (int j = 0; j < k; ++j) {
    const int pp = apos[t * k + j];
    if (pp >= 0) acc += dXp[(size_t)pp * d + c];
  }
  if (has_shared) acc += dXp[(size_t)(poff[E] + t) * d + c];
  float r = 0.f;
  if (SPARSE) {                                   // renormalised: dl is zero off the chosen experts
    for (int j = 0; j < k; ++j) {
      const int e = topk_idx[t * k + j];
      r = __fmaf_rn(dl[(size_t)t * E + e], ActTraits<TW>::load(Wg, (size_t)c * E + e), r);
    }
  } else {
    for (int e = 0; e < E; ++e) r = __fmaf_rn(dl[(size_t)t * E + e], ActTraits<TW>::load(Wg, (size_t)c * E + e), r);
  }
  dx[(size_t)t * d + c] = acc + r;
}

// dW_g[c, e] = sum_t x[t, c] dl[t, e] and d_bias[e] = sum_t dl[t, e] (row
// c = d of the partials, x taken as 1): tokens in chunks of kRwChunk; a
// work-group covers 256 c x 16 e of one chunk, a thread 4 consecutive c x 4
// consecutive e, with the loads of 8 tokens in flight before their FMAs (each
// sum still runs over the chunk's tokens in order); a second launch adds the
// chunks in order.
constexpr int kRwChunk = 256;

template <typename TX>
__global__ __launch_bounds__(256) void router_wgrad_partial_kernel(const TX* __restrict__ x,
                                                                   const float* __restrict__ dl, int T, int d, int E,
                                                                   float* __restrict__ part) {
  const int c = blockIdx.x * 256 + 4 * (threadIdx.x & 63);     // d % 4 == 0: a 4-block is all x or the bias row
  const int e = blockIdx.y * 16 + 4 * (threadIdx.x >> 6);
  if (c > d || e >= E) return;
  const int t0 = blockIdx.z * kRwChunk;
  const int t1 = min(T, t0 + kRwChunk);
  const bool bias_row = c == d;
  const int ne = min(4, E - e);
  const bool vec = ne == 4 && (E & 3) == 0;     // 16-byte aligned dl rows and partial rows
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
  constexpr int U = 8;
  for (int tb = t0; tb < t1; tb += U) {
    f32x4_t xr[U];
    float4 lr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {             // clamped tokens: every load unconditional
      const int t = min(tb + u, t1 - 1);
      if (bias_row) {
        xr[u] = f32x4_t{1.f, 0.f, 0.f, 0.f};
      } else if constexpr (std::is_same<TX, float>::value) {
        xr[u] = *reinterpret_cast<const f32x4_t*>(x + (size_t)t * d + c);
      } else {
        const uint2 q = *reinterpret_cast<const uint2*>(x + (size_t)t * d + c);
        xr[u] = f32x4_t{bf16lo(q.x), bf16hi(q.x), bf16lo(q.y), bf16hi(q.y)};
      }
      const float* r = dl + (size_t)t * E + e;
      lr[u] = vec ? *reinterpret_cast<const float4*>(r)
                  : make_float4(r[0], ne > 1 ? r[1] : 0.f, ne > 2 ? r[2] : 0.f, ne > 3 ? r[3] : 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tb + u >= t1) break;
      const float xv[4] = {xr[u][0], xr[u][1], xr[u][2], xr[u][3]};
      const float lv[4] = {lr[u].x, lr[u].y, lr[u].z, lr[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __fmaf_rn(xv[i], lv[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (c + i > d) break;
    float* o = part + ((size_t)blockIdx.z * (d + 1) + c + i) * E + e;
    if (vec) *reinterpret_cast<float4*>(o) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    else
      for (int j = 0; j < ne; ++j) o[j] = acc[i][j];
  }
}

__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(const float* __restrict__ part, int nchunk, int d,
                                                                  int E, float* __restrict__ dWg,
                                                                  float* __restrict__ db) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long n = (long)(d + 1) * E;
  if (i >= n) return;
  float s = 0.f;
  for (int z = 0; z < nchunk; ++z) s += part[(size_t)z * n + i];
  if (i < (long)d * E) dWg[i] = s;
  else if (db) db[i - (long)d * E] = s;
}

size_t router_wgrad_ws_bytes(int T, int d, int E) {
  const size_t nchunk = (T + kRwChunk - 1) / kRwChunk;
  return nchunk * (size_t)(d + 1) * E * 4;
}

// fp8 layers: out[m, r, c] = bf16(e4m3(codes[m, r, c]) * scale[m, c]) for
// n_mats matrices of R x C (the scale is per output channel, the column), so
// the bf16 GEMMs below run on the weights' values; 8 codes per thread.
__global__ __launch_bounds__(256) void dequant_fp8_kernel(const uint8_t* __restrict__ codes,
                                                          const float* __restrict__ scale, long n8, int R, int C,
                                                          bf16_t* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const long e0 = i * 8;
  const long per_mat = (long)R * C;
  const long m = e0 / per_mat;
  const int c = (int)(e0 % C);
  const uint2 w = *reinterpret_cast<const uint2*>(codes + e0);
  const float* s = scale + m * C + c;
  float v[8];
  fp8x4_to_f32(w.x, v);
  fp8x4_to_f32(w.y, v + 4);
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(v[2 * j] * s[2 * j], v[2 * j + 1] * s[2 * j + 1]);
  *reinterpret_cast<u32x4_t*>(out + e0) = o;
}

hipError_t launch_dequant_fp8(const void* codes, const float* scale, long n_mats, int R, int C, bf16_t* out,
                              hipStream_t s) {
  const long n8 = n_mats * R * (long)C / 8;
  if (n8 <= 0) return hipSuccess;
  dequant_fp8_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>((const uint8_t*)codes, scale, n8, R, C, out);
  return hipGetLastError();
}

// Block-scaled layers: H = silu(G) U in fp32 (as the forward's gate/up
// epilogue forms it before quantising), 4 values per thread.
__global__ __launch_bounds__(256) void swiglu_h_kernel(const float* __restrict__ G, const float* __restrict__ U,
                                                       long n4, float* __restrict__ H) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4_t g = reinterpret_cast<const f32x4_t*>(G)[i];
  const f32x4_t u = reinterpret_cast<const f32x4_t*>(U)[i];
  f32x4_t h;
#pragma unroll
  for (int j = 0; j < 4; ++j) h[j] = g[j] / (1.f + __expf(-g[j])) * u[j];
  reinterpret_cast<f32x4_t*>(H)[i] = h;
}

// MXFP8 rows -> bf16 values (code x 2^(scale - 127)), same layout; 8 per thread.
__global__ __launch_bounds__(256) void dequant_mx_rows_kernel(const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales, long n8,
                                                              bf16_t* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint2 w = reinterpret_cast<const uint2*>(codes)[i];
  const int e = (int)scales[i >> 2] - 127;        // 8 values = a quarter of a 32-value block
  float v[8];
  fp8x4_to_f32(w.x, v);
  fp8x4_to_f32(w.y, v + 4);
  u32x4_t o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(ldexpf(v[2 * j], e), ldexpf(v[2 * j + 1], e));
  reinterpret_cast<u32x4_t*>(out)[i] = o;
}

// E2M1 code (sign, 2 exponent bits with bias 1, 1 mantissa bit) -> value.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t m = c & 7u;
  const float mag = m < 2 ? 0.5f * (float)m : ldexpf(1.f + 0.5f * (float)(m & 1u), (int)(m >> 1) - 1);
  return (c & 8u) ? -mag : mag;
}

// Block-scaled weights -> the bf16 backward's input-major layout: codes
// [mats, N, K] (K contiguous; E2M1: two per byte, element 2j in the low
// nibble) with E8M0 scales [mats, N, K / 32] become out[m, k, n] = value.
// One 64 (N) x 64 (K) tile per work-group, transposed through LDS.
template <bool W4>
__global__ __launch_bounds__(256) void dequant_mx_transpose_kernel(const uint8_t* __restrict__ codes,
                                                                   const uint8_t* __restrict__ scales, int N, int K,
                                                                   bf16_t* __restrict__ out) {
  __shared__ float tile[64][65];
  const int k0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const size_t m = blockIdx.z;
  const int tid = threadIdx.x;
  {                                               // row n0 + tid / 4, K values k0 + 16 (tid % 4) .. + 15
    const int n = tid >> 2, kc = 16 * (tid & 3);
    const size_t row = m * N + n0 + n;
    const int e = (int)scales[row * (size_t)(K >> 5) + ((k0 + kc) >> 5)] - 127;
    float v[16];
    if constexpr (W4) {
      const uint2 w = *reinterpret_cast<const uint2*>(codes + row * (size_t)(K >> 1) + ((k0 + kc) >> 1));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t b = ((j < 4 ? w.x : w.y) >> (8 * (j & 3))) & 0xffu;
        v[2 * j] = e2m1_value(b & 15u);
        v[2 * j + 1] = e2m1_value(b >> 4);
      }
    } else {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(codes + row * (size_t)K + k0 + kc);
#pragma unroll
      for (int j = 0; j < 4; ++j) fp8x4_to_f32(w[j], v + 4 * j);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) tile[kc + j][n] = ldexpf(v[j], e);
  }
  __syncthreads();
  {                                               // K row k0 + tid / 4, columns n0 + 16 (tid % 4) .. + 15
    const int k = tid >> 2, nc = 16 * (tid & 3);
    u32x4_t o0, o1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o0[j] = pack_bf16x2(tile[k][nc + 2 * j], tile[k][nc + 2 * j + 1]);
      o1[j] = pack_bf16x2(tile[k][nc + 8 + 2 * j], tile[k][nc + 8 + 2 * j + 1]);
    }
    bf16_t* dst = out + (m * K + k0 + k) * (size_t)N + n0 + nc;
    *reinterpret_cast<u32x4_t*>(dst) = o0;
    *reinterpret_cast<u32x4_t*>(dst + 8) = o1;
  }
}

hipError_t launch_dequant_mx_rows(const uint8_t* codes, const uint8_t* scales, long n, bf16_t* out, hipStream_t s) {
  const long n8 = n / 8;
  if (n8 <= 0) return hipSuccess;
  dequant_mx_rows_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(codes, scales, n8, out);
  return hipGetLastError();
}

hipError_t launch_dequant_mx_transpose(const void* codes, const uint8_t* scales, bool w4, int mats, int N, int K,
                                       bf16_t* out, hipStream_t s) {
  if (mats <= 0) return hipSuccess;
  const dim3 grid(K / 64, N / 64, mats);
  if (w4) dequant_mx_transpose_kernel<true><<<grid, 256, 0, s>>>((const uint8_t*)codes, scales, N, K, out);
  else dequant_mx_transpose_kernel<false><<<grid, 256, 0, s>>>((const uint8_t*)codes, scales, N, K, out);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// The dX GEMM's light row tiles (a group's last <= 128 padded rows) run after
// its heavy ones; when they are few (groups x column tiles <= 256, e.g. 8
// Mixtral experts x 16) each is split into up to 4 K parts, reduced in order.
int backward_dx_ksplit(int d, int f, int G) {
  const int slots = G * ((d + 255) / 256);
  if (slots > 256) return 1;
  for (int ks : {4, 2})
    if ((2 * f) % (ks * 64) == 0) return ks;
  return 1;
}

size_t backward_dx_part_bytes(int d, int f, int G) {
  const int ks = backward_dx_ksplit(d, f, G);
  return (size_t)(ks - 1) * (size_t)G * ((d + 255) / 256) * 128 * 256 * sizeof(float);
}

long backward_pad_rows(long routed, int T, int E, int has_shared) {
  const long padded = routed + (long)(kPadRows - 1) * E;
  const long shared = has_shared ? ((long)T + kPadRows - 1) / kPadRows * kPadRows : 0;
  return (padded + shared + 63) / 64 * 64;
}

size_t backward_sched_ints(long routed, int T, int E, int has_shared) {
  const int G = E + (has_shared ? 1 : 0);
  const long pmax = backward_pad_rows(routed, T, E, has_shared);
  return kSchedHead + 4 * (size_t)grouped_max_row_tiles((int)pmax, 0, G, 0, 64) + 4 * (size_t)(G + 1) + 16;
}

hipError_t launch_zero(float* p, long n, hipStream_t s) {
  if (!p || n <= 0) return hipSuccess;
  fill_zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

static hipError_t backward_gemms_bf16(const BackwardArgs& a, long pmax, int G, hipStream_t s);
static hipError_t backward_gemms_f32(const BackwardArgs& a, long pmax, int G, hipStream_t s);
template <typename TA>
static hipError_t backward_router_t(const BackwardArgs& a, hipStream_t s);
static hipError_t backward_router(const BackwardArgs& a, hipStream_t s) {
  return a.f32 ? backward_router_t<float>(a, s) : backward_router_t<bf16_t>(a, s);
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  hipError_t err;
  const int G = a.E + (a.has_shared ? 1 : 0);
  const bool ec = a.ec_C > 0;
  const long pmax = backward_pad_rows(a.routed, a.T, a.E, a.has_shared);
  pad_offsets_kernel<<<1, 1024, 0, s>>>(a.offsets, a.E, a.has_shared ? a.T : 0, a.poff);
  const long nslot = ec ? (long)a.T * a.E : (long)a.T * a.k;
  const long npr = pmax > nslot ? pmax : nslot;
  if (ec)
    pad_rows_ec_kernel<<<(unsigned)((npr + 255) / 256), 256, 0, s>>>(a.poff, a.offsets, a.sorted_assign, a.ec_crow,
                                                                      a.ec_w, a.ec_count, a.ec_C, a.E, G, a.T,
                                                                      (int)pmax, a.ptok, a.pw, a.apos);
  else
    pad_rows_kernel<<<(unsigned)((npr + 255) / 256), 256, 0, s>>>(a.poff, a.offsets, a.sorted_assign, a.inv_perm,
                                                                   a.topk_idx, a.topk_w, a.E, G, a.k, a.T, (int)pmax,
                                                                   a.ptok, a.pw, a.apos);
  const int row_bytes = a.d * (a.f32 ? 4 : 2);
  gather_rows_kernel<<<(unsigned)((pmax * (row_bytes / 16) + 255) / 256), 256, 0, s>>>(
      (const uint8_t*)(a.x_rows ? a.x_rows : a.x), (const uint8_t*)a.dout, a.ptok, (int)pmax, row_bytes,
      (uint8_t*)a.Xp, (uint8_t*)a.Dp);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (a.f32) {
    if ((err = backward_gemms_f32(a, pmax, G, s)) != hipSuccess) return err;
  } else if ((err = backward_gemms_bf16(a, pmax, G, s)) != hipSuccess) {
    return err;
  }
  return backward_router(a, s);
}

// Steps 1-5 for bf16 layers (fp8 layers arrive here with their weights'
// values already in bf16): the MFMA row-tile and weight-gradient GEMMs.
static hipError_t backward_gemms_bf16(const BackwardArgs& a, long pmax, int G, hipStream_t s) {
  hipError_t err;

  // row tiles of the G padded groups (the shared expert is group E, read from poff like the others)
  const int maxQ = grouped_max_row_tiles((int)pmax, 0, G, 0, 256);
  if ((err = launch_tile_schedule(a.poff, G, 256, 0, 0, maxQ, a.sched, s)) != hipSuccess) return err;

  // 1. recompute G = Xp W_gate, U = Xp W_up (fp32)
  BwdGemmParams p{};
  p.sched = a.sched; p.maxQ = maxQ; p.E = a.E; p.G = G; p.poff = a.poff;
  {
    BwdGemmParams q = p;
    q.A0 = a.Xp; q.lda = a.d;
    q.B0 = (const bf16_t*)a.w.Wg; q.B1 = (const bf16_t*)a.w.Wu;
    q.Bs0 = (const bf16_t*)a.w.Wsg; q.Bs1 = (const bf16_t*)a.w.Wsu;
    q.ldb = a.f; q.bgs = (long)a.d * a.f;
    q.K = a.d; q.K1 = a.d; q.N = a.f;
    q.C0 = a.G; q.C1 = a.U;
    if ((err = launch_bwd_rows(0, q, s)) != hipSuccess) return err;
  }
  // 2. dH' = Dp W_down^T (fp32)
  {
    BwdGemmParams q = p;
    q.A0 = a.Dp; q.lda = a.d;
    q.B0 = (const bf16_t*)a.w.Wd; q.Bs0 = (const bf16_t*)a.w.Wsd;
    q.ldb = a.d; q.bgs = (long)a.f * a.d;
    q.K = a.d; q.K1 = a.d; q.N = a.f;
    q.C0 = a.dH;
    if ((err = launch_bwd_rows(1, q, s)) != hipSuccess) return err;
  }
  // 3. SwiGLU backward per padded row (block-scaled layers: H as the forward
  //    quantised it, MXFP8 per 32 columns of a row)
  if (a.hq) {
    const long n4 = pmax * (long)a.f / 4;
    swiglu_h_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(a.G, a.U, n4, a.Hf);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = launch_mx_quantize(a.Hf, true, pmax, a.f, a.hq, a.hs, s)) != hipSuccess) return err;
  }
  swiglu_bwd_kernel<bf16_t><<<(unsigned)pmax, 256, 0, s>>>(a.G, a.U, a.dH, a.pw, a.poff + G, a.f, a.dG, a.dU, a.Hw,
                                                           a.gsc, a.hq, a.hs);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // 4. dXp = dG W_gate^T + dU W_up^T (fp32)
  {
    BwdGemmParams q = p;
    q.A0 = a.dG; q.A1 = a.dU; q.lda = a.f;
    q.B0 = (const bf16_t*)a.w.Wg; q.B1 = (const bf16_t*)a.w.Wu;
    q.Bs0 = (const bf16_t*)a.w.Wsg; q.Bs1 = (const bf16_t*)a.w.Wsu;
    q.ldb = a.f; q.bgs = (long)a.d * a.f;
    q.K = 2 * a.f; q.K1 = a.f; q.N = a.d;
    q.C0 = a.dXp;
    q.ksplit = backward_dx_ksplit(a.d, a.f, G);
    q.part_slots = G * ((a.d + 255) / 256);
    q.part = a.dx_part;
    if (a.ev_begin && (err = hipEventRecord(a.ev_begin, s)) != hipSuccess) return err;
    if ((err = launch_bwd_rows(2, q, s)) != hipSuccess) return err;
    if (a.ev_end && (err = hipEventRecord(a.ev_end, s)) != hipSuccess) return err;
  }
  // 5. weight gradients: dW_gate = Xp^T dG, dW_up = Xp^T dU ([d, f] per group), dW_down = Hw^T Dp ([f, d])
  {
    BwdGemmParams q = p;
    q.A0 = a.Xp; q.lda = a.d; q.M = a.d;
    q.ldb = a.f; q.N = a.f; q.cstride = (long)a.d * a.f;
    q.B0 = a.dG; q.C0 = a.dW_gate; q.Cs = a.dWs_gate;
    if ((err = launch_bwd_wgrad(q, s)) != hipSuccess) return err;
    q.B0 = a.dU; q.C0 = a.dW_up; q.Cs = a.dWs_up;
    if ((err = launch_bwd_wgrad(q, s)) != hipSuccess) return err;
    BwdGemmParams r = p;
    r.A0 = a.Hw; r.lda = a.f; r.M = a.f;
    r.B0 = a.Dp; r.ldb = a.d; r.N = a.d; r.cstride = (long)a.f * a.d;
    r.C0 = a.dW_down; r.Cs = a.dWs_down;
    if ((err = launch_bwd_wgrad(r, s)) != hipSuccess) return err;
  }
  return hipSuccess;
}

// Steps 1-5 for fp32 layers: the same products with the SIMT fp32 GEMMs, and
// the SwiGLU backward keeping fp32 (no bf16 rounding of H, dG, dU, w H).
static hipError_t backward_gemms_f32(const BackwardArgs& a, long pmax, int G, hipStream_t s) {
  hipError_t err;
  const float* Xp = (const float*)a.Xp;
  const float* Dp = (const float*)a.Dp;
  float* dG = (float*)a.dG;
  float* dU = (float*)a.dU;
  float* Hw = (float*)a.Hw;
  BwdF32Params p{};
  p.poff = a.poff; p.G = G; p.E = a.E;
  // 1. G = Xp W_gate, U = Xp W_up
  {
    BwdF32Params q = p;
    q.A0 = Xp; q.lda = a.d; q.ldb = a.f; q.bgs = (long)a.d * a.f; q.b_kc = false;
    q.K = a.d; q.N = a.f;
    q.B0 = (const float*)a.w.Wg; q.Bs0 = (const float*)a.w.Wsg; q.C = a.G;
    if ((err = launch_bwd_rows_f32(q, pmax, s)) != hipSuccess) return err;
    q.B0 = (const float*)a.w.Wu; q.Bs0 = (const float*)a.w.Wsu; q.C = a.U;
    if ((err = launch_bwd_rows_f32(q, pmax, s)) != hipSuccess) return err;
  }
  // 2. dH' = Dp W_down^T
  {
    BwdF32Params q = p;
    q.A0 = Dp; q.lda = a.d; q.ldb = a.d; q.bgs = (long)a.f * a.d; q.b_kc = true;
    q.K = a.d; q.N = a.f;
    q.B0 = (const float*)a.w.Wd; q.Bs0 = (const float*)a.w.Wsd; q.C = a.dH;
    if ((err = launch_bwd_rows_f32(q, pmax, s)) != hipSuccess) return err;
  }
  // 3. SwiGLU backward per padded row
  swiglu_bwd_kernel<float><<<(unsigned)pmax, 256, 0, s>>>(a.G, a.U, a.dH, a.pw, a.poff + G, a.f, dG, dU, Hw, a.gsc);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // 4. dXp = dG W_gate^T + dU W_up^T
  {
    BwdF32Params q = p;
    q.A0 = dG; q.A1 = dU; q.lda = a.f; q.ldb = a.f; q.bgs = (long)a.d * a.f; q.b_kc = true;
    q.K = 2 * a.f; q.K1 = a.f; q.N = a.d;
    q.B0 = (const float*)a.w.Wg; q.B1 = (const float*)a.w.Wu;
    q.Bs0 = (const float*)a.w.Wsg; q.Bs1 = (const float*)a.w.Wsu;
    q.C = a.dXp;
    if (a.ev_begin && (err = hipEventRecord(a.ev_begin, s)) != hipSuccess) return err;
    if ((err = launch_bwd_rows_f32(q, pmax, s)) != hipSuccess) return err;
    if (a.ev_end && (err = hipEventRecord(a.ev_end, s)) != hipSuccess) return err;
  }
  // 5. weight gradients
  {
    BwdF32Params q = p;
    q.A0 = Xp; q.lda = a.d; q.M = a.d; q.ldb = a.f; q.N = a.f; q.cstride = (long)a.d * a.f;
    q.B0 = dG; q.C = a.dW_gate; q.Cs = a.dWs_gate;
    if ((err = launch_bwd_wgrad_f32(q, s)) != hipSuccess) return err;
    q.B0 = dU; q.C = a.dW_up; q.Cs = a.dWs_up;
    if ((err = launch_bwd_wgrad_f32(q, s)) != hipSuccess) return err;
    BwdF32Params r = p;
    r.A0 = Hw; r.lda = a.f; r.M = a.f; r.B0 = Dp; r.ldb = a.d; r.N = a.d; r.cstride = (long)a.f * a.d;
    r.C = a.dW_down; r.Cs = a.dWs_down;
    if ((err = launch_bwd_wgrad_f32(r, s)) != hipSuccess) return err;
  }
  return hipSuccess;
}

// Step 6: dL/dlogits, then dx, dW_g and d_bias (TA: the activation type).
template <typename TA>
static hipError_t backward_router_t(const BackwardArgs& a, hipStream_t s) {
  const bool ec = a.ec_C > 0;
  const TA* Wg = (const TA*)a.W_g;
  const dim3 gx((a.d + 255) / 256, a.T);
  if (ec) {
    router_bwd_ec_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a.ec_scores, a.ec_pos, a.ec_crow, a.ec_count, a.poff, a.gsc,
                                                       a.pw, a.T, a.E, a.ec_C, a.renormalize, a.dl);
    if (a.renormalize)
      dx_ec_kernel<true, TA><<<gx, 256, 0, s>>>(a.dXp, a.apos, a.poff, a.dl, a.ec_crow, a.ec_count, a.ec_C, Wg, a.T,
                                                a.d, a.E, a.has_shared, a.dx);
    else
      dx_ec_kernel<false, TA><<<gx, 256, 0, s>>>(a.dXp, a.apos, a.poff, a.dl, a.ec_crow, a.ec_count, a.ec_C, Wg, a.T,
                                                 a.d, a.E, a.has_shared, a.dx);
  } else {
    router_bwd_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a.logits, a.topk_idx, a.topk_w, a.apos, a.gsc, a.T, a.E, a.k,
                                                    a.renormalize, a.dl);
    if (a.renormalize)
      dx_kernel<true, TA><<<gx, 256, 0, s>>>(a.dXp, a.apos, a.poff, a.dl, a.topk_idx, Wg, a.T, a.d, a.E, a.k,
                                             a.has_shared, a.dx);
    else
      dx_kernel<false, TA><<<gx, 256, 0, s>>>(a.dXp, a.apos, a.poff, a.dl, a.topk_idx, Wg, a.T, a.d, a.E, a.k,
                                              a.has_shared, a.dx);
  }
  const int nchunk = (a.T + kRwChunk - 1) / kRwChunk;
  router_wgrad_partial_kernel<TA><<<dim3((a.d + 1 + 255) / 256, (a.E + 15) / 16, nchunk), 256, 0, s>>>(
      (const TA*)a.x, a.dl, a.T, a.d, a.E, a.rw_part);
  const long nout = (long)(a.d + 1) * a.E;
  router_wgrad_reduce_kernel<<<(unsigned)((nout + 255) / 256), 256, 0, s>>>(a.rw_part, nchunk, a.d, a.E, a.dW_g,
                                                                           a.d_bias);
  return hipGetLastError();
}

}  // namespace moe
