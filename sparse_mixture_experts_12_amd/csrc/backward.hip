// Backward of the token-choice layer on gfx950: everything around the grouped
// GEMMs of bwd_gemm.hip.
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
// Every sum runs in a fixed order: the result is bitwise reproducible.
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

// Xp[p] = x[ptok[p]], Dp[p] = dout[ptok[p]] (zero rows for padding); 8 bf16 per thread.
__global__ __launch_bounds__(256) void gather_rows_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ dout,
                                                          const int32_t* __restrict__ ptok, int pmax, int d,
                                                          bf16_t* __restrict__ Xp, bf16_t* __restrict__ Dp) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const int per_row = d / 8;
  const long p = i / per_row;
  if (p >= pmax) return;
  const int c = (int)(i - p * per_row) * 8;
  const int t = ptok[p];
  u32x4_t vx = {0u, 0u, 0u, 0u}, vd = {0u, 0u, 0u, 0u};
  if (t >= 0) {
    vx = *reinterpret_cast<const u32x4_t*>(x + (size_t)t * d + c);
    vd = *reinterpret_cast<const u32x4_t*>(dout + (size_t)t * d + c);
  }
  *reinterpret_cast<u32x4_t*>(Xp + (size_t)p * d + c) = vx;
  *reinterpret_cast<u32x4_t*>(Dp + (size_t)p * d + c) = vd;
}

// One work-group per padded row: SwiGLU backward and the row's slot gradient
//   H = bf16(silu(G) U) (the forward's rounding), gsc = dH' . H,
//   dG = w dH' U silu'(G), dU = w dH' silu(G), Hw = bf16(w H)   (bf16 out)
// The dot product: each thread sums its columns in order, then a fixed tree.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ G, const float* __restrict__ U,
                                                         const float* __restrict__ dH, const float* __restrict__ pw,
                                                         const int32_t* __restrict__ pend, int f,
                                                         bf16_t* __restrict__ dG, bf16_t* __restrict__ dU,
                                                         bf16_t* __restrict__ Hw, float* __restrict__ gsc) {
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
    float og[4], ou[4], oh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g = g4[i], u = u4[i], dh = d4[i];
      const float s = 1.f / (1.f + __expf(-g));
      const float si = g * s;
      const float h = bf16_to_f32(f32_to_bf16(si * u));
      part = __fmaf_rn(dh, h, part);
      og[i] = w * dh * u * (s * (1.f + g * (1.f - s)));
      ou[i] = w * dh * si;
      oh[i] = w * h;
    }
    uint2 vg, vu, vh;
    vg.x = pack_bf16x2(og[0], og[1]); vg.y = pack_bf16x2(og[2], og[3]);
    vu.x = pack_bf16x2(ou[0], ou[1]); vu.y = pack_bf16x2(ou[2], ou[3]);
    vh.x = pack_bf16x2(oh[0], oh[1]); vh.y = pack_bf16x2(oh[2], oh[3]);
    *reinterpret_cast<uint2*>(dG + base + c) = vg;
    *reinterpret_cast<uint2*>(dU + base + c) = vu;
    *reinterpret_cast<uint2*>(Hw + base + c) = vh;
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

// dx[t, c] = sum_j [kept] dXp[apos[t k + j], c] + dXp[shared row of t, c]
//            + sum_e dl[t, e] W_g[c, e]       (fp32, in this order)
template <bool SPARSE>
__global__ __launch_bounds__(256) void dx_kernel(const float* __restrict__ dXp, const int32_t* __restrict__ apos,
                                                 const int32_t* __restrict__ poff, const float* __restrict__ dl,
                                                 const int32_t* __restrict__ topk_idx, const bf16_t* __restrict__ Wg,
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
      r = __fmaf_rn(dl[(size_t)t * E + e], bf16_to_f32(Wg[(size_t)c * E + e]), r);
    }
  } else {
    for (int e = 0; e < E; ++e) r = __fmaf_rn(dl[(size_t)t * E + e], bf16_to_f32(Wg[(size_t)c * E + e]), r);
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

__global__ __launch_bounds__(256) void router_wgrad_partial_kernel(const bf16_t* __restrict__ x,
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
    uint2 xr[U];
    float4 lr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {             // clamped tokens: every load unconditional
      const int t = min(tb + u, t1 - 1);
      xr[u] = bias_row ? make_uint2(0x3f80u, 0u) : *reinterpret_cast<const uint2*>(x + (size_t)t * d + c);
      const float* r = dl + (size_t)t * E + e;
      lr[u] = vec ? *reinterpret_cast<const float4*>(r)
                  : make_float4(r[0], ne > 1 ? r[1] : 0.f, ne > 2 ? r[2] : 0.f, ne > 3 ? r[3] : 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tb + u >= t1) break;
      const float xv[4] = {bf16lo(xr[u].x), bf16hi(xr[u].x), bf16lo(xr[u].y), bf16hi(xr[u].y)};
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

long backward_pad_rows(int T, int E, int k, int has_shared) {
  const long routed = (long)T * k + (long)(kPadRows - 1) * E;
  const long shared = has_shared ? ((long)T + kPadRows - 1) / kPadRows * kPadRows : 0;
  return (routed + shared + 63) / 64 * 64;
}

size_t backward_sched_ints(int T, int E, int k, int has_shared) {
  const int G = E + (has_shared ? 1 : 0);
  const long pmax = backward_pad_rows(T, E, k, has_shared);
  return kSchedHead + 4 * (size_t)grouped_max_row_tiles((int)pmax, 0, G, 0, 64) + 4 * (size_t)(G + 1) + 16;
}

hipError_t launch_zero(float* p, long n, hipStream_t s) {
  if (!p || n <= 0) return hipSuccess;
  fill_zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  hipError_t err;
  const int G = a.E + (a.has_shared ? 1 : 0);
  const long pmax = backward_pad_rows(a.T, a.E, a.k, a.has_shared);
  pad_offsets_kernel<<<1, 1024, 0, s>>>(a.offsets, a.E, a.has_shared ? a.T : 0, a.poff);
  const long npr = pmax > (long)a.T * a.k ? pmax : (long)a.T * a.k;
  pad_rows_kernel<<<(unsigned)((npr + 255) / 256), 256, 0, s>>>(a.poff, a.offsets, a.sorted_assign, a.inv_perm,
                                                                 a.topk_idx, a.topk_w, a.E, G, a.k, a.T, (int)pmax,
                                                                 a.ptok, a.pw, a.apos);
  gather_rows_kernel<<<(unsigned)((pmax * (a.d / 8) + 255) / 256), 256, 0, s>>>(
      (const bf16_t*)a.x, (const bf16_t*)a.dout, a.ptok, (int)pmax, a.d, a.Xp, a.Dp);
  if ((err = hipGetLastError()) != hipSuccess) return err;

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
  // 3. SwiGLU backward per padded row
  swiglu_bwd_kernel<<<(unsigned)pmax, 256, 0, s>>>(a.G, a.U, a.dH, a.pw, a.poff + G, a.f, a.dG, a.dU, a.Hw, a.gsc);
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
    if (a.ev_begin) hipEventRecord(a.ev_begin, s);
    if ((err = launch_bwd_rows(2, q, s)) != hipSuccess) return err;
    if (a.ev_end) hipEventRecord(a.ev_end, s);
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
  // 6. router: dL/dlogits, then dx, dW_g, d_bias
  router_bwd_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a.logits, a.topk_idx, a.topk_w, a.apos, a.gsc, a.T, a.E, a.k,
                                                  a.renormalize, a.dl);
  const dim3 gx((a.d + 255) / 256, a.T);
  if (a.renormalize)
    dx_kernel<true><<<gx, 256, 0, s>>>(a.dXp, a.apos, a.poff, a.dl, a.topk_idx, (const bf16_t*)a.W_g, a.T, a.d, a.E,
                                       a.k, a.has_shared, a.dx);
  else
    dx_kernel<false><<<gx, 256, 0, s>>>(a.dXp, a.apos, a.poff, a.dl, a.topk_idx, (const bf16_t*)a.W_g, a.T, a.d,
                                        a.E, a.k, a.has_shared, a.dx);
  const int nchunk = (a.T + kRwChunk - 1) / kRwChunk;
  router_wgrad_partial_kernel<<<dim3((a.d + 1 + 255) / 256, (a.E + 15) / 16, nchunk), 256, 0, s>>>(
      (const bf16_t*)a.x, a.dl, a.T, a.d, a.E, a.rw_part);
  const long nout = (long)(a.d + 1) * a.E;
  router_wgrad_reduce_kernel<<<(unsigned)((nout + 255) / 256), 256, 0, s>>>(a.rw_part, nchunk, a.d, a.E, a.dW_g,
                                                                           a.d_bias);
  return hipGetLastError();
}

}  // namespace moe
