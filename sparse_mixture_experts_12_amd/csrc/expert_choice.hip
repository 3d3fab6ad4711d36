// Expert-choice routing on gfx950: every expert takes its C best tokens.
//
// Pages: "MoE Model Architectures", Design Patterns, Pattern 3 "Expert Choice
// Routing" (experts select their top tokens instead of tokens selecting
// experts; every expert gets the same number of tokens, a token may be taken
// by several experts); Switch Transformers "Top-1 Routing" (router scores
// are the softmax of the router logits).
//
//   score[t, e] = fp32( exp(l[t, e] - max_e' l[t, e']) / sum_e' exp(...) )   (fp64 inside)
//   expert e takes the C tokens of largest score (equal scores -> lower token),
//   its rows hold them in ascending token order: row = e * C + rank
//   w[t, e] = score[t, e] (/ sum of t's scores over the experts that took it)
//   out[t] = sum over e ascending with (t, e) taken of w[t, e] * y[row(t, e)]
//            (+ the shared expert's row), fp32, one rounding
// Launches: scores (one wave per token), select (one work-group per expert:
// bitonic sort of (score, token) keys in LDS, T <= kEcMaxT), weights (one
// wave per token, which also lists the token's (row, weight) pairs in
// ascending expert order); the expert FFN is the grouped GEMM path with one
// assignment per row; then the combine below walks each token's list.  No
// atomics except one integer count; every floating-point sum has a fixed order.
#include "common.h"
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void ec_scores_kernel(const float* __restrict__ logits, int T, int E,
                                                        float* __restrict__ scores, int32_t* __restrict__ n_unchosen) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_unchosen = 0;     // counted by the weights launch
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, l[e]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  double z = 0.0;
  for (int e = lane; e < E; e += 64) z += exp((double)l[e] - (double)m);
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  z = __shfl(z, 0);                                            // lane 0's fixed-order sum for all
  for (int e = lane; e < E; e += 64) scores[(size_t)e * T + t] = (float)(exp((double)l[e] - (double)m) / z);
}

// One work-group per expert.  Key = (~bits(score)) << 32 | token, so ascending
// keys are descending scores (scores are >= 0) with ties in token order.
__global__ __launch_bounds__(1024) void ec_select_kernel(const float* __restrict__ scores, int T, int E, int C,
                                                        int32_t* __restrict__ pos, int32_t* __restrict__ sorted_tokens,
                                                        int32_t* __restrict__ offsets, int32_t* __restrict__ counts) {
  __shared__ uint64_t key[kEcMaxT];
  __shared__ int32_t flag[kEcMaxT];
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int e = blockIdx.x;
  int N = 1;
  while (N < T) N <<= 1;
  const float* s = scores + (size_t)e * T;
  for (int i = tid; i < N; i += 1024)
    key[i] = i < T ? ((uint64_t)(~__float_as_uint(s[i])) << 32) | (uint32_t)i : ~0ull;
  for (int i = tid; i < T; i += 1024) flag[i] = 0;
  __syncthreads();
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (N >> 1); i += 1024) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = key[lo], b = key[hi];
        if ((a > b) == up) {
          key[lo] = b;
          key[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < C; i += 1024) flag[(int)(key[i] & 0xffffffffu)] = 1;
  __syncthreads();
  // rows in ascending token order: exclusive prefix count of the flags
  const int per = (T + 1023) / 1024;
  const int b0 = tid * per, b1 = min(T, b0 + per);
  int c = 0;
  for (int t = b0; t < b1; ++t) c += flag[t];
  part[tid] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int r = part[tid] - c;
  for (int t = b0; t < b1; ++t) {
    if (flag[t]) {
      const int row = e * C + r++;
      pos[(size_t)t * E + e] = row;
      sorted_tokens[row] = t;
    } else {
      pos[(size_t)t * E + e] = -1;
    }
  }
  if (tid == 0) {
    offsets[e] = e * C;
    if (e == E - 1) offsets[E] = E * C;
    if (counts) counts[e] = C;
  }
}

// One wave per token, lanes over experts (64 at a time, ascending).  The
// token's chosen (row, weight) pairs are compacted in ascending expert order
// for the combine; the renormalising sum adds each lane's experts in order,
// then the lanes in a fixed butterfly (lane 0's value is used by all).
__global__ __launch_bounds__(256) void ec_weights_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ pos, int T, int E, int renorm,
                                                         int32_t* __restrict__ crow, float* __restrict__ cw,
                                                         int32_t* __restrict__ ccount, int32_t* __restrict__ n_unchosen) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  double den = 0.0;
  for (int e = lane; e < E; e += 64)
    if (pos[(size_t)t * E + e] >= 0) den += (double)scores[(size_t)e * T + t];
  for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o);
  den = __shfl(den, 0);
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int row = e < E ? pos[(size_t)t * E + e] : -1;
    const uint64_t m = ballot64(row >= 0);
    if (row >= 0) {
      const int i = base + __popcll(m & lanemask_lt());
      const double sc = (double)scores[(size_t)e * T + t];
      crow[(size_t)t * E + i] = row;
      cw[(size_t)t * E + i] = (float)(renorm ? sc / den : sc);
    }
    base += __popcll(m);
  }
  if (lane == 0) {
    ccount[t] = base;
    if (base == 0) atomicAdd(n_unchosen, 1);
  }
}

template <bool OUT_F32>
__global__ __launch_bounds__(256) void ec_combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ crow,
                                                         const float* __restrict__ cw,
                                                         const int32_t* __restrict__ ccount, int T, int d, int E,
                                                         int routed_rows, int has_shared, void* __restrict__ out) {
  const int t = blockIdx.y;
  const int col = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (col >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int n = ccount[t];
  for (int i = 0; i < n; ++i) {                 // the token's experts in ascending order
    const int row = crow[(size_t)t * E + i];
    const float wt = cw[(size_t)t * E + i];
    const float4 v = *reinterpret_cast<const float4*>(y + (size_t)row * d + col);
    acc.x = __fmaf_rn(wt, v.x, acc.x);
    acc.y = __fmaf_rn(wt, v.y, acc.y);
    acc.z = __fmaf_rn(wt, v.z, acc.z);
    acc.w = __fmaf_rn(wt, v.w, acc.w);
  }
  if (has_shared) {
    const float4 v = *reinterpret_cast<const float4*>(y + ((size_t)routed_rows + t) * d + col);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  if (OUT_F32) {
    *reinterpret_cast<float4*>((float*)out + (size_t)t * d + col) = acc;
  } else {
    uint2 o;
    o.x = pack_bf16x2(acc.x, acc.y);
    o.y = pack_bf16x2(acc.z, acc.w);
    *reinterpret_cast<uint2*>((bf16_t*)out + (size_t)t * d + col) = o;
  }
}

hipError_t launch_expert_choice(const ExpertChoiceArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.T > kEcMaxT || a.C < 1 || a.C > a.T) return hipErrorInvalidValue;
  ec_scores_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a.logits, a.T, a.E, a.scores, a.n_unchosen);
  ec_select_kernel<<<a.E, 1024, 0, s>>>(a.scores, a.T, a.E, a.C, a.pos, a.sorted_tokens, a.offsets, a.counts);
  ec_weights_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a.scores, a.pos, a.T, a.E, a.renormalize, a.crow, a.w, a.ccount,
                                                   a.n_unchosen);
  return hipGetLastError();
}

hipError_t launch_ec_combine(const EcCombineArgs& a, hipStream_t s) {
  dim3 g((a.d / 4 + 255) / 256, a.T);
  if (a.act_f32)
    ec_combine_kernel<true><<<g, 256, 0, s>>>(a.y, a.crow, a.w, a.ccount, a.T, a.d, a.E, a.routed_rows, a.has_shared,
                                              a.out);
  else
    ec_combine_kernel<false><<<g, 256, 0, s>>>(a.y, a.crow, a.w, a.ccount, a.T, a.d, a.E, a.routed_rows, a.has_shared,
                                               a.out);
  return hipGetLastError();
}

}  // namespace moe
