// Router telemetry on gfx950: per-expert routed load, mean full-softmax
// probability and the load-balancing loss of one routing.
//
// Pages: "MoE Model Architectures", Switch Transformers "Load Balancing Loss"
// (E times the sum over experts of the mean router probability times the
// fraction of tokens routed there); DeepSeek-V3 "Auxiliary-Loss-Free Load
// Balancing" (a per-expert bias steers the per-expert load reported here).
//
// Inputs are the router's fp32 logits [T, E] and chosen experts [T, k]
// (before any capacity limit).  With k slots per token, the token-mean of the
// one-hot of each slot summed over the slots is routed[e] / T, so
//   prob_mean[e] = (1/T) sum_t softmax(logits[t])[e]      (fp64, rounded to fp32)
//   lb_loss      = E * sum_e prob_mean[e] * routed[e] / T
// Every sum is taken in a fixed order (bitwise reproducible).  Up to 64
// tokens: one work-group does everything.  More tokens: three launches,
//   1. one wave per token: max and fp64 softmax denominator of its logits;
//   2. work-group (64 experts, 64-token chunk): fp64 probability sums and
//      integer routed counts of the chunk, waves combined in a fixed order;
//   3. one work-group: chunks added in order, then the loss terms in expert order.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kTelChunk = 64;     // tokens per chunk in launch 2

__global__ __launch_bounds__(256) void telemetry_token_kernel(const float* __restrict__ logits, int T, int E,
                                                              double* __restrict__ mz) {
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
  if (lane == 0) {
    mz[2 * t] = (double)m;
    mz[2 * t + 1] = z;
  }
}

// grid (ceil(E / 64), nchunk); lane = expert, wave w takes the chunk's tokens
// w, w + 4, ...  The chunk's top-k indices and per-token (max, denominator)
// are staged in LDS first and each thread issues its logit loads together,
// so no load waits on another.
__global__ __launch_bounds__(256) void telemetry_chunk_kernel(const float* __restrict__ logits,
                                                              const double* __restrict__ mz,
                                                              const int32_t* __restrict__ idx, int T, int E, int k,
                                                              double* __restrict__ psum, int32_t* __restrict__ pcnt) {
  constexpr int TPW = kTelChunk / 4;                  // tokens per wave
  __shared__ int32_t sidx[kTelChunk * kMaxTopK];
  __shared__ double smz[kTelChunk][2];
  __shared__ double sp[4][64];
  __shared__ int sc[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 64 + lane;
  const int c = blockIdx.y;
  const int t0 = c * kTelChunk;
  const int nt = min(T - t0, kTelChunk);
  for (int i = threadIdx.x; i < nt * k; i += 256) sidx[i] = idx[(size_t)t0 * k + i];
  for (int i = threadIdx.x; i < nt * 2; i += 256) smz[i >> 1][i & 1] = mz[2 * (size_t)t0 + i];
  float lv[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tl = wave + 4 * i;
    const bool ok = tl < nt && e < E;
    lv[i] = logits[(size_t)(t0 + (ok ? tl : 0)) * E + (ok ? e : 0)];
  }
  __syncthreads();
  double s = 0.0;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tl = wave + 4 * i;
    if (tl < nt) {
      if (e < E) s += exp((double)lv[i] - smz[tl][0]) / smz[tl][1];
      for (int j = 0; j < k; ++j) cnt += (sidx[tl * k + j] == e) ? 1 : 0;
    }
  }
  sp[wave][lane] = s;
  sc[wave][lane] = cnt;
  __syncthreads();
  if (wave == 0 && e < E) {
    psum[(size_t)c * E + e] = ((sp[0][lane] + sp[1][lane]) + sp[2][lane]) + sp[3][lane];
    pcnt[(size_t)c * E + e] = sc[0][lane] + sc[1][lane] + sc[2][lane] + sc[3][lane];
  }
}

__global__ __launch_bounds__(1024) void telemetry_final_kernel(const double* __restrict__ psum,
                                                               const int32_t* __restrict__ pcnt, int nchunk, int T,
                                                               int E, int32_t* __restrict__ routed,
                                                               float* __restrict__ prob_mean,
                                                               float* __restrict__ lb_loss) {
  __shared__ double term[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double s = 0.0;
    int cnt = 0;
    int c = 0;
    for (; c + 8 <= nchunk; c += 8) {          // eight independent loads in flight, summed in order
      double v[8];
      int n[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = psum[(size_t)(c + i) * E + e];
        n[i] = pcnt[(size_t)(c + i) * E + e];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s += v[i];
        cnt += n[i];
      }
    }
    for (; c < nchunk; ++c) {
      s += psum[(size_t)c * E + e];
      cnt += pcnt[(size_t)c * E + e];
    }
    const double pm = s / (double)T;
    if (routed) routed[e] = cnt;
    if (prob_mean) prob_mean[e] = (float)pm;
    term[e] = pm * ((double)cnt / (double)T);
  }
  __syncthreads();
  if (threadIdx.x == 0 && lb_loss) {
    double acc = 0.0;
    for (int e = 0; e < E; ++e) acc += term[e];
    *lb_loss = (float)((double)E * acc);
  }
}

// T <= kTelChunk (decode and small batches): the three stages in one
// work-group of 1024 threads, tokens summed in order 0..T-1 per expert.
__global__ __launch_bounds__(1024) void telemetry_small_kernel(const float* __restrict__ logits,
                                                              const int32_t* __restrict__ idx, int T, int E, int k,
                                                              int32_t* __restrict__ routed,
                                                              float* __restrict__ prob_mean,
                                                              float* __restrict__ lb_loss) {
  __shared__ double smz[kTelChunk][2];
  __shared__ int32_t sidx[kTelChunk * kMaxTopK];
  __shared__ double term[kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < T * k; i += blockDim.x) sidx[i] = idx[i];
  for (int t = wave; t < T; t += 16) {
    const float* l = logits + (size_t)t * E;
    float m = -INFINITY;
    for (int e = lane; e < E; e += 64) m = fmaxf(m, l[e]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    double z = 0.0;
    for (int e = lane; e < E; e += 64) z += exp((double)l[e] - (double)m);
    for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
    if (lane == 0) {
      smz[t][0] = (double)m;
      smz[t][1] = z;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    double s = 0.0;
    int cnt = 0;
    for (int t = 0; t < T; ++t) {
      s += exp((double)logits[(size_t)t * E + e] - smz[t][0]) / smz[t][1];
      for (int j = 0; j < k; ++j) cnt += (sidx[t * k + j] == e) ? 1 : 0;
    }
    const double pm = s / (double)T;
    if (routed) routed[e] = cnt;
    if (prob_mean) prob_mean[e] = (float)pm;
    term[e] = pm * ((double)cnt / (double)T);
  }
  __syncthreads();
  if (threadIdx.x == 0 && lb_loss) {
    double acc = 0.0;
    for (int e = 0; e < E; ++e) acc += term[e];
    *lb_loss = (float)((double)E * acc);
  }
}

size_t telemetry_ws_bytes(int T, int E) {
  const size_t nchunk = (T + kTelChunk - 1) / kTelChunk;
  return (size_t)T * 2 * sizeof(double) + nchunk * E * (sizeof(double) + sizeof(int32_t)) + 64;
}

hipError_t launch_telemetry(const TelemetryArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  if (a.T <= kTelChunk) {
    telemetry_small_kernel<<<1, 1024, 0, s>>>(a.logits, a.idx, a.T, a.E, a.k, a.routed, a.prob_mean, a.lb_loss);
    return hipGetLastError();
  }
  const int nchunk = (a.T + kTelChunk - 1) / kTelChunk;
  double* mz = (double*)a.ws;
  double* psum = mz + 2 * (size_t)a.T;
  int32_t* pcnt = (int32_t*)(psum + (size_t)nchunk * a.E);
  telemetry_token_kernel<<<(a.T + 3) / 4, 256, 0, s>>>(a.logits, a.T, a.E, mz);
  telemetry_chunk_kernel<<<dim3((a.E + 63) / 64, nchunk), 256, 0, s>>>(a.logits, mz, a.idx, a.T, a.E, a.k, psum,
                                                                      pcnt);
  telemetry_final_kernel<<<1, 1024, 0, s>>>(psum, pcnt, nchunk, a.T, a.E, a.routed, a.prob_mean, a.lb_loss);
  return hipGetLastError();
}

}  // namespace moe
