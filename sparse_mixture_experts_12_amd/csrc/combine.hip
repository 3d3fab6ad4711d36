// Weighted combine of the expert outputs of the MoE layer on gfx950.
//
// Pages: "MoE Model Architectures", Mixtral "Sparse MoE Block" (each expert
// output scaled by its routing weight and added to the token's row);
// DeepSeek-V3 "DeepSeekMoE Architecture" and "Design Patterns" (shared
// output + routed output).
//
// out[t] = sum_{j < k, kept} w[t, j] * y[inv_perm[t*k + j]]  (+ y[T*k + t])
// The sum runs in slot order in fp32 and is rounded once to the activation
// type; every output element has a single owner thread (no atomics).
#include "common.h"
#include "kernels.h"

namespace moe {

template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ inv_perm,
                                                      const float* __restrict__ w, int T, int d, int k,
                                                      int has_shared, void* __restrict__ out) {
  const int t = blockIdx.y;
  const int col = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (col >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int row = inv_perm[(size_t)t * k + j];
    if (row < 0) continue;
    const float wt = w[(size_t)t * k + j];
    const float4 v = *reinterpret_cast<const float4*>(y + (size_t)row * d + col);
    acc.x = __fmaf_rn(wt, v.x, acc.x);
    acc.y = __fmaf_rn(wt, v.y, acc.y);
    acc.z = __fmaf_rn(wt, v.z, acc.z);
    acc.w = __fmaf_rn(wt, v.w, acc.w);
  }
  if (has_shared) {
    const float4 v = *reinterpret_cast<const float4*>(y + ((size_t)T * k + t) * d + col);
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

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  dim3 g((a.d / 4 + 255) / 256, a.T);
  if (a.act_f32)
    combine_kernel<true><<<g, 256, 0, s>>>(a.y, a.inv_perm, a.w, a.T, a.d, a.k, a.has_shared, a.out);
  else
    combine_kernel<false><<<g, 256, 0, s>>>(a.y, a.inv_perm, a.w, a.T, a.d, a.k, a.has_shared, a.out);
  return hipGetLastError();
}

}  // namespace moe
