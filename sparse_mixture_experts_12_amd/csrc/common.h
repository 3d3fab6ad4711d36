// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;   // raw bf16 bits
typedef uint8_t fp8_t;     // raw OCP e4m3fn bits

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// Four OCP e4m3fn codes (one dword) -> four fp32 with the gfx950 converter.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float* o) {
  f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  o[0] = a[0]; o[1] = a[1]; o[2] = b[0]; o[3] = b[1];
}

template <typename T> struct ActTraits;
template <> struct ActTraits<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
};
template <> struct ActTraits<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
};

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Wave-wide helpers (64 lanes).
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
