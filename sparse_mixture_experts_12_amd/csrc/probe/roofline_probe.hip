// Roofline probes for MI355X (gfx950): what the chip itself sustains, as the
// ceilings the layer's kernels are compared with.  Not part of the MoE layer;
// bench.py --probe times these launches and rocprofv3 reads their counters.
//
//   probe_hbm_read:  every byte of a buffer (much larger than the 256 MB
//                    last-level cache) read once with 16-byte non-temporal
//                    loads, eight in flight per lane, in 32 KB chunks dealt to
//                    the work-groups; one word per thread written at the end.
//   probe_mfma_bf16: v_mfma_f32_32x32x16_bf16 back to back on operands held
//                    in registers (no memory traffic inside the loop), eight
//                    independent accumulators per wave.  Operands come from a
//                    buffer the caller fills: random values exercise the data
//                    paths the way a real GEMM does, zeros show the clock the
//                    chip holds when they toggle nothing.
//
// C ABI: plain device pointers, a stream; returns a hipError_t code.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 32 KB chunks: chunk c (c = blockIdx.x, blockIdx.x + gridDim.x, ...) is read
// as 8 coalesced 4 KB rows of 16-byte loads, all 8 in flight per lane.
constexpr int kReadUnroll = 8;
constexpr size_t kReadChunk16 = 256 * kReadUnroll;   // 16-byte words per chunk

__global__ __launch_bounds__(256) void probe_hbm_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                            uint32_t* __restrict__ sink) {
  const int tid = threadIdx.x;
  uint32_t acc = 0;
  const size_t nchunks = n16 / kReadChunk16;
  for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const u32x4_t* p = src + c * kReadChunk16 + tid;
    u32x4_t v[kReadUnroll];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) v[j] = __builtin_nontemporal_load(p + 256 * j);
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  sink[(size_t)blockIdx.x * 256 + tid] = acc;
}

// src: 8 fragments of 8 bf16 per lane for every thread of the grid
// (gridDim.x * 256 * 64 bf16); out: one float per thread.
__global__ __launch_bounds__(256) void probe_mfma_bf16_kernel(const bf16x8_t* __restrict__ src, int iters,
                                                             float* __restrict__ out) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = src[tid * 8 + i];
    b[i] = src[tid * 8 + 4 + i];
  }
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  // two iterations per trip, so every operand index is a compile-time constant
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j & 3], b[(j >> 2) + 2 * h], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  out[tid] = s;
}

extern "C" {

// Reads bytes (a multiple of 32 KB) from src; sink holds grid * 256 words.
int probe_hbm_read(const void* src, size_t bytes, void* sink, int grid, hipStream_t s) {
  if (!src || !sink || grid <= 0 || bytes % (kReadChunk16 * 16)) return (int)hipErrorInvalidValue;
  probe_hbm_read_kernel<<<grid, 256, 0, s>>>((const u32x4_t*)src, bytes / 16, (uint32_t*)sink);
  return (int)hipGetLastError();
}

// grid * 256 threads, iters (even) * 8 MFMAs per wave; src holds
// grid * 256 * 64 bf16, out grid * 256 floats.  Flops = grid * 4 * iters * 8 * 32768.
int probe_mfma_bf16(const void* src, int grid, int iters, void* out, hipStream_t s) {
  if (!src || !out || grid <= 0 || iters <= 0 || iters % 2) return (int)hipErrorInvalidValue;
  probe_mfma_bf16_kernel<<<grid, 256, 0, s>>>((const bf16x8_t*)src, iters, (float*)out);
  return (int)hipGetLastError();
}

}  // extern "C"
