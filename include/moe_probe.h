/* Roofline probes for MI355X (gfx950), built as libmoe_probe.so.
 *
 * Measurement tools, not part of the MoE layer: they show what the part
 * itself sustains, the ceilings the layer's kernels are compared with
 * (bench.py --probe times them; rocprofv3 reads their counters).
 *
 * Both take plain device pointers and a HIP stream (NULL: the default
 * stream), enqueue one kernel and return a hipError_t value (0 on success,
 * hipErrorInvalidValue for the argument errors listed).  The caller owns
 * every buffer.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` bytes of `src` once (16-byte non-temporal loads, 32 KB chunks
 * dealt to `grid` work-groups of 256 threads) and write one 32-bit word per
 * thread to `sink` (grid * 256 words).  Errors: NULL pointers, grid <= 0,
 * bytes not a multiple of 32768. */
int probe_hbm_read(const void* src, size_t bytes, void* sink, int grid, hipStream_t stream);

/* grid work-groups of 256 threads; each wave runs iters * 8
 * v_mfma_f32_32x32x16_bf16 on operands loaded once from `src`
 * (grid * 256 * 64 bf16) into registers and writes one float per thread to
 * `out` (grid * 256 floats).  Work: grid * 4 * iters * 8 * 32768 flop.
 * Errors: NULL pointers, grid <= 0, iters <= 0 or odd. */
int probe_mfma_bf16(const void* src, int grid, int iters, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
