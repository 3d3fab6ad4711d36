// Device helpers shared by the gfx950 grouped GEMM kernels: the tile
// schedule decoder, LDS swizzles, wait-count and scheduling helpers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace moe {

// Map this work-group to (group, row0, rows, n-tile).  The schedule holds a
// heavy segment (row tiles of more than BM / 2 rows) and a light segment; each
// is split into 8 contiguous ranges of equal tile count, range x running on
// XCD x (work-groups are dealt to the XCDs round-robin by id), heavy tiles
// first.  Within the heavy segment a group's tiles are ordered column-major,
// so neighbouring row tiles of one weight column tile share an XCD's L2.
// Work-groups past both ranges return false.
// SEG selects the segments one launch covers: 0 both (heavy first), 1 the
// heavy segment only, 2 the light segment only (separate launches may use
// kernels shaped for each segment).
// lslot (optional): a light tile's index pt * n_tiles + nt in the light segment.
template <int SEG = 0>
__device__ __forceinline__ bool decode_tile(const int32_t* sched, int maxQ, int E, int n_tiles, int* g, int* row0,
                                            int* rows, int* nt, int* lslot = nullptr) {
  const int QH = SEG == 2 ? 0 : sched[0], QL = SEG == 1 ? 0 : sched[1];
  const int totH = QH * n_tiles, totL = QL * n_tiles;
  const int perH = (totH + 7) >> 3, perL = (totL + 7) >> 3;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int32_t* hs = sched + kSchedHead;
  if (slot < perH) {
    const int logical = xcd * perH + slot;
    if (logical >= totH) return false;
    const int q0 = logical / n_tiles;
    const int grp = hs[4 * q0 + 0];
    const int first = hs[4 * q0 + 3];
    const int mg = hs[4 * maxQ + grp];
    const int local = logical - first * n_tiles;
    const int j = local / mg;
    const int q = first + (local - j * mg);
    *g = grp;
    *row0 = hs[4 * q + 1];
    *rows = hs[4 * q + 2];
    *nt = j;
    return true;
  }
  const int s = slot - perH;
  if (s >= perL) return false;
  const int logical = xcd * perL + s;
  if (logical >= totL) return false;
  const int pt = logical / n_tiles;
  const int32_t* ls = hs + 4 * maxQ + (E + 1) + 3 * pt;
  *g = ls[0];
  *row0 = ls[1];
  *rows = ls[2];
  *nt = logical - pt * n_tiles;
  if (lslot) *lslot = logical;
  return true;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// s_waitcnt: vmcnt(N) alone, or vmcnt(N) together with lgkmcnt(0)
template <int N> __device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}
template <int N> __device__ __forceinline__ void wait_vmem_le_lds0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}

// A tile rows hold BK bf16 = CPR 16-byte chunks; the chunk index is XOR-ed
// with a function of the row so that each 16-lane pass of a ds_read_b128
// (rows r .. r + 15, one chunk each) hits distinct banks.  Both keys were
// checked against the LDS bank-conflict counter on gfx950.
template <int CPR> __device__ __forceinline__ int aswz(int r, int c) {
  if constexpr (CPR == 8) return c ^ ((r ^ (r >> 3)) & 7);
  else return c ^ ((r >> 2) & 3);
}

// Scheduling hint for one K sub-step: each MFMA is followed by its share of
// the LDS fragment reads (DS) and of the global->LDS loads (VM), so the
// memory instructions issue while the matrix core is busy.
template <int NMF, int NDS, int NVM, int I = 0>
__device__ __forceinline__ void sched_interleave() {
  if constexpr (I < NMF) {
    constexpr int DPM = (NDS + NMF - 1) / NMF, VPM = (NVM + NMF - 1) / NMF;
    constexpr int D = (NDS - I * DPM) < DPM ? (NDS - I * DPM) : DPM;
    constexpr int V = (NVM - I * VPM) < VPM ? (NVM - I * VPM) : VPM;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (D > 0) __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x010, V, 0);
    sched_interleave<NMF, NDS, NVM, I + 1>();
  }
}

}  // namespace moe
