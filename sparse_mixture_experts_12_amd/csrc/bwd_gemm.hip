// Grouped bf16 GEMMs of the layer's backward pass on gfx950.
//
// Pages: "Testing using claude to graft ETHOS onto modded-nanogpt base", "Key
// Implementation Details" (a backward that recomputes the forward values and
// accumulates each weight gradient over the tokens that chose the expert;
// there with atomics, here as one deterministic reduction per output tile);
// "MoE Model Architectures", Mixtral "Expert FFN" (the forward being
// differentiated: w2(silu(w1 x) * w3 x)).
//
// Every backward GEMM runs over the padded permuted row space: the rows of
// group g (expert g, or the shared expert as group E) sit at [poff[g],
// poff[g + 1]), a multiple of 64 rows whose tail rows hold zeros.  One tile
// routine covers the five products through the two layouts an operand can
// have in memory:
//   KC  K contiguous:   A(m, k) = A[m * lda + k]   (B(k, n) = B[n * ldb + k])
//   MC  K selects rows: A(m, k) = A[k * lda + m]   (B(k, n) = B[k * ldb + n])
//   MODE_GU  G, U = Xp W_gate, Xp W_up      A KC (padded rows), B MC (weights)
//   MODE_NT  C = A B^T-style products       A KC (padded rows), B KC (weights,
//            output-major rows); MODE_NTS the same with K split over two
//            (A, B) pairs
//   MODE_TN  dW = A^T B over a group's rows A MC, B MC (activations), K = rows
// KC tiles live in LDS as rows of 64 K values (128 bytes, 16-byte chunks
// swizzled by aswz<8>) and reach the MFMA with ds_read_b128; MC tiles as 64
// K-rows of 256 values (swizzled by bswz) read with the transposing
// ds_read_b64_tr_b16 -- the two layouts of the forward kernel's A and B.
// Tiles: up to 256 x 256, 4 waves (2 x 2 of 128 x 128, or 1 x 4 for the
// 128- and 64-row bodies of a group's last row tile), v_mfma_f32_32x32x16_bf16,
// 64 K per LDS stage, two stages filled by global_load_lds.
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int MODE_GU = 0, MODE_NT = 1, MODE_NTS = 2, MODE_TN = 3;   // NTS: NT with K split over two pairs
constexpr int kBK = 64;

__device__ __forceinline__ int bswz_key(int k) { return ((k & 3) << 4) | ((k & 1) << 6); }
__device__ __forceinline__ int bswz(int k, int n) { return k * 256 + (n ^ bswz_key(k)); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// 8 consecutive K of one M (or N) index per lane from an MC tile (64 K-rows
// x 256, swizzled by bswz) with two transposing reads: within each 16-lane
// group, output lane 4a + b receives element b of the 4-element rows of
// input lanes a, a + 4, a + 8, a + 12.
__device__ __forceinline__ bf16x8_t mc_frag(const bf16_t* Ls, int kbase, int nbase, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int a = i & 3, j = i >> 2;
  const int n = nbase + 16 * (g & 1) + 4 * a;
  const int k0 = kbase + 8 * (g >> 1) + j;
  typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(Ls + bswz(k0, n)));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(Ls + bswz(k0 + 4, n)));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace

// One output tile of at most BMV rows (see the file comment for the modes).
// LDS stages hold BMMAX A rows (KC) or 256 A columns (MC) plus the B tile;
// NST stages form the ring (3: light row tiles, two steps of loads in flight).
// K runs over [kbeg, kbeg + nK kBK).  NT / NTS tiles with kpart > 0 (light
// row tiles split over K) write their fp32 block to p.part slot `slot`.
// Work-group barrier for LDS only: this wave's LDS operations complete, then
// s_barrier.  Unlike __syncthreads() it does not wait for outstanding global
// stores or direct-to-LDS loads, so the weight-gradient stores keep draining
// across it (the empty asm statements keep the compiler from moving memory
// operations across the barrier).
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  wait_vmem_le_lds0<63>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// TN (weight-gradient) tiles of a persistent work-group also take:
//   pre: this tile's only K step (nK == 1) was issued into L0 by the previous
//        tile, before that tile's 64 stores per thread;
//   nx:  issue the next tile's only K step (tile origin nx_m0, nx_n0, first
//        padded row nx_k) into L1 here, after the K loop and before this
//        tile's stores (this tile must lie wholly inside the output, so that
//        every wave issues exactly 64 stores after those loads).
template <int MODE, int BMV, int BMMAX = 256, int NST = 2>
__device__ __forceinline__ void bwd_tile(const BwdGemmParams& p, int g, int row0, int rows, int n0, int kbeg,
                                         int nK, bf16_t* L0, bf16_t* L1, bf16_t* L2 = nullptr, int kpart = 0,
                                         int slot = 0, bool pre = false, bool nx = false, int nx_m0 = 0,
                                         int nx_n0 = 0, int nx_k = 0) {
  constexpr bool A_KC = MODE != MODE_TN;
  constexpr bool B_KC = MODE == MODE_NT || MODE == MODE_NTS;
  constexpr bool DUAL = MODE == MODE_GU;
  constexpr int WM = (BMV >= 256) ? 2 : 1, WN = 4 / WM;
  constexpr int NMAT = DUAL ? 2 : 1;
  constexpr int BN_MAT = DUAL ? 128 : 256;
  constexpr int NI_MAT = BN_MAT / WN / 32;
  constexpr int NI = NI_MAT * NMAT;
  constexpr int MI = BMV / WM / 32;
  constexpr int WROWS = BMV / WM;
  constexpr int A_LD = A_KC ? BMV / 8 / 4 : 8;      // 1 KB blocks per wave per stage
  constexpr int B_LD = 8;
  constexpr int LDS_B = (MODE == MODE_TN ? 256 : BMMAX) * kBK;   // B tile offset (elements) inside a stage
  static_assert(BMV <= BMMAX && (NST == 2 || NST == 3) && (MODE != MODE_TN || (BMMAX == 256 && NST == 2)),
                "backward tile configuration");
  constexpr int NMF = MI * NI;
  constexpr int NDS = (A_KC ? MI : 2 * MI) + (B_KC ? NI : 2 * NI);
  constexpr int NVM = A_LD + B_LD;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const bool shared = (g == p.E);

  // ---- A sources ----
  // KC: block b = wave + 4 i holds tile rows 8 b .. 8 b + 7; this lane fills
  //     row r = 8 b + lane / 8, LDS chunk lane % 8 = global chunk
  //     aswz<8>(r, lane % 8) (8 K values).  Rows past the valid ones read the
  //     tile's first row (never stored).
  // MC: block b = 8 wave + i holds K-rows 2 b, 2 b + 1; this lane fills K-row
  //     2 b + lane / 32, LDS chunk lane % 32 = global chunk (lane % 32) ^
  //     (bswz_key(krow) / 8) of the 256 M columns from row0 (clamped to M).
  uint32_t aoff[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    if constexpr (A_KC) {
      const int r = 8 * (wave + 4 * i) + (lane >> 3);
      const int rr = row0 + (r < rows ? r : 0);
      aoff[i] = (uint32_t)rr * (uint32_t)p.lda + aswz<8>(r, lane & 7) * 8;
    } else {
      const int krow = 2 * (8 * wave + i) + (lane >> 5);
      int m = row0 + ((lane & 31) ^ (bswz_key(krow) >> 3)) * 8;
      if (m > p.M - 8) m = p.M - 8;
      aoff[i] = (uint32_t)krow * (uint32_t)p.lda + m;
    }
  }
  // ---- B sources (same two layouts) ----
  const bf16_t* bb0;
  const bf16_t* bb1;
  if constexpr (MODE == MODE_TN) {
    bb0 = p.B0;
    bb1 = p.B0;
  } else {
    const size_t gs = shared ? 0 : (size_t)g * (size_t)p.bgs;
    bb0 = shared ? p.Bs0 : p.B0 + gs;
    bb1 = shared ? p.Bs1 : (p.B1 ? p.B1 + gs : nullptr);
  }
  uint32_t boff[B_LD];
#pragma unroll
  for (int j = 0; j < B_LD; ++j) {
    if constexpr (B_KC) {
      const int r = 8 * (B_LD * wave + j) + (lane >> 3);
      int c = n0 + r;
      if (c > p.N - 1) c = p.N - 1;
      boff[j] = (uint32_t)c * (uint32_t)p.ldb + aswz<8>(r, lane & 7) * 8;
    } else {
      const int krow = 2 * (B_LD * wave + j) + (lane >> 5);
      const int gc = (lane & 31) ^ (bswz_key(krow) >> 3);
      int c;
      if (DUAL) c = n0 + (gc & 15) * 8;          // columns 0..127 gate, 128..255 up
      else c = n0 + gc * 8;
      if (c > p.N - 8) c = p.N - 8;
      boff[j] = (uint32_t)krow * (uint32_t)p.ldb + c;
    }
  }

  // Load K-step k0 (absolute K index kbeg + k0) into stage L.
  auto issue = [&](bf16_t* L, int k0) {
    const bf16_t* a_base;
    const bf16_t* b_base;
    const bf16_t* b_base_up = nullptr;
    uint32_t ak, bk;
    if constexpr (MODE == MODE_NTS) {
      const int ka = kbeg + k0;
      const bool second = ka >= p.K1;             // K split over two (A, B) pairs
      const int kk = second ? ka - p.K1 : ka;
      a_base = second ? p.A1 : p.A0;
      b_base = second ? bb1 : bb0;
      ak = (uint32_t)kk;
      bk = (uint32_t)kk;
    } else if constexpr (MODE == MODE_NT) {
      a_base = p.A0;
      b_base = bb0;
      ak = (uint32_t)(kbeg + k0);
      bk = (uint32_t)(kbeg + k0);
    } else if constexpr (MODE == MODE_GU) {
      a_base = p.A0;
      b_base = bb0;
      b_base_up = bb1;
      ak = (uint32_t)(kbeg + k0);
      bk = (uint32_t)(kbeg + k0) * (uint32_t)p.ldb;
    } else {
      a_base = p.A0;
      b_base = bb0;
      ak = (uint32_t)(kbeg + k0) * (uint32_t)p.lda;
      bk = (uint32_t)(kbeg + k0) * (uint32_t)p.ldb;
    }
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int blk = A_KC ? wave + 4 * i : 8 * wave + i;
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(a_base + (aoff[i] + ak)), (lds_ptr_t)(L + blk * 512), 16, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
      const bf16_t* bsrc = b_base;
      if constexpr (DUAL) {
        const int krow = 2 * (B_LD * wave + j) + (lane >> 5);
        const int gc = (lane & 31) ^ (bswz_key(krow) >> 3);
        bsrc = (gc >> 4) ? b_base_up : b_base;
      }
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(bsrc + (boff[j] + bk)), (lds_ptr_t)(L + LDS_B + (B_LD * wave + j) * 512),
                                       16, 0, 0);
    }
  };

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  auto b_col = [&](int ni) -> int {           // tile-local B index (N) of fragment ni
    if (DUAL) return (ni / NI_MAT) * 128 + wn * (128 / WN) + (ni % NI_MAT) * 32;
    return wn * (256 / WN) + ni * 32;
  };
  auto frags = [&](const bf16_t* L, int ks, bf16x8_t* af, bf16x8_t* bfr) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int mb = wm * WROWS + mi * 32;
      if constexpr (A_KC) {
        const int row = mb + l32;
        af[mi] = *reinterpret_cast<const bf16x8_t*>(L + row * kBK + aswz<8>(row, ks * 2 + lhi) * 8);
      } else {
        af[mi] = mc_frag(L, ks * 16, mb, lane);
      }
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int nb = b_col(ni);
      if constexpr (B_KC) {
        const int j = nb + l32;
        bfr[ni] = *reinterpret_cast<const bf16x8_t*>(L + LDS_B + j * kBK + aswz<8>(j, ks * 2 + lhi) * 8);
      } else {
        bfr[ni] = mc_frag(L + LDS_B, ks * 16, nb, lane);
      }
    }
  };
  // TN tiles multiply with the operands swapped, so the accumulators hold the
  // transposed fragment: a lane then owns 4 consecutive output columns of one
  // output row per register quad (16-byte stores in the epilogue).
  auto mfmas = [&](const bf16x8_t* af, const bf16x8_t* bfr) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        if constexpr (MODE == MODE_TN)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
        else
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
      }
  };

  // Two-stage pipeline over 16-wide K sub-steps (the forward kernel's): the
  // next sub-step's fragments are read while the current one multiplies; the
  // stage just read is refilled two steps ahead (past the end: the last step
  // again, never read), so the vmcnt thresholds are exact.
  if (MODE == MODE_TN && nK > 0 && nK <= 2) {
    // weight-gradient tiles of small groups (one or two K steps): both stages
    // are loaded once and used once, without the pipeline's refills of the
    // last step (which would triple the loads of a one-step tile and add a
    // round trip to wait for them)
    bf16x8_t fa[MI], fb[NI];
    if (pre) {
      // 16 loads, then exactly 64 stores per wave were issued: at most 63
      // outstanding means the loads are done (vmcnt retires in issue order),
      // while the stores keep draining under this tile's MFMAs
      wait_vmem_le<63>();
    } else {
      issue(L0, 0);
      if (nK == 2) issue(L1, kBK);
      wait_vmem_le<0>();
    }
    __builtin_amdgcn_s_barrier();
    for (int st = 0; st < nK; ++st) {
      const bf16_t* L = st ? L1 : L0;
#pragma unroll
      for (int sub = 0; sub < kBK / 16; ++sub) {
        frags(L, sub, fa, fb);
        mfmas(fa, fb);
      }
    }
  } else if (nK > 0) {
    bf16x8_t fa0[MI], fb0[NI], fa1[MI], fb1[NI];
    issue(L0, 0);
    issue(L1, min(1, nK - 1) * kBK);
    if constexpr (NST > 2) issue(L2, min(2, nK - 1) * kBK);
    wait_vmem_le<(NST - 1) * NVM>();
    __builtin_amdgcn_s_barrier();
    frags(L0, 0, fa0, fb0);
    auto step = [&](bf16_t* L, const bf16_t* Ln, int k) {
#pragma unroll
      for (int sub = 0; sub < 3; ++sub) {
        if (sub & 1) {
          frags(L, sub + 1, fa0, fb0);
          mfmas(fa1, fb1);
        } else {
          frags(L, sub + 1, fa1, fb1);
          mfmas(fa0, fb0);
        }
        sched_interleave<NMF, NDS, 0>();
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_vmem_le_lds0<(NST - 2) * NVM>();
      __builtin_amdgcn_s_barrier();
      issue(L, min(k + NST, nK - 1) * kBK);
      frags(Ln, 0, fa0, fb0);
      mfmas(fa1, fb1);
      sched_interleave<NMF, NDS, NVM>();
      __builtin_amdgcn_sched_barrier(0);
    };
    int k = 0;
    if constexpr (NST == 2) {
      for (; k + 2 <= nK; k += 2) {
        step(L0, L1, k);
        step(L1, L0, k + 1);
      }
      if (k < nK) step(L0, L1, k);
    } else {
      for (; k + 3 <= nK; k += 3) {
        step(L0, L1, k);
        step(L1, L2, k + 1);
        step(L2, L0, k + 2);
      }
      if (k < nK) step(L0, L1, k);
      if (k + 1 < nK) step(L1, L2, k + 1);
    }
    wait_vmem_le<0>();
  }

  // ---- epilogue: fp32 stores ----
  if constexpr (MODE == MODE_TN) {
    // acc[mi][ni][4 q + i] = C[row, col0 + i] with row = row0 + mb + l32 and
    // col0 = n0 + nb + 8 q + 4 lhi (transposed fragment, see mfmas).  The
    // 256 x 256 fp32 tile leaves through L0 in four quarters of 64 rows, so
    // the global stores are whole 1 KB rows (64 lanes x 16 bytes) and L1 is
    // free for the next tile's loads.  LDS row r
    // (1 KB) holds 16-byte chunk c at position c ^ (r & 15): the 16-lane
    // passes of both the fragment writes (16 rows, one chunk) and the row
    // reads (one row, 16 chunks) hit distinct banks.
    static_assert(BMV == 256 && WM == 2, "weight-gradient tiles are 256 x 256");
    float* C = shared ? p.Cs : p.C0 + (size_t)g * p.cstride;
    float* Lq = reinterpret_cast<float*>(L0);     // one 64-row quarter (64 KB) at a time
    // quarter h of the accumulators -> Lq (the waves holding its 64 rows)
    auto stage_quarter = [&](int h) {
      if (wm == (h >> 1)) {
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
          const int mi = 2 * (h & 1) + m2;
          const int r = m2 * 32 + l32;
          float* Lr = Lq + r * 256;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int chunk = (b_col(ni) + 8 * q + 4 * lhi) >> 2;
              const f32x4_t v = {acc[mi][ni][4 * q], acc[mi][ni][4 * q + 1], acc[mi][ni][4 * q + 2],
                                 acc[mi][ni][4 * q + 3]};
              *reinterpret_cast<f32x4_t*>(Lr + ((chunk ^ (r & 15)) << 2)) = v;
            }
        }
      }
    };
    // 64 rows x 64 chunks per quarter; thread t takes chunk t % 64 of rows
    // t / 64, + 4, ...  Stores are non-temporal: the gradients are not read
    // again here, and streaming writes would otherwise evict the group's rows
    // that the next tiles reuse.
    const int chunk = tid & 63;
    const int col = n0 + chunk * 4;
    if (row0 + 256 <= p.M && n0 + 256 <= p.N) {
      // whole tile in range: 16 unconditional stores per thread and quarter,
      // so every path the compiler sees from a prefetch passes 64 stores
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        lds_sync();                               // LDS free (K loop or previous quarter done)
        if (h == 0 && nx) {
          // the next tile's K step into L1 (the sources issue() computes)
          const uint32_t ka = (uint32_t)nx_k * (uint32_t)p.lda, kb = (uint32_t)nx_k * (uint32_t)p.ldb;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int krow = 2 * (8 * wave + i) + (lane >> 5);
            const int sw = (lane & 31) ^ (bswz_key(krow) >> 3);
            int m = nx_m0 + sw * 8;
            if (m > p.M - 8) m = p.M - 8;
            int c = nx_n0 + sw * 8;
            if (c > p.N - 8) c = p.N - 8;
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(p.A0 + ((uint32_t)krow * (uint32_t)p.lda + m + ka)),
                                             (lds_ptr_t)(L1 + (8 * wave + i) * 512), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_ptr_t)(p.B0 + ((uint32_t)krow * (uint32_t)p.ldb + c + kb)),
                                             (lds_ptr_t)(L1 + LDS_B + (8 * wave + i) * 512), 16, 0, 0);
          }
        }
        stage_quarter(h);
        lds_sync();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = (tid >> 6) + 4 * i;
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(Lq + r * 256 + ((chunk ^ (r & 15)) << 2));
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(C + (size_t)(row0 + 64 * h + r) * p.N + col));
        }
      }
    } else {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        lds_sync();
        stage_quarter(h);
        lds_sync();
#pragma unroll 4
        for (int r = tid >> 6; r < 64; r += 4) {
          const int grow = row0 + 64 * h + r;
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(Lq + r * 256 + ((chunk ^ (r & 15)) << 2));
          if (grow < p.M && col < p.N)
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(C + (size_t)grow * p.N + col));
        }
      }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int nl = 0; nl < NI_MAT; ++nl) {
        const int col = n0 + b_col(nl) + l32;
        if (col >= p.N) continue;
        // K part 0 (or no split): C0 rows; parts 1..: this slot's 128 x 256 block
        float* out = kpart == 0 ? p.C0 + (size_t)row0 * p.N + col
                                : p.part + ((size_t)(kpart - 1) * p.part_slots + slot) * (128 * 256) + (col - n0);
        const size_t ostride = kpart == 0 ? (size_t)p.N : 256;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WROWS + mi * 32 + (v >> 2) * 8 + lhi * 4 + (v & 3);
          if (r >= rows) continue;
          out[(size_t)r * ostride] = acc[mi][nl][v];
          if constexpr (DUAL) p.C1[(size_t)(row0 + r) * p.N + col] = acc[mi][nl + NI_MAT][v];
        }
      }
  }
}

// GU / NT: row tiles of the padded groups from the device schedule.
// SEG 1: heavy row tiles (> 128 rows), 256-row stages two deep; SEG 2: light
// row tiles (a group's last <= 128 rows), 128-row stages three deep (two steps
// of loads in flight: these tiles mostly stream weights).
template <int MODE, int SEG>
__global__ __launch_bounds__(256, 1) void bwd_rows_kernel(BwdGemmParams p) {
  constexpr int BMMAX = SEG == 1 ? 256 : 128;
  constexpr int NST = SEG == 1 ? 2 : 3;
  constexpr int LDS_S = (BMMAX + 256) * kBK;
  __shared__ __attribute__((aligned(1024))) bf16_t L0[LDS_S];
  __shared__ __attribute__((aligned(1024))) bf16_t L1[LDS_S];
  __shared__ __attribute__((aligned(1024))) bf16_t L2[NST > 2 ? LDS_S : 8];
  constexpr int BN_MAT = MODE == MODE_GU ? 128 : 256;
  const int n_tiles = (p.N + BN_MAT - 1) / BN_MAT;
  int g, row0, rows, nt, slot = 0;
  // the schedule lists the G padded groups (the shared expert is group E)
  if (!decode_tile<SEG>(p.sched, p.maxQ, p.G, n_tiles, &g, &row0, &rows, &nt, &slot)) return;
  // light NT / NTS tiles may be split over K (blockIdx.y = K part)
  constexpr bool KSPLIT = SEG == 2 && MODE != MODE_GU;
  const int kparts = KSPLIT && p.ksplit > 1 ? p.ksplit : 1;
  const int kpart = KSPLIT ? (int)blockIdx.y : 0;
  const int nK = p.K / kBK / kparts;
  const int kbeg = kpart * nK * kBK;
  if constexpr (SEG == 1) {
    bwd_tile<MODE, 256, BMMAX, NST>(p, g, row0, rows, nt * BN_MAT, kbeg, nK, L0, L1, L2);
  } else {
    if (rows > 64) bwd_tile<MODE, 128, BMMAX, NST>(p, g, row0, rows, nt * BN_MAT, kbeg, nK, L0, L1, L2, kpart, slot);
    else bwd_tile<MODE, 64, BMMAX, NST>(p, g, row0, rows, nt * BN_MAT, kbeg, nK, L0, L1, L2, kpart, slot);
  }
}

// TN: 256 x 256 tiles of the groups' weight gradients.  A tile's K loop runs
// over its group's padded rows, so with skewed groups (a Zipf router bias)
// equal tile counts per XCD would leave most of the work on one XCD.  Each
// XCD instead takes the contiguous range of tiles (group-major, as before,
// so a group's tiles share that XCD's L2) whose cost prefix falls in its
// eighth of the total cost, a tile costing its group's rows plus a fixed
// kWgTileCost for the prologue and the 256 KB of stores; the XCD's
// work-groups stride through the range.
constexpr long long kWgTileCost = 96;   // measured on fine_grained: 64-128 best (16: +16 %, 384: +18 %)

// First tile (group-major index) whose cost prefix is >= w.
__device__ long long wgrad_first_tile(const int32_t* __restrict__ poff, int G, int per_g, long long w) {
  // cost prefix of group g's first tile: per_g * (poff[g] + g * kWgTileCost)
  auto gstart = [&](int g) { return (long long)per_g * ((long long)poff[g] + g * kWgTileCost); };
  int lo = 0, hi = G;                  // largest g in [0, G] with gstart(g) <= w
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (gstart(mid) <= w) lo = mid;
    else hi = mid - 1;
  }
  const int g = lo;
  if (g >= G) return (long long)G * per_g;
  const long long cost = (long long)(poff[g + 1] - poff[g]) + kWgTileCost;
  long long t = (w - gstart(g) + cost - 1) / cost;     // ceil
  if (t > per_g) t = per_g;
  return (long long)g * per_g + t;
}

__global__ __launch_bounds__(256, 1) void bwd_wgrad_kernel(BwdGemmParams p, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) bf16_t L0[512 * kBK];
  __shared__ __attribute__((aligned(1024))) bf16_t L1[512 * kBK];
  __shared__ int32_t s_poff[kMaxExperts + 1];   // G + 1 <= kMaxExperts + 1 group offsets
  const int per_g = tiles_m * tiles_n;
  const int G = p.G;
  // the group offsets live in LDS: reading them per tile then never waits on
  // the vector-memory counter, which the previous tile's stores still hold
  for (int i = threadIdx.x; i <= G; i += 256) s_poff[i] = p.poff[i];
  __syncthreads();
  const long long total = (long long)G * per_g;
  const long long W = (long long)per_g * ((long long)p.poff[G] + G * kWgTileCost);
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
  const long long t0 = xcd == 0 ? 0 : wgrad_first_tile(p.poff, G, per_g, W * xcd / 8);
  const long long t1 = xcd == 7 ? total : wgrad_first_tile(p.poff, G, per_g, W * (xcd + 1) / 8);
  // tile t -> group, tile row, tile column, first padded row, K steps.
  // Inside a group: strips of 4 tile rows walked column by column, so the 32
  // tiles an XCD runs together are 4 row blocks x 8 column blocks and share
  // 4 + 8 operand blocks from L2 (row-major order would share 1 + 32).
  // (all wave-uniform: the group index goes through readfirstlane so the
  // offsets come in by scalar loads, which do not wait behind the stores)
  auto tile_of = [&](long long t, int* g, int* tm, int* tn, int* kbeg, int* nK) {
    *g = __builtin_amdgcn_readfirstlane((int)(t / per_g));
    const int r = (int)(t - (long long)*g * per_g);
    constexpr int GM = 4;
    const int strip = r / (GM * tiles_n);
    const int rs = r - strip * GM * tiles_n;
    const int gm = min(GM, tiles_m - strip * GM);
    *tm = strip * GM + rs % gm;
    *tn = rs / gm;
    *kbeg = __builtin_amdgcn_readfirstlane(s_poff[*g]);
    *nK = (__builtin_amdgcn_readfirstlane(s_poff[*g + 1]) - *kbeg) / kBK;
  };
  // Tiles of one K step (groups of <= 64 rows) are mostly store time (256 KB
  // of fp32 each).  When the next tile has one K step, its loads go out into
  // the other stage buffer before this tile's stores, so its MFMAs need not
  // wait for those stores to drain; the two buffers then swap roles.
  bf16_t* Lc = L0;
  bf16_t* Ln = L1;
  bool pre = false;
  for (long long t = t0 + slot; t < t1; t += nslots) {
    // retires a prefetch for this tile (issued before the previous tile's 64
    // stores per thread) before any LDS access; otherwise it does not wait
    wait_vmem_le<63>();
    int g, tm, tn, kbeg, nK;
    tile_of(t, &g, &tm, &tn, &kbeg, &nK);
    int nx[3] = {0, 0, 0};
    bool pf = false;
    if (t + nslots < t1 && tm * 256 + 256 <= p.M && tn * 256 + 256 <= p.N) {
      int g2, tm2, tn2, kbeg2, nK2;
      tile_of(t + nslots, &g2, &tm2, &tn2, &kbeg2, &nK2);
      if (nK2 == 1) {
        pf = true;
        nx[0] = tm2 * 256; nx[1] = tn2 * 256; nx[2] = kbeg2;
      }
    }
    bwd_tile<MODE_TN, 256>(p, g, tm * 256, 256, tn * 256, kbeg, nK, Lc, Ln, nullptr, 0, 0, pre, pf, nx[0], nx[1],
                           nx[2]);
    if (pf) {
      bf16_t* tmp = Lc;
      Lc = Ln;
      Ln = tmp;
    }
    pre = pf;
    lds_sync();                        // the next tile reads or refills the LDS stages
  }
}

hipError_t launch_bwd_rows(int mode, const BwdGemmParams& p, hipStream_t s) {
  const int bn = mode == MODE_GU ? 128 : 256;
  const int n_tiles = (p.N + bn - 1) / bn;
  const int gh = grouped_grid(p.maxQ, n_tiles);   // heavy tiles, then light tiles
  const int ks = mode == MODE_GU ? 1 : (p.ksplit > 1 ? p.ksplit : 1);
  const dim3 gl(grouped_grid(p.G, n_tiles), ks);
  // many expert groups: the light launch on the second stream, joined back
  // before anything that reads its rows (as in the forward's grouped GEMMs)
  SideStream* side = p.G >= kConcurrentMinGroups ? side_stream(s) : nullptr;
  const hipStream_t sl = side ? side->s : s;
  hipError_t e = hipSuccess;
  if (side) {
    if ((e = hipEventRecord(side->fork, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(sl, side->fork, 0)) != hipSuccess) return e;
  }
  if (mode == MODE_GU) {
    bwd_rows_kernel<MODE_GU, 1><<<gh, 256, 0, s>>>(p);
    bwd_rows_kernel<MODE_GU, 2><<<gl, 256, 0, sl>>>(p);
  } else if (mode == MODE_NTS) {
    bwd_rows_kernel<MODE_NTS, 1><<<gh, 256, 0, s>>>(p);
    bwd_rows_kernel<MODE_NTS, 2><<<gl, 256, 0, sl>>>(p);
  } else {
    bwd_rows_kernel<MODE_NT, 1><<<gh, 256, 0, s>>>(p);
    bwd_rows_kernel<MODE_NT, 2><<<gl, 256, 0, sl>>>(p);
  }
  e = hipGetLastError();
  if (side && e == hipSuccess) {
    if ((e = hipEventRecord(side->join, sl)) == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
  }
  if (e != hipSuccess || ks == 1) return e;
  return launch_down_split_reduce(p.sched, p.maxQ, p.G, n_tiles, p.N, ks, p.part_slots, p.part, p.C0, s);
}

hipError_t launch_bwd_wgrad(const BwdGemmParams& p, hipStream_t s) {
  const int tm = (p.M + 255) / 256, tn = (p.N + 255) / 256;
  // persistent: one work-group per CU (their LDS allows one), dealt round-robin to the 8 XCDs
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int grid = 8 * ((cus + 7) / 8);
  bwd_wgrad_kernel<<<grid, 256, 0, s>>>(p, tm, tn);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 layers: the same products in fp32 with SIMT FMA (64 x 64 output tiles,
// 256 threads of 4 x 4 outputs, 16-wide K steps staged in LDS; each output one
// FMA chain in K order).  Groups are padded to 64 rows, so a 64-row tile of the
// padded row space lies inside one group.
// ---------------------------------------------------------------------------
namespace {

__device__ __forceinline__ void f32_tile_fma(const float (*As)[68], const float (*Bs)[68], int tx, int ty,
                                             float (*acc)[4]) {
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&As[kk][4 * ty]);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&Bs[kk][4 * tx]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __fmaf_rn(a[i], b[j], acc[i][j]);
  }
}

// Row products: C[p, n] = sum_k A(p, k) B_g(k, n) over the padded rows p of
// group g, A rows K-contiguous; B_g(k, n) = B[k ldb + n] (b_kc false) or
// B[n ldb + k] (b_kc true), the shared expert's matrix for g = E; with A1 the
// K range splits at K1 into (A0, B0) and (A1, B1).
__global__ __launch_bounds__(256) void bwd_rows_f32_kernel(BwdF32Params p) {
  __shared__ __attribute__((aligned(16))) float As[16][68];
  __shared__ __attribute__((aligned(16))) float Bs[16][68];
  const int row0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  if (row0 >= p.poff[p.G]) return;
  int lo = 0, hi = p.G;                             // the group holding row0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.poff[mid] <= row0) lo = mid;
    else hi = mid;
  }
  const bool shared = lo == p.E;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int part = 0; part < (p.A1 ? 2 : 1); ++part) {
    const float* A = part ? p.A1 : p.A0;
    const float* B = part ? (shared ? p.Bs1 : p.B1 + (size_t)lo * p.bgs) : (shared ? p.Bs0 : p.B0 + (size_t)lo * p.bgs);
    const int K = p.A1 ? (part ? p.K - p.K1 : p.K1) : p.K;
    for (int k0 = 0; k0 < K; k0 += 16) {
      {                                             // A: row tid / 4, K columns 4 (tid % 4) .. + 3
        const int r = tid >> 2, c = 4 * (tid & 3);
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(A + (size_t)(row0 + r) * p.lda + k0 + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) As[c + j][r] = v[j];
      }
      if (p.b_kc) {                                 // B: column tid / 4, K rows 4 (tid % 4) .. + 3
        const int n = tid >> 2, c = 4 * (tid & 3);
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(B + (size_t)(n0 + n) * p.ldb + k0 + c);
#pragma unroll
        for (int j = 0; j < 4; ++j) Bs[c + j][n] = v[j];
      } else {                                      // B: K row tid / 16, columns 4 (tid % 16) .. + 3
        const int kk = tid >> 4, n = 4 * (tid & 15);
        *reinterpret_cast<f32x4_t*>(&Bs[kk][n]) = *reinterpret_cast<const f32x4_t*>(B + (size_t)(k0 + kk) * p.ldb + n0 + n);
      }
      __syncthreads();
      f32_tile_fma(As, Bs, tx, ty, acc);
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<f32x4_t*>(p.C + (size_t)(row0 + 4 * ty + i) * p.N + n0 + 4 * tx) =
        f32x4_t{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
}

// Weight gradients: C_g[m, n] = sum over group g's padded rows r of
// A[r lda + m] B[r ldb + n] (group E: the shared expert's Cs); an empty group
// writes zeros.
__global__ __launch_bounds__(256) void bwd_wgrad_f32_kernel(BwdF32Params p) {
  __shared__ __attribute__((aligned(16))) float As[16][68];
  __shared__ __attribute__((aligned(16))) float Bs[16][68];
  const int n0 = blockIdx.x * 64, m0 = blockIdx.y * 64, g = blockIdx.z;
  const int r0 = p.poff[g], r1 = p.poff[g + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int kk = tid >> 4, c4 = 4 * (tid & 15);
  float acc[4][4] = {};
  for (int k0 = r0; k0 < r1; k0 += 16) {
    *reinterpret_cast<f32x4_t*>(&As[kk][c4]) = *reinterpret_cast<const f32x4_t*>(p.A0 + (size_t)(k0 + kk) * p.lda + m0 + c4);
    *reinterpret_cast<f32x4_t*>(&Bs[kk][c4]) = *reinterpret_cast<const f32x4_t*>(p.B0 + (size_t)(k0 + kk) * p.ldb + n0 + c4);
    __syncthreads();
    f32_tile_fma(As, Bs, tx, ty, acc);
    __syncthreads();
  }
  float* C = g == p.E ? p.Cs : p.C + (size_t)g * p.cstride;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<f32x4_t*>(C + (size_t)(m0 + 4 * ty + i) * p.N + n0 + 4 * tx) =
        f32x4_t{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
}

}  // namespace

hipError_t launch_bwd_rows_f32(const BwdF32Params& p, long pmax, hipStream_t s) {
  if (pmax <= 0) return hipSuccess;
  bwd_rows_f32_kernel<<<dim3(p.N / 64, (unsigned)(pmax / 64)), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_bwd_wgrad_f32(const BwdF32Params& p, hipStream_t s) {
  bwd_wgrad_f32_kernel<<<dim3(p.N / 64, p.M / 64, p.G), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace moe
