// Grouped SwiGLU expert FFN on gfx950.
//
// Pages: "MoE Model Architectures", Mixtral "Expert FFN" (w2(silu(w1 x) *
// w3 x), no biases) and "Sparse MoE Block" (only experts that received
// tokens run); DeepSeek-V3 "DeepSeekMoE Architecture" (an always-on shared
// expert); "Faster writing: run only the chosen experts; uncap the large
// profile" (read only the chosen experts' weights).
//
// Two kernels per call, both driven by a device-side tile schedule built from
// the expert offsets (so no count is read back to the host):
//   gate/up: H[r, n] = silu(A[r] . Wg[:, n]) * (A[r] . Wu[:, n]), A[r] the x
//            row of the token owning permuted row r;  H is bf16 (fp32 for the
//            fp32 layer)
//   down:    Y[r, n] = H[r] . Wd[:, n]  (fp32)
//
// Tiles are up to 256 permuted rows x 256 "B columns" (the gate/up GEMM
// takes 128 gate and the same 128 up columns), 256 threads (4 waves),
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The weights stay in their
// stored layout ([K, N], N contiguous) in LDS and reach the MFMA as
// K-contiguous fragments through gfx950's transposing LDS reads
// (ds_read_b64_tr_b16); the activation rows are K-contiguous already.
//   bf16 weights (gemm_dl_kernel): A and B move global -> LDS directly
//     (global_load_lds, 16 bytes per lane) into a ring of LDS stages, with
//     the LDS swizzles applied on the source side.
//   fp8 e4m3fn weights (the same kernel, F8): the codes move global -> LDS
//     the same way (half the bytes), ds_read_b64_tr_b8 gathers them
//     K-contiguous and they widen to bf16 (exact) in registers; the
//     per-output-channel scales multiply the accumulators in the epilogue.
//   fp32 layer: SIMT fp32 FMA, 64 x 64 tiles (gemm_f32_kernel), or 64 x 16 tiles
//     with K split over the threads when the layer has few tiles
//     (gemm_f32_narrow_kernel).
// Every LDS layout was checked against the bank-conflict counter on gfx950
// (16-lane passes for 16-byte reads, 32-lane passes for 8-byte reads).
//
// Work-group ids are remapped so that consecutive tiles (same weight column
// tile, neighbouring row tiles of one expert) run on the same XCD and share
// its L2.  Each GEMM is two launches, full-height ("heavy") tiles and each
// expert's small last ("light") tile, whose body matches its rows (256, 128,
// 64 or 32); with 64 or more expert groups the light launch runs on a second
// stream beside the heavy one.  With bf16 weights a last tile is light only
// at <= 64 rows (64-row stages two deep, two work-groups per CU); last tiles
// of 65..128 rows run in the heavy launch with the 128-row body.  fp8 layers
// whose groups all fit 64 rows run one 64-row launch per GEMM.
#include <atomic>
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

struct GemmParams {
  const bf16_t* x;               // DUAL: activations [T, d]
  const int32_t* sorted_assign;  // DUAL: permuted row -> assignment
  const bf16_t* a_rows;          // !DUAL: H [rows, f]
  const void* W0;                // DUAL: gate [E, K, N]; !DUAL: down [E, K, N]
  const void* W1;                // DUAL: up
  const void* Ws0;               // shared expert matrices
  const void* Ws1;
  const float* s0;               // fp8 scales [E, N] (gate or down)
  const float* s1;               // fp8 scales up
  const float* ss0;
  const float* ss1;
  const int32_t* sched;
  int maxQ;
  int T, k, E, K, N;
  int shared_row0;               // T*k
  bf16_t* h_out;                 // DUAL output [rows, N]
  float* y_out;                  // !DUAL output [rows, N]
  float* y_part;                 // !DUAL light tiles split over K: parts 1.. [ksplit - 1][part_slots][128][256]
  int ksplit;                    // K parts of the down GEMM's light tiles (1: none)
  int part_slots;                // light-segment slots (groups x column tiles) covered by y_part
};

// LDS B tile: 64 K-rows x 256 output columns, N-contiguous as in global
// memory.  A transposing LDS read touches four consecutive K-rows (512 bytes
// apart, so the same banks) at 16 columns per 16-lane group; the column index
// is XOR-swizzled by 16 h(k), h(k) = (k & 3) | (k & 1) << 2, which puts the
// 4 rows x 2 neighbouring 16-lane groups on 8 distinct 32-byte bank segments.
__device__ __forceinline__ int bswz_key(int k) { return ((k & 3) << 4) | ((k & 1) << 6); }
__device__ __forceinline__ int bswz(int k, int n) { return k * 256 + (n ^ bswz_key(k)); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// MFMA B fragment (8 consecutive K of one output column per lane) from the
// N-contiguous LDS tile with two gfx950 transposing reads.  Within each group
// of 16 lanes, input lane x supplies a 4-element row R_x and output lane
// 4a + b receives R_a[b], R_{a+4}[b], R_{a+8}[b], R_{a+12}[b].
__device__ __forceinline__ bf16x8_t load_b_frag(const bf16_t* Bs, int kbase, int nbase, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int a = i & 3, j = i >> 2;
  const int n = nbase + 16 * (g & 1) + 4 * a;
  const int k0 = kbase + 8 * (g >> 1) + j;
  typedef __attribute__((address_space(3))) i16x4_t* lds_i16x4;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(Bs + bswz(k0, n)));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(Bs + bswz(k0 + 4, n)));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// fp8 LDS B tile: BK K-rows x 256 output columns of one byte, N-contiguous.
// The 16-byte column chunk of K-row k sits at chunk ^ bkey8(k): the eight
// K-rows one transposing read touches then fall on eight distinct chunks, and
// the neighbouring 16-lane group (the next 16 columns, odd chunks) on the other
// eight, so half a wave reads all 64 banks once.
__device__ __forceinline__ int bkey8(int k) { return (k & 7) << 1; }

// MFMA B fragment (8 consecutive K of one output column per lane, as bf16)
// from the fp8 tile with one gfx950 byte-transposing read: within each group
// of 16 lanes, input lane x supplies 8 bytes R_x and output lane 8a + b
// receives R_a[b], R_{a+2}[b], ..., R_{a+14}[b].  Input lane x = a + 2j
// therefore points at K-row kbase + j, columns c0 + 8a .. +7, and output lane
// y holds column c0 + y, K-rows kbase .. +7.  e4m3 codes widen to bf16
// exactly.
__device__ __forceinline__ bf16x8_t load_b_frag8(const unsigned char* Bs, int kbase, int nbase, int lane) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2_t* lds_i32x2;
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const int g = lane >> 4, x = lane & 15;
  const int n = nbase + 16 * (g & 1) + 8 * (x & 1);
  const int k = kbase + 8 * (g >> 1) + (x >> 1);
  const i32x2_t q = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (lds_i32x2)(Bs + k * 256 + ((((n >> 4) ^ bkey8(k)) << 4) | (n & 15))));
  const bf16x2_t c0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[0], 1.f, false);
  const bf16x2_t c1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[0], 1.f, true);
  const bf16x2_t c2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[1], 1.f, false);
  const bf16x2_t c3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)q[1], 1.f, true);
  const bf16x8_t v = {c0[0], c0[1], c1[0], c1[1], c2[0], c2[1], c3[0], c3[1]};
  return v;
}

// Work-groups per CU for a kernel whose LDS stages hold BM rows.
template <int BM> struct TileCfg {
  static constexpr int OCC = (BM == 64) ? 2 : 1;
};

// ---------------------------------------------------------------------------
// bf16 weights: operands move from global memory straight into LDS
// (global_load_lds, 16 bytes per lane), so no register staging and no LDS
// store instructions.  One such load fills 1 KB of LDS in lane order; the LDS
// swizzles are therefore applied on the source side: the lane that owns LDS
// chunk c fetches the global chunk that the swizzle maps to c.
//
// NST LDS stages of BK columns of K form a ring: the loads of step k + NST
// are issued as soon as every wave has finished reading step k's stage, so
// NST - 1 steps of MFMA work cover each load's latency.
// ---------------------------------------------------------------------------
// One output tile of at most BMV rows: waves 2 x 2 (128 rows x 128 B-columns
// each) for BMV = 256, 1 x 4 (BMV rows x 64 B-columns each) for 128 and 64.
// The LDS stages are sized for BMMAX rows.  F8: the weights are e4m3 codes with
// per-output-column fp32 scales; their LDS tile holds the codes (half the
// bytes of bf16), the fragment reads widen them to bf16 and the epilogue
// applies the column scales.
//
// K range: [k_lo, k_lo + nK BK).  A tile with kpart > 0 (light down tiles
// split over K) writes its fp32 block to y_part slot `slot` instead of Y.
template <bool DUAL, int BMV, int BMMAX, int BK, int NST, bool F8 = false>
__device__ __forceinline__ void dl_tile(const GemmParams& p, int g, int row0, int rows, int nt, bf16_t* L0,
                                        bf16_t* L1, bf16_t* L2, bf16_t* L3, int k_lo, int nK, int kpart = 0,
                                        int slot = 0) {
  constexpr int WM = (BMV >= 256) ? 2 : 1, WN = 4 / WM;
  constexpr int NMAT = DUAL ? 2 : 1;
  constexpr int BN_MAT = DUAL ? 128 : 256;
  constexpr int NI_MAT = BN_MAT / WN / 32;
  constexpr int NI = NI_MAT * NMAT;
  constexpr int MI = BMV / WM / 32;
  constexpr int WROWS = BMV / WM;
  constexpr int CPR = BK / 8;                      // 16-byte chunks per A row
  constexpr int A_RPB = 64 / CPR;                  // A rows per 1 KB block
  constexpr int A_LD = BMV / A_RPB / 4;            // 1 KB A blocks per wave per step
  constexpr int B_RPB = F8 ? 4 : 2;                // K-rows per 1 KB B block
  constexpr int B_LD = BK / B_RPB / 4;             // 1 KB B blocks per wave per step
  constexpr int SUB = BK / 16;                     // 16-wide MFMA sub-steps per step
  constexpr int LDS_A = BMMAX * BK;                // B tile offset inside a stage
  constexpr int NMF = MI * NI;                     // MFMAs per sub-step
  constexpr int NDS = MI + (F8 ? 1 : 2) * NI;      // LDS fragment reads per sub-step
  constexpr int NVM = A_LD + B_LD;                 // global->LDS loads per step
  static_assert(SUB % 2 == 0 && NST >= 2 && NST <= 4 && A_LD >= 1 && B_LD % 2 == 0 && BMV <= BMMAX,
                "tile configuration");
  static_assert((NST - 1) * NVM < 64, "outstanding loads exceed the vmcnt range");
  // A light tile (<= 128 rows) is an expert's only row tile for its weight
  // columns, so its weight loads are streamed with the non-temporal policy;
  // full-height tiles keep the default so sibling row tiles hit in L2.
  constexpr int kBPolicy = (BMV <= 128) ? 2 : 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int n0 = nt * BN_MAT;
  const bool shared = (g == p.E);

  // ---- A sources: block b = wave + 4 i holds tile rows A_RPB b .. +A_RPB-1;
  // this lane fills row A_RPB b + lane / CPR, LDS chunk lane % CPR, i.e. the
  // global chunk aswz(row, lane % CPR).  Rows past the tile's valid rows read
  // its first row (never stored). ----
  const bf16_t* asrc[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = A_RPB * (wave + 4 * i) + lane / CPR;
    const int gc = aswz<CPR>(r, lane % CPR);
    const int grow = row0 + (r < rows ? r : 0);
    if (DUAL) {
      const int tok = shared ? (grow - p.shared_row0) : (p.sorted_assign[grow] / p.k);
      asrc[i] = p.x + (size_t)tok * p.K + k_lo + gc * 8;
    } else {
      asrc[i] = p.a_rows + (size_t)grow * p.K + k_lo + gc * 8;
    }
  }
  // ---- B sources: block b = B_LD wave + j holds K-rows B_RPB b .. +B_RPB-1.
  // bf16: this lane fills K-row 2 b + lane / 32, LDS chunk lane % 32, i.e.
  // tile column chunk (lane % 32) ^ (bswz_key(krow) / 8) of 8 columns; fp8:
  // K-row 4 b + lane / 16, LDS chunk lane % 16, i.e. tile column chunk
  // (lane % 16) ^ bkey8(krow) of 16 columns.  Tile columns 0..127 are gate,
  // 128..255 up for the gate/up GEMM.  Both keys depend only on krow's bits
  // that the parity of j fixes.  Columns past N read the last valid chunk
  // (never stored). ----
  constexpr int ES = F8 ? 1 : 2;                   // bytes per weight
  constexpr int CW = 16 / ES;                      // columns per 16-byte chunk
  const size_t goff = shared ? 0 : (size_t)g * (size_t)p.K * p.N;
  const size_t brow = (size_t)p.N * ES;
  const unsigned char* bsrc[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    int krow, gc;
    if constexpr (F8) {
      krow = 4 * (B_LD * wave + par) + (lane >> 4);
      gc = (lane & 15) ^ bkey8(krow);
    } else {
      krow = 2 * (B_LD * wave + par) + (lane >> 5);
      gc = (lane & 31) ^ (bswz_key(krow) >> 3);
    }
    constexpr int HALF = 128 / CW;                 // chunks per matrix in a gate/up tile
    const int mat = DUAL ? (gc >= HALF) : 0;
    int ncol = DUAL ? n0 + (gc % HALF) * CW : n0 + gc * CW;
    if (ncol > p.N - CW) ncol = p.N - CW;
    const void* Wbase = shared ? (mat ? p.Ws1 : p.Ws0) : (mat ? p.W1 : p.W0);
    bsrc[par] = (const unsigned char*)Wbase + (goff + (size_t)(k_lo + krow) * p.N + ncol) * ES;
  }

  auto issue = [&](bf16_t* L, int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(asrc[i] + k0), (lds_ptr_t)(L + (wave + 4 * i) * 512), 16, 0, 0);
    const size_t kb = (size_t)k0 * brow;
#pragma unroll
    for (int j = 0; j < B_LD; ++j)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(bsrc[j & 1] + kb + (size_t)(B_RPB * (j & ~1)) * brow),
                                       (lds_ptr_t)(L + LDS_A + (B_LD * wave + j) * 512), 16, 0, kBPolicy);
  };

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  auto frags = [&](const bf16_t* L, int ks, bf16x8_t* af, bf16x8_t* bfr) {
    const int chunk = ks * 2 + lhi;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * WROWS + mi * 32 + l32;
      af[mi] = *reinterpret_cast<const bf16x8_t*>(L + row * BK + aswz<CPR>(row, chunk) * 8);
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      int nbase;
      if (DUAL) {
        const int m_ = ni / NI_MAT, nl = ni % NI_MAT;
        nbase = m_ * 128 + wn * (128 / WN) + nl * 32;
      } else {
        nbase = wn * (256 / WN) + ni * 32;
      }
      if constexpr (F8) bfr[ni] = load_b_frag8(reinterpret_cast<const unsigned char*>(L + LDS_A), ks * 16, nbase, lane);
      else bfr[ni] = load_b_frag(L + LDS_A, ks * 16, nbase, lane);
    }
  };
  auto mfmas = [&](const bf16x8_t* af, const bf16x8_t* bfr) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
  };

  // Software pipeline over 16-wide K sub-steps: the fragments of sub-step
  // s + 1 are read while sub-step s's MFMAs run, across step boundaries too.
  // A step's last sub-step runs after the barrier that publishes the next
  // step's stage, so its MFMAs cover the first reads of the next step; by that
  // barrier every wave has also read all of the step's own stage, which is
  // then refilled NST steps ahead.  Past the end the refill repeats the last
  // step (never read again), so every wave issues the same number of loads per
  // step and the vmcnt thresholds below are exact.
  bf16x8_t fa0[MI], fb0[NI], fa1[MI], fb1[NI];
  auto stage = [&](auto S) -> bf16_t* {
    constexpr int s = decltype(S)::value % NST;
    if constexpr (s == 0) return L0;
    else if constexpr (s == 1) return L1;
    else if constexpr (s == 2) return L2;
    else return L3;
  };
  issue(L0, 0);
  issue(L1, min(1, nK - 1) * BK);
  if constexpr (NST > 2) issue(L2, min(2, nK - 1) * BK);
  if constexpr (NST > 3) issue(L3, min(3, nK - 1) * BK);
  wait_vmem_le<(NST - 1) * NVM>();
  __builtin_amdgcn_s_barrier();
  frags(L0, 0, fa0, fb0);

  auto step = [&](auto S, int k) {
    bf16_t* L = stage(S);
    const bf16_t* Ln = stage(std::integral_constant<int, decltype(S)::value + 1>{});
#pragma unroll
    for (int sub = 0; sub + 1 < SUB; ++sub) {
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
    issue(L, min(k + NST, nK - 1) * BK);
    frags(Ln, 0, fa0, fb0);
    mfmas(fa1, fb1);
    sched_interleave<NMF, NDS, NVM>();
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  int k = 0;
  for (; k + NST <= nK; k += NST) {
    step(I0{}, k);
    step(I1{}, k + 1);
    if constexpr (NST > 2) step(I2{}, k + 2);
    if constexpr (NST > 3) step(I3{}, k + 3);
  }
  if (k < nK) step(I0{}, k);
  if constexpr (NST > 2) if (k + 1 < nK) step(I1{}, k + 1);
  if constexpr (NST > 3) if (k + 2 < nK) step(I2{}, k + 2);
  wait_vmem_le<0>();

  // ---- epilogue ----
  if constexpr (DUAL) {
    // H = bf16(silu(gate) * up).  Register v holds row 8 (v / 4) + 4 lhi + v % 4
    // of column l32; neighbouring lanes (columns c, c + 1) swap halves so that
    // the even lane stores (row v, columns c..c+1) and the odd lane (row v + 1,
    // columns c - 1..c) as one dword each.
    const bool odd = lane & 1;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int nl = 0; nl < NI_MAT; ++nl) {
        const int c2 = n0 + wn * (BN_MAT / WN) + nl * 32 + (l32 & ~1);
        if (c2 >= p.N) continue;
        float sc0 = 1.f, sc1 = 1.f;                // this lane's column scales (fp8)
        if constexpr (F8) {
          const size_t c = (shared ? 0 : (size_t)g * p.N) + c2 + (l32 & 1);
          sc0 = (shared ? p.ss0 : p.s0)[c];
          sc1 = (shared ? p.ss1 : p.s1)[c];
        }
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          float hv[2];
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const float g = acc[mi][nl][v + i] * sc0;
            hv[i] = g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * (acc[mi][nl + NI_MAT][v + i] * sc1);
          }
          const uint32_t own = pack_bf16x2(hv[0], hv[1]);
          const uint32_t x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0xB1, 0xF, 0xF, false);
          const uint32_t out = __builtin_amdgcn_perm(x, own, sel);
          const int r = wm * WROWS + mi * 32 + (v >> 2) * 8 + lhi * 4 + (v & 3) + (odd ? 1 : 0);
          if (r < rows) *reinterpret_cast<uint32_t*>(p.h_out + (size_t)(row0 + r) * p.N + c2) = out;
        }
      }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int nl = 0; nl < NI_MAT; ++nl) {
        const int col = n0 + wn * (BN_MAT / WN) + nl * 32 + l32;
        if (col >= p.N) continue;
        float sc0 = 1.f;
        if constexpr (F8) sc0 = shared ? p.ss0[col] : p.s0[(size_t)g * p.N + col];
        // K part 0 (or no split): Y rows; parts 1..: this slot's 128 x 256 block
        float* out = kpart == 0 ? p.y_out + (size_t)row0 * p.N + col
                                : p.y_part + ((size_t)(kpart - 1) * p.part_slots + slot) * (128 * 256) + (col - n0);
        const size_t ostride = kpart == 0 ? (size_t)p.N : 256;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WROWS + mi * 32 + (v >> 2) * 8 + lhi * 4 + (v & 3);
          if (r < rows) out[(size_t)r * ostride] = F8 ? acc[mi][nl][v] * sc0 : acc[mi][nl][v];
        }
      }
    }
  }
}


// SEG 0: every tile of the schedule (bodies of 256, 128 or 64 rows);
// SEG 1: the heavy segment only (tiles of more than 128 rows, 256-row body);
// SEG 2: the light segment only (an expert's last tile of at most 128 rows),
//        with LDS stages sized for 128 rows so that three of them fit and two
//        steps of loads are in flight: light tiles do little MFMA work per
//        stage and are bound by load latency.
template <bool DUAL, int BMMAX, int BK, int NST, int SEG = 0, bool F8 = false>
__global__ __launch_bounds__(256, TileCfg<BMMAX>::OCC) void gemm_dl_kernel(GemmParams p) {
  constexpr int LDS_S = BMMAX * BK + (F8 ? 128 : 256) * BK;   // bf16 elements per stage
  __shared__ __attribute__((aligned(1024))) bf16_t L0[LDS_S];
  __shared__ __attribute__((aligned(1024))) bf16_t L1[LDS_S];
  __shared__ __attribute__((aligned(1024))) bf16_t L2[NST > 2 ? LDS_S : 8];
  __shared__ __attribute__((aligned(1024))) bf16_t L3[NST > 3 ? LDS_S : 8];
  constexpr int BN_MAT = DUAL ? 128 : 256;
  const int n_tiles = (p.N + BN_MAT - 1) / BN_MAT;
  int g, row0, rows, nt, slot = 0;
  if (!decode_tile<SEG>(p.sched, p.maxQ, p.E, n_tiles, &g, &row0, &rows, &nt, &slot)) return;
  // light down tiles may be split over K (blockIdx.y = K part)
  const int kparts = (!DUAL && SEG == 2) ? p.ksplit : 1;
  const int kpart = (!DUAL && SEG == 2) ? (int)blockIdx.y : 0;
  const int nK = p.K / BK / kparts;
  const int k_lo = kpart * nK * BK;
  // An expert's last row tile is usually partial: run it with a body whose
  // MFMA work matches its rows (<= 64, <= 128) instead of the full height.
  if constexpr (SEG == 1) {
    // heavy tiles: full ones, and last tiles above the light bound (65..128
    // rows for bf16 weights take the 128-row body)
    if (F8 || rows > 128) dl_tile<DUAL, 256, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
    else dl_tile<DUAL, 128, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
  } else if constexpr (BMMAX >= 256) {
    if (rows > 128) dl_tile<DUAL, 256, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
    else if (rows > 64) dl_tile<DUAL, 128, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
    else if (rows > 32) dl_tile<DUAL, 64, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
    else dl_tile<DUAL, 32, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
  } else if constexpr (BMMAX >= 128) {
    if (rows > 64) dl_tile<DUAL, 128, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
    else if (rows > 32) dl_tile<DUAL, 64, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
    else dl_tile<DUAL, 32, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
  } else {
    if (rows > 32) dl_tile<DUAL, BMMAX, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
    else dl_tile<DUAL, 32, BMMAX, BK, NST, F8>(p, g, row0, rows, nt, L0, L1, L2, L3, k_lo, nK, kpart, slot);
  }
}

// ---------------------------------------------------------------------------
// fp32 layer: SIMT grouped GEMM, 64 rows x 64 columns per tile, fp32 FMA.
// ---------------------------------------------------------------------------
struct GemmParamsF32 {
  const float* x;
  const int32_t* sorted_assign;
  const float* a_rows;
  const float *W0, *W1, *Ws0, *Ws1;
  const int32_t* sched;
  int maxQ, T, k, E, K, N, shared_row0;
  float* h_out;
  float* y_out;
};

template <bool DUAL>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParamsF32 p) {
  // 64-wide K steps, 16-byte loads (4 A and 4 B vectors per matrix per
  // thread), and the next step's loads issued into registers before the
  // current step's FMAs, so each step's memory latency hides behind the
  // previous step's arithmetic.  K and N are multiples of 64.
  constexpr int BM = 64, BN = 64, BK = 64;
  __shared__ float As[BK][BM + 4];
  __shared__ __attribute__((aligned(16))) float Bs[DUAL ? 2 : 1][BK][BN + 4];
  const int n_tiles = (p.N + BN - 1) / BN;
  int g, row0, rows, nt;
  if (!decode_tile(p.sched, p.maxQ, p.E, n_tiles, &g, &row0, &rows, &nt)) return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int n0 = nt * BN;
  const bool shared = (g == p.E);
  const size_t goff = shared ? 0 : (size_t)g * p.K * p.N;
  const float* B0 = (shared ? p.Ws0 : p.W0 + goff);
  const float* B1 = DUAL ? (shared ? p.Ws1 : p.W1 + goff) : nullptr;
  // A: tile rows ty + 16 i, K columns 4 tx .. 4 tx + 3 of each step; rows
  // past the tile's rows read its first row and stage zeros.  B: K-rows
  // ty + 16 i of the step, columns n0 + 4 tx .. + 3.
  const float* arow[4];
  bool alive[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty + 16 * i;
    alive[i] = r < rows;
    const int grow = row0 + (alive[i] ? r : 0);
    if (DUAL) {
      const int tok = shared ? (grow - p.shared_row0) : (p.sorted_assign[grow] / p.k);
      arow[i] = p.x + (size_t)tok * p.K + 4 * tx;
    } else {
      arow[i] = p.a_rows + (size_t)grow * p.K + 4 * tx;
    }
  }
  const float* b0p = B0 + (size_t)ty * p.N + n0 + 4 * tx;
  const float* b1p = DUAL ? B1 + (size_t)ty * p.N + n0 + 4 * tx : nullptr;
  float acc0[4][4], acc1[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc0[i][j] = acc1[i][j] = 0.f;
  const int rpt = rows <= 16 ? 1 : rows <= 32 ? 2 : 4;   // rows per thread
  auto kloop = [&](auto RC) {
    constexpr int R = decltype(RC)::value;
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[R], b0[4], b1[4];
#pragma unroll
      for (int i = 0; i < R; ++i) a[i] = As[kk][ty * R + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        b0[j] = Bs[0][kk][tx * 4 + j];
        if (DUAL) b1[j] = Bs[DUAL ? 1 : 0][kk][tx * 4 + j];
      }
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc0[i][j] = __fmaf_rn(a[i], b0[j], acc0[i][j]);
          if (DUAL) acc1[i][j] = __fmaf_rn(a[i], b1[j], acc1[i][j]);
        }
    }
  };
  f32x4_t va[4], vb0[4], vb1[DUAL ? 4 : 1];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) va[i] = *reinterpret_cast<const f32x4_t*>(arow[i] + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t o = (size_t)(k0 + 16 * i) * p.N;
      vb0[i] = *reinterpret_cast<const f32x4_t*>(b0p + o);
      if (DUAL) vb1[DUAL ? i : 0] = *reinterpret_cast<const f32x4_t*>(b1p + o);
    }
  };
  load(0);
  for (int k0 = 0; k0 < p.K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) As[4 * tx + j][ty + 16 * i] = alive[i] ? va[i][j] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f32x4_t*>(&Bs[0][ty + 16 * i][4 * tx]) = vb0[i];
      if (DUAL) *reinterpret_cast<f32x4_t*>(&Bs[DUAL ? 1 : 0][ty + 16 * i][4 * tx]) = vb1[DUAL ? i : 0];
    }
    __syncthreads();
    if (k0 + BK < p.K) load(k0 + BK);                 // next step's loads fly during this step's FMAs
    // R rows x 4 columns per thread (rows ty R .. ty R + R - 1): R = 1 for
    // tiles of at most 16 rows, 2 for at most 32, else 4, so all four waves
    // do useful work
    if (rpt == 1) kloop(std::integral_constant<int, 1>{});
    else if (rpt == 2) kloop(std::integral_constant<int, 2>{});
    else kloop(std::integral_constant<int, 4>{});
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = i < rpt ? ty * rpt + i : rows;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      const size_t o = (size_t)(row0 + r) * p.N + col;
      if (DUAL) p.h_out[o] = silu_f(acc0[i][j]) * acc1[i][j];
      else p.y_out[o] = acc0[i][j];
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 layer, few tiles: 64-row x 16-column tiles whose K range is split over
// the 256 threads as 16 columns x 16 K parts.  Small fp32 layers (a few rows
// per expert) give the 64 x 64 kernel fewer work-groups than CUs, each with a
// long dependent K loop in which every B value read from LDS feeds only a
// handful of rows; here four times as many work-groups each run a quarter of
// the columns, a thread reads its own column of B straight from memory
// (16 lanes -> 64 contiguous bytes) and the tile's A rows come from LDS as
// broadcasts.  K moves in steps of 128 (8 per part; a last step of 64 gives 4),
// the next step's loads in flight during the current step's FMAs.  The 16 part
// sums of each output are added in part order through LDS (deterministic);
// the gate/up GEMM applies SwiGLU to the two finished sums.
// ---------------------------------------------------------------------------
template <bool DUAL, int R>
__device__ __forceinline__ void f32_narrow_tile(const GemmParamsF32& p, int g, int row0, int rows, int nt,
                                                float* As /* LDS [64][132] */) {
  constexpr int NMAT = DUAL ? 2 : 1;
  constexpr int KS = 128, LDA = KS + 4;
  constexpr int NA = R / 8;                        // A float4 loads per thread per step
  const int tid = threadIdx.x;
  const int c = tid & 15, part = tid >> 4;
  const int n0 = nt * 16;
  const bool shared = (g == p.E);
  const size_t goff = shared ? 0 : (size_t)g * p.K * p.N;
  const float* Bm[NMAT];
  Bm[0] = (shared ? p.Ws0 : p.W0 + goff) + n0 + c;
  if (DUAL) Bm[DUAL ? 1 : 0] = (shared ? p.Ws1 : p.W1 + goff) + n0 + c;
  // A: load i of this thread covers tile row tid / 32 + 8 i, float4 tid % 32
  // of the step; rows past the tile's rows read its first row (never stored)
  const float* arow[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = tid / 32 + 8 * i;
    const int grow = row0 + (r < rows ? r : 0);
    if (DUAL) {
      const int tok = shared ? (grow - p.shared_row0) : (p.sorted_assign[grow] / p.k);
      arow[i] = p.x + (size_t)tok * p.K + 4 * (tid % 32);
    } else {
      arow[i] = p.a_rows + (size_t)grow * p.K + 4 * (tid % 32);
    }
  }
  f32x4_t va[NA];
  float vb[NMAT][8];
  // loads of the step at k0 (kp = 8 values per part, 4 on a last step of 64)
  auto load = [&](int k0, int kp) {
    const bool full = kp == 8;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      va[i] = (full || (tid % 32) < 16) ? *reinterpret_cast<const f32x4_t*>(arow[i] + k0) : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        vb[m][j] = (j < kp) ? Bm[m][(size_t)(k0 + part * kp + j) * p.N] : 0.f;
  };
  float acc[NMAT][R];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[m][r] = 0.f;
  int kp = p.K >= KS ? 8 : 4;
  load(0, kp);
  for (int k0 = 0; k0 < p.K; k0 += KS) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
      *reinterpret_cast<f32x4_t*>(As + (tid / 32 + 8 * i) * LDA + 4 * (tid % 32)) = va[i];
    float b[NMAT][8];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) b[m][j] = vb[m][j];
    const int kcur = kp;
    __syncthreads();
    const int kn = k0 + KS;
    if (kn < p.K) {
      kp = p.K - kn >= KS ? 8 : 4;
      load(kn, kp);                                // next step's loads fly during this step's FMAs
    }
    // this part's K values of the step: LDS columns part * kcur .. + kcur - 1
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1 && kcur == 4) break;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const f32x4_t a4 = *reinterpret_cast<const f32x4_t*>(As + r * LDA + part * kcur + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int m = 0; m < NMAT; ++m) acc[m][r] = __fmaf_rn(a4[j], b[m][4 * h + j], acc[m][r]);
      }
    }
    __syncthreads();
  }
  // part sums through LDS, 16 rows at a time: red[part][m][row][col]
  float* red = As;
#pragma unroll
  for (int r0 = 0; r0 < R; r0 += 16) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((part * NMAT + m) * 16 + r) * 16 + c] = acc[m][r0 + r];
    __syncthreads();
    const int rr = tid >> 4;                       // output row r0 + rr, column c
    float sum[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      sum[m] = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) sum[m] += red[((q * NMAT + m) * 16 + rr) * 16 + c];
    }
    const int r = r0 + rr;
    if (r < rows) {
      const size_t o = (size_t)(row0 + r) * p.N + n0 + c;
      if (DUAL) p.h_out[o] = silu_f(sum[0]) * sum[DUAL ? 1 : 0];
      else p.y_out[o] = sum[0];
    }
    __syncthreads();
  }
}

template <bool DUAL>
__global__ __launch_bounds__(256) void gemm_f32_narrow_kernel(GemmParamsF32 p) {
  __shared__ __attribute__((aligned(16))) float As[64 * 132];
  const int n_tiles = p.N / 16;
  int g, row0, rows, nt;
  if (!decode_tile(p.sched, p.maxQ, p.E, n_tiles, &g, &row0, &rows, &nt)) return;
  if (rows <= 16) f32_narrow_tile<DUAL, 16>(p, g, row0, rows, nt, As);
  else if (rows <= 32) f32_narrow_tile<DUAL, 32>(p, g, row0, rows, nt, As);
  else f32_narrow_tile<DUAL, 64>(p, g, row0, rows, nt, As);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// direct-to-LDS bf16 kernels: K columns per step and LDS ring depth.
// Measured on MI355X (Mixtral prefill and fine-grained gate/up): 64 x 2 beats
// 32 x 3 and 32 x 4 by 2-4%; the loads are not latency-bound at two stages.
constexpr int kDlBK = 64;
constexpr int kDlNST = 2;

SideStream* side_stream(hipStream_t caller) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  thread_local SideStream ss[64];
  SideStream& r = ss[dev];
  if (r.bad) return nullptr;
  if (!r.s) {
    // creating a stream or an event while a graph is being captured is not
    // allowed (and may end the capture): such a call stays on one stream
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &st) != hipSuccess || st != hipStreamCaptureStatusNone) return nullptr;
    if (hipStreamCreateWithFlags(&r.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&r.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&r.join, hipEventDisableTiming) != hipSuccess) {
      r.bad = true;
      return nullptr;
    }
  }
  return &r;
}

static int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0, c = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if ((c = cached[dev].load(std::memory_order_relaxed)) > 0) return c;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) return 256;
  cached[dev].store(c, std::memory_order_relaxed);
  return c;
}

// 64-row fp8 tiles: three LDS stages (72 KB) fit two work-groups per CU, two
// stages (48 KB) fit three.  The tiles (at most one per group and column
// tile) are equal, so the depth whose work-group slots they fill best (fewest
// idle slots in the last round) is taken; three stages on a tie.
static bool small_f8_two_stages(int n_wg) {
  const long cus = device_cus();
  auto fill = [&](int per_cu) {
    const long slots = cus * per_cu;
    const long rounds = (n_wg + slots - 1) / slots;
    return (double)n_wg / (double)(rounds * slots);
  };
  return fill(3) > fill(2);
}

// The down GEMM's light tiles (an expert's last <= 128 rows) run after all of
// its heavy tiles.  When there are few of them (groups x column tiles <= 256,
// e.g. 8 Mixtral experts x 16) that launch leaves most CUs idle for a whole
// K loop, so each light tile is split into up to 4 K parts on as many
// work-groups; part 0 writes Y, the others fp32 blocks that a small kernel
// then adds to Y in part order (deterministic).
int grouped_down_ksplit(int d, int f, int E, int has_shared, int wkind, int act_f32) {
  if (act_f32) return 1;
  const int slots = (E + (has_shared ? 1 : 0)) * ((d + 255) / 256);
  if (slots > 256) return 1;
  const int bk = (wkind == W_MX || wkind == W_MX4) ? 128 : kDlBK;     // K per LDS stage of the light kernel
  for (int ks : {4, 2})
    if (f % (ks * bk) == 0) return ks;
  return 1;
}

size_t grouped_down_part_bytes(int d, int f, int E, int has_shared, int wkind, int act_f32) {
  const int ks = grouped_down_ksplit(d, f, E, has_shared, wkind, act_f32);
  const size_t slots = (size_t)(E + (has_shared ? 1 : 0)) * ((d + 255) / 256);
  return (size_t)(ks - 1) * slots * 128 * 256 * sizeof(float);
}

// Y[rows of light slot, its 256 columns] += parts 1 .. ksplit - 1, in order.
// Work-group (slot, 16-row block); each thread owns one column and issues the
// loads of all its 16 rows (clamped, so none waits behind a branch) before
// adding.
constexpr int kReduceRows = 16;
__global__ __launch_bounds__(256) void down_split_reduce_kernel(const int32_t* __restrict__ sched, int maxQ, int E,
                                                                int n_tiles, int N, int ksplit, int part_slots,
                                                                const float* __restrict__ part,
                                                                float* __restrict__ y) {
  const int slot = blockIdx.x;
  if (slot >= sched[1] * n_tiles) return;
  const int pt = slot / n_tiles, nt = slot - pt * n_tiles;
  const int32_t* ls = sched + kSchedHead + 4 * maxQ + (E + 1) + 3 * pt;
  const int row0 = ls[1], rows = ls[2];
  const int rb = blockIdx.y * kReduceRows;
  if (rb >= rows) return;
  const int c = threadIdx.x, col = nt * 256 + c;
  if (col >= N) return;
  float v[kReduceRows];
#pragma unroll
  for (int i = 0; i < kReduceRows; ++i) v[i] = y[(size_t)(row0 + min(rb + i, rows - 1)) * N + col];
  for (int kp = 1; kp < ksplit; ++kp) {
    const float* pp = part + ((size_t)(kp - 1) * part_slots + slot) * (128 * 256) + c;
    float w[kReduceRows];
#pragma unroll
    for (int i = 0; i < kReduceRows; ++i) w[i] = pp[min(rb + i, rows - 1) * 256];
#pragma unroll
    for (int i = 0; i < kReduceRows; ++i) v[i] += w[i];
  }
#pragma unroll
  for (int i = 0; i < kReduceRows; ++i)
    if (rb + i < rows) y[(size_t)(row0 + rb + i) * N + col] = v[i];
}

hipError_t launch_down_split_reduce(const int32_t* sched, int maxQ, int E, int n_tiles, int N, int ksplit,
                                    int part_slots, const float* part, float* y, hipStream_t s) {
  down_split_reduce_kernel<<<dim3(part_slots, 128 / kReduceRows), 256, 0, s>>>(sched, maxQ, E, n_tiles, N, ksplit,
                                                                               part_slots, part, y);
  return hipGetLastError();
}

static int pick_bm(const GroupedArgs& a) {
  if (a.act_f32) return 64;
  // bf16 and fp8 weights: 256-row tiles, whose small last tiles run 64/128-row
  // bodies.  Measured on MI355X, this also wins for skewed fine-grained loads
  // (256 experts of 0..1507 rows): fewer row tiles re-read each expert's weights.
  return 256;
}

int grouped_max_row_tiles(int routed_rows, int T, int E, int has_shared, int BM) {
  int q = routed_rows / BM + (routed_rows < E ? routed_rows : E);
  if (has_shared) q += (T + BM - 1) / BM;
  return q;
}

size_t grouped_sched_ints(int routed_rows, int T, int E, int has_shared) {
  // enough for the smallest tile height used (64 rows)
  return kSchedHead + 4 * (size_t)grouped_max_row_tiles(routed_rows, T, E, has_shared, 64) + 4 * (size_t)(E + 1) + 16;
}

// Work-groups: per XCD, enough slots for both schedule segments.  With
// QH + QL <= maxQ row tiles, ceil(QH n / 8) + ceil(QL n / 8) <= ceil(maxQ n / 8) + 2.
int grouped_grid(int maxQ, int n_tiles) {
  const long per = ((long)maxQ * n_tiles + 7) / 8 + 2;
  return (int)(8 * per);
}

// bf16 weights: a group's last tile is light only at <= 64 rows (run by the
// 64-row light kernel, two work-groups per CU); last tiles of 65..128 rows
// join the heavy launch with its 128-row body.
constexpr int kBf16LightMax = 64;

SchedSpec grouped_sched_spec(const GroupedArgs& a) {
  const int BM = (a.wkind == W_MX || a.wkind == W_MX4) ? 256 : pick_bm(a);
  const int lm = (a.wkind == W_BF16 && !a.act_f32) ? kBf16LightMax : 0;
  return SchedSpec{a.sched, BM, a.has_shared ? a.T : 0, a.routed_rows,
                   grouped_max_row_tiles(a.routed_rows, a.T, a.E, a.has_shared, BM), lm};
}

hipError_t launch_grouped_ffn(const GroupedArgs& a, hipStream_t s) {
  if (a.wkind == W_MX || a.wkind == W_MX4) return launch_grouped_ffn_mx(a, s);
  const SchedSpec sp = grouped_sched_spec(a);
  const int maxQ = sp.maxQ;
  const int shared_row0 = a.routed_rows;
  hipError_t err = hipSuccess;
  if (!a.sched_ready &&
      (err = launch_tile_schedule(a.offsets, a.E, sp.BM, sp.shared_rows, shared_row0, maxQ, a.sched, s,
                                  sp.light_max)) != hipSuccess)
    return err;

  if (a.act_f32) {
    GemmParamsF32 p{};
    p.x = (const float*)a.x;
    p.sorted_assign = a.sorted_assign;
    p.sched = a.sched;
    p.maxQ = maxQ;
    p.T = a.T; p.k = a.assign_div; p.E = a.E; p.shared_row0 = shared_row0;
    // a GEMM whose 64 x 64 tiles (at most maxQ x N / 64) would not give every
    // CU a work-group runs the 16-column kernel with its K split over threads
    const auto narrow = [&](int N) { return (long)maxQ * (N / 64) < device_cus(); };
    // gate/up
    p.W0 = (const float*)a.w.Wg; p.W1 = (const float*)a.w.Wu;
    p.Ws0 = (const float*)a.w.Wsg; p.Ws1 = (const float*)a.w.Wsu;
    p.K = a.d; p.N = a.f;
    p.h_out = (float*)a.h;
    const bool ng = narrow(a.f);
    const dim3 gg(grouped_grid(maxQ, ng ? a.f / 16 : (a.f + 63) / 64));
    const void* kg = ng ? (const void*)gemm_f32_narrow_kernel<true> : (const void*)gemm_f32_kernel<true>;
    if (a.ev_begin || a.ev_end) {
      if (ng) hipExtLaunchKernelGGL(gemm_f32_narrow_kernel<true>, gg, dim3(256), 0, s, a.ev_begin, a.ev_end, 0, p);
      else hipExtLaunchKernelGGL(gemm_f32_kernel<true>, gg, dim3(256), 0, s, a.ev_begin, a.ev_end, 0, p);
    } else {
      void* args[] = {&p};
      if ((err = hipLaunchKernel(kg, gg, dim3(256), args, 0, s)) != hipSuccess) return err;
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // down
    GemmParamsF32 q = p;
    q.a_rows = (const float*)a.h;
    q.W0 = (const float*)a.w.Wd; q.Ws0 = (const float*)a.w.Wsd;
    q.W1 = nullptr; q.Ws1 = nullptr;
    q.K = a.f; q.N = a.d;
    q.y_out = a.y;
    if (narrow(a.d)) gemm_f32_narrow_kernel<false><<<grouped_grid(maxQ, a.d / 16), 256, 0, s>>>(q);
    else gemm_f32_kernel<false><<<grouped_grid(maxQ, (a.d + 63) / 64), 256, 0, s>>>(q);
    return hipGetLastError();
  }

  GemmParams p{};
  p.x = (const bf16_t*)a.x;
  p.sorted_assign = a.sorted_assign;
  p.sched = a.sched;
  p.maxQ = maxQ;
  p.T = a.T; p.k = a.assign_div; p.E = a.E; p.shared_row0 = shared_row0;
  p.W0 = a.w.Wg; p.W1 = a.w.Wu; p.Ws0 = a.w.Wsg; p.Ws1 = a.w.Wsu;
  p.s0 = a.w.sg; p.s1 = a.w.su; p.ss0 = a.w.ssg; p.ss1 = a.w.ssu;
  p.K = a.d; p.N = a.f;
  p.h_out = (bf16_t*)a.h;
  p.ksplit = 1;
  // heavy tiles, then light tiles with their own kernel shape; the events
  // (when requested) span both launches.  Layers of many small experts run
  // the two launches on two streams (fork / join through events): the light
  // launch streams the small experts' weights while the heavy launch's last
  // round of tiles would otherwise leave most CUs idle.  With few experts the
  // light tiles re-read the heavy experts' weights and running them alongside
  // slowed the heavy launch, so those stay in order on one stream.
  const int groups = a.E + (a.has_shared ? 1 : 0);
  SideStream* side = (a.concurrent && groups >= kConcurrentMinGroups) ? side_stream(s) : nullptr;
  hipError_t ferr = hipSuccess;
  auto chk = [&](hipError_t e) { if (ferr == hipSuccess) ferr = e; };
  auto launch_split = [&](auto heavy, auto light, const GemmParams& prm, int n_tiles, hipEvent_t eb, hipEvent_t ee,
                          int kparts = 1) {
    const int gh = grouped_grid(maxQ, n_tiles);
    const dim3 gl(grouped_grid(groups, n_tiles), kparts);
    hipError_t fe = side ? hipEventRecord(side->fork, s) : hipErrorInvalidValue;
    if (fe == hipSuccess) fe = hipStreamWaitEvent(side->s, side->fork, 0);
    if (side && fe != hipSuccess) chk(fe);      // no fork: both launches stay on `s`, in order
    if (side && fe == hipSuccess) {
      if (eb) hipExtLaunchKernelGGL(heavy, dim3(gh), dim3(256), 0, s, eb, nullptr, 0, prm);
      else heavy<<<gh, 256, 0, s>>>(prm);
      chk(hipGetLastError());
      light<<<gl, 256, 0, side->s>>>(prm);
      chk(hipGetLastError());
      chk(hipEventRecord(side->join, side->s));
      chk(hipStreamWaitEvent(s, side->join, 0));
      if (ee) chk(hipEventRecord(ee, s));
      return;
    }
    if (eb || ee) {
      hipExtLaunchKernelGGL(heavy, dim3(gh), dim3(256), 0, s, eb, nullptr, 0, prm);
      hipExtLaunchKernelGGL(light, gl, dim3(256), 0, s, nullptr, ee, 0, prm);
    } else {
      heavy<<<gh, 256, 0, s>>>(prm);
      light<<<gl, 256, 0, s>>>(prm);
    }
  };

  // fp8 layers whose groups all fit 64 rows (e.g. capped by the capacity):
  // only light tiles exist, and 64-row stages (24 KB) let two work-groups
  // share a CU, doubling the weight loads in flight
  const bool small_f8 = a.wkind == W_FP8 && a.max_group_rows <= 64;
  if (small_f8) {
    const int gl = grouped_grid(groups, (a.f + 127) / 128);
    auto gu = [&](auto kern) {
      if (a.ev_begin || a.ev_end)
        hipExtLaunchKernelGGL(kern, dim3(gl), dim3(256), 0, s, a.ev_begin, a.ev_end, 0, p);
      else
        kern<<<gl, 256, 0, s>>>(p);
    };
    if (small_f8_two_stages(groups * ((a.f + 127) / 128))) gu(gemm_dl_kernel<true, 64, kDlBK, 2, 2, true>);
    else gu(gemm_dl_kernel<true, 64, kDlBK, 3, 2, true>);
  } else if (a.wkind == W_FP8) {
    launch_split(gemm_dl_kernel<true, 256, kDlBK, kDlNST, 1, true>, gemm_dl_kernel<true, 128, kDlBK, 3, 2, true>, p,
                 (a.f + 127) / 128, a.ev_begin, a.ev_end);
  } else {
    launch_split(gemm_dl_kernel<true, 256, kDlBK, kDlNST, 1>, gemm_dl_kernel<true, kBf16LightMax, kDlBK, 2, 2>, p,
                 (a.f + 127) / 128, a.ev_begin, a.ev_end);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ferr != hipSuccess) return ferr;

  GemmParams q = p;
  q.a_rows = (const bf16_t*)a.h;
  q.W0 = a.w.Wd; q.W1 = nullptr; q.Ws0 = a.w.Wsd; q.Ws1 = nullptr;
  q.s0 = a.w.sd; q.s1 = nullptr; q.ss0 = a.w.ssd; q.ss1 = nullptr;
  q.K = a.f; q.N = a.d;
  q.y_out = a.y;
  const int dn_tiles = (a.d + 255) / 256;
  q.ksplit = small_f8 ? 1 : grouped_down_ksplit(a.d, a.f, a.E, a.has_shared, a.wkind, a.act_f32);
  q.part_slots = groups * dn_tiles;
  q.y_part = a.y_part;
  if (small_f8) {
    const int gd = grouped_grid(groups, dn_tiles);
    if (small_f8_two_stages(groups * dn_tiles)) gemm_dl_kernel<false, 64, kDlBK, 2, 2, true><<<gd, 256, 0, s>>>(q);
    else gemm_dl_kernel<false, 64, kDlBK, 3, 2, true><<<gd, 256, 0, s>>>(q);
  } else if (a.wkind == W_FP8) {
    launch_split(gemm_dl_kernel<false, 256, kDlBK, kDlNST, 1, true>, gemm_dl_kernel<false, 128, kDlBK, 3, 2, true>, q,
                 dn_tiles, nullptr, nullptr, q.ksplit);
  } else if (q.ksplit > 1) {
    // few light tiles, each split over K parts: the 128-row stages three deep
    // keep more of each part's weight stream in flight (Mixtral prefill light
    // down 81 us against 104 us with the 64-row two-stage kernel)
    launch_split(gemm_dl_kernel<false, 256, kDlBK, kDlNST, 1>, gemm_dl_kernel<false, 128, kDlBK, 3, 2>, q,
                 dn_tiles, nullptr, nullptr, q.ksplit);
  } else {
    launch_split(gemm_dl_kernel<false, 256, kDlBK, kDlNST, 1>, gemm_dl_kernel<false, kBf16LightMax, kDlBK, 2, 2>, q,
                 dn_tiles, nullptr, nullptr, q.ksplit);
  }
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ferr != hipSuccess) return ferr;
  if (q.ksplit > 1)
    return launch_down_split_reduce(a.sched, maxQ, a.E, dn_tiles, a.d, q.ksplit, q.part_slots, a.y_part, a.y, s);
  return hipGetLastError();
}

}  // namespace moe
