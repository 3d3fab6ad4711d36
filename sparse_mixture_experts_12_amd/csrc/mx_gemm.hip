// Block-scaled (MXFP8) grouped SwiGLU expert FFN on gfx950.
//
// Pages: "Current Bug: CuTeDSLMoERunner produces wrong output", "Root Cause:
// scale_a layout doesn't match expert_offsets" (a grouped MoE whose
// activations carry per-token block scale factors, addressed per expert
// through its row offsets; NVFP4 on another chip); "MoE Model Architectures",
// Mixtral "Expert FFN" (w2(silu(w1 x) * w3 x)) and "Sparse MoE Block" (only
// experts with tokens run).
//
// Format (OCP Microscaling MXFP8): E4M3 codes, one E8M0 power-of-two scale
// per 32 consecutive values along the reduction axis.  A block with largest
// magnitude m gets the exponent s = floor(log2 m) - 8 (clamped to
// [-127, 127], an all-zero block -127); its elements are v / 2^s rounded to
// nearest even E4M3, magnitudes above 448 saturated.
//
//   quantise: x rows [T, d] (bf16 or fp32) -> codes [T, d], scales [T, d/32]
//   gate/up:  H[r, n] = silu(A[r] . Wg[n]) * (A[r] . Wu[n]) in fp32, A[r] the
//             quantised x row of the token owning permuted row r; H is then
//             quantised per 32 columns in the epilogue -> codes + scales
//   down:     Y[r, n] = H[r] . Wd[n]  (fp32)
// Weights are stored output-major with K contiguous ([E, N, K] codes,
// [E, N, K/32] scales), so both operands are K-contiguous rows: no
// transposing reads.  The product runs on v_mfma_scale_f32_32x32x64_f8f6f4,
// which applies both operands' block scales inside the matrix core.
//
// Tiles: BM (256, with 128- and 64-row bodies for an expert's short last
// tile) permuted rows x 256 B-rows (the gate/up GEMM takes 128 gate and the
// same 128 up columns), 4 waves, 128 K per LDS stage, two stages.  A and B
// tiles move global -> LDS directly (16 bytes per lane) with the LDS swizzle
// applied on the source side; the block scales (4 bytes per row per stage)
// go to registers with plain loads issued beside them.
//
// MFMA operand layout (32x32x64, 8 bit): lane l = (i, h), i = l % 32 the row
// (A) or column (B), h = l / 32; its 32 bytes hold K = 16 h .. 16 h + 15 and
// 32 + 16 h .. 32 + 16 h + 15 of the 64; its scale byte (selected by the
// instruction's op_sel from a 32-bit register) is that of K block h.
//
// MXFP4 weights (E2M1, two codes per byte, element 2j in the low nibble): the
// B operand of the same instruction in its 4-bit format takes 16 bytes per
// lane, lane (i, h) holding K = 32 h .. 32 h + 31 in order, low nibble first
// (checked with an in-bounds probe of the instruction), so one 16-byte LDS
// read per lane and sub-step; B rows of a stage are 64 bytes (128 K) with
// the 4-chunk swizzle aswz<4>.  Scales, A (MXFP8 x or H) and the epilogues
// are as for MXFP8 weights.
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int kMxBK = 128;    // K per LDS stage (bytes of codes)

struct MxParams {
  const uint8_t* aq;             // DUAL: x codes [T, K]; !DUAL: H codes [rows, K]
  const uint8_t* as;             // matching scales [., K / 32]
  const int32_t* sorted_assign;  // DUAL: permuted row -> assignment
  const uint8_t* W0;             // codes [E, N, K]: gate (DUAL) or down
  const uint8_t* W1;             // up (DUAL)
  const uint8_t* S0;             // scales [E, N, K / 32]
  const uint8_t* S1;
  const uint8_t* Ws0;            // shared expert [N, K], [N, K / 32]
  const uint8_t* Ws1;
  const uint8_t* Ss0;
  const uint8_t* Ss1;
  const int32_t* sched;
  int maxQ;
  int k, E, K, N;
  int shared_row0;
  uint8_t* hq_out;               // DUAL: H codes [rows, N]
  uint8_t* hs_out;               // DUAL: H scales [rows, N / 32]
  float* y_out;                  // !DUAL: [rows, N]
  float* y_part;                 // !DUAL light tiles split over K: parts 1.. [ksplit - 1][part_slots][128][256]
  int ksplit;                    // K parts of the down GEMM's light tiles (1: none)
  int part_slots;
};

// Per 16-bit half, the largest value over the 32 lanes of each half-wave
// (lanes 0..31, 32..63) as packed unsigned 16-bit integers: quad swap, quad
// pair swap, rotations by 4 and 8 inside each 16-lane row, then the two rows
// of the half exchanged.
__device__ __forceinline__ uint32_t half_wave_max_u16x2(uint32_t v) {
  typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
  auto mx = [](uint32_t a, uint32_t b) -> uint32_t {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                  __builtin_bit_cast(u16x2_t, b)));
  };
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  v = mx(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  return v;
}

// Biased E8M0 scale code of a block whose largest magnitude is m (fp32):
// floor(log2 m) - 8 + 127 = exponent field - 8, at least 0 (zero and
// subnormal blocks take -127).
__device__ __forceinline__ int mx_scale_code(float m) { return max((int)((__float_as_uint(m) >> 23) & 0xff) - 8, 0); }

// v / 2^(code - 127) rounded to E4M3 (RNE, saturated at 448).  The factor
// 2^(127 - code) is a normal fp32 for every code this kernel produces
// (code <= 246), so the scaling is exact.
__device__ __forceinline__ float mx_scaled(float v, int code) {
  const float f = __uint_as_float((uint32_t)(254 - code) << 23);
  return fminf(fmaxf(v * f, -448.f), 448.f);
}

// ---------------------------------------------------------------------------
// Quantiser: 4 lanes per 32-value block, 8 values per lane.
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const TIn* __restrict__ in, long nblk,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long blk = gid >> 2;
  const bool ok = blk < nblk;
  const long e0 = (ok ? gid : 0) * 8;
  float v[8];
  if constexpr (std::is_same<TIn, float>::value) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(in + e0);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(in + e0 + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  } else {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(in + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16lo(w[i]);
      v[2 * i + 1] = bf16hi(w[i]);
    }
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  const int code = mx_scale_code(m);
  u32x2_t o;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(v[4 * w], code), mx_scaled(v[4 * w + 1], code), 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(v[4 * w + 2], code), mx_scaled(v[4 * w + 3], code), p, true);
    o[w] = (uint32_t)p;
  }
  if (ok) {
    *reinterpret_cast<u32x2_t*>(codes + e0) = o;
    if ((gid & 3) == 0) scales[blk] = (uint8_t)code;
  }
}

hipError_t launch_mx_quantize(const void* in, bool in_f32, long rows, int cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const long nblk = rows * (long)(cols / 32);
  if (nblk == 0) return hipSuccess;
  const long threads = nblk * 4;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  if (in_f32)
    mx_quantize_kernel<float><<<grid, 256, 0, s>>>((const float*)in, nblk, codes, scales);
  else
    mx_quantize_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t*)in, nblk, codes, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Grouped GEMM tile
// ---------------------------------------------------------------------------
// One output tile of at most BMV rows: waves 2 x 2 (128 rows x 128 B-rows
// each) for BMV = 256, 1 x 4 (BMV rows x 64 B-rows each) for 128 and 64.
// LDS stage: 256 A rows then 256 B rows of 128 code bytes each (16-byte chunk
// c of row r at chunk position aswz<8>(r, c): conflict-free 16-lane passes of
// ds_read_b128 down a column of rows), then the stage's scale dwords (4 K
// blocks) of the 256 A rows and of the 256 B rows.
// K range [k_lo, k_lo + nK BK); K part kpart > 0 writes its fp32 block to
// y_part slot `slot` (light down tiles split over K).
template <bool DUAL, int BMV, int BMMAX, int NST, bool W4>
__device__ __forceinline__ void mx_tile(const MxParams& p, int g, int row0, int rows, int nt, uint8_t* L0,
                                        uint8_t* L1, uint8_t* L2, int k_lo, int nK, int kpart, int slot) {
  constexpr int BK = kMxBK;
  constexpr int BKB = W4 ? BK / 2 : BK;              // bytes of a B row per stage (E2M1: two per byte)
  constexpr int WM = (BMV >= 256) ? 2 : 1, WN = 4 / WM;
  constexpr int NMAT = DUAL ? 2 : 1;
  constexpr int BN_MAT = DUAL ? 128 : 256;
  constexpr int NI_MAT = BN_MAT / WN / 32;
  constexpr int NI = NI_MAT * NMAT;
  constexpr int MI = BMV / WM / 32;
  constexpr int WROWS = BMV / WM;
  constexpr int A_LD = BMV / 8 / 4;                // 1 KB (8-row) A blocks per wave per stage
  constexpr int B_RPB = 1024 / BKB;                // B rows per 1 KB block
  constexpr int B_LD = 256 / B_RPB / 4;            // 1 KB B blocks per wave per stage
  constexpr int LDS_B = BMMAX * BK;                // B codes
  constexpr int LDS_SA = BMMAX * BK + 256 * BKB;   // A scale dwords [256]
  constexpr int LDS_SB = LDS_SA + 1024;            // B scale dwords [256]
  constexpr int NMF = MI * NI;                      // MFMAs per 64-K sub-step
  constexpr int NDS = 2 * MI + (W4 ? 1 : 2) * NI + MI + NI;   // LDS reads per sub-step (codes, scales)
  constexpr int NVM = A_LD + B_LD + 2;              // global -> LDS loads per stage
  static_assert(BK == 128 && (NST == 2 || NST == 3) && A_LD >= 1 && BMV <= BMMAX, "tile configuration");
  static_assert((NST - 1) * NVM < 64, "outstanding loads exceed the vmcnt range");
  const int KS = p.K >> 5;                         // scale bytes per row

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int l32 = lane & 31;
  const int lhi = lane >> 5;
  const int n0 = nt * BN_MAT;
  const bool shared = (g == p.E);

  // A row (x row of the owning token, or the H row) of tile row r; rows past
  // the valid ones read the tile's first row (never stored).
  auto a_row = [&](int r) -> uint32_t {
    const int grow = row0 + (r < rows ? r : 0);
    if (DUAL) return (uint32_t)(shared ? (grow - p.shared_row0) : (p.sorted_assign[grow] / p.k));
    return (uint32_t)grow;
  };
  // B rows: wave w's 64 LDS B rows 64 w .. 64 w + 63 are one matrix's
  // consecutive output columns from cb(w); a block past N (the down GEMM's
  // last, half-used tile) re-reads the block 128 columns before (never stored).
  const size_t gN = shared ? 0 : (size_t)g * p.N;
  auto b_first = [&](int w, int* mat) -> int {
    int c;
    if (DUAL) {
      *mat = w >> 1;
      c = n0 + 64 * (w & 1);
    } else {
      *mat = 0;
      c = n0 + 64 * w;
    }
    return c < p.N ? c : c - 128;
  };
  auto b_codes = [&](int mat) -> const uint8_t* { return shared ? (mat ? p.Ws1 : p.Ws0) : (mat ? p.W1 : p.W0); };
  auto b_scales = [&](int mat) -> const uint8_t* { return shared ? (mat ? p.Ss1 : p.Ss0) : (mat ? p.S1 : p.S0); };

  // ---- global -> LDS sources.  Code block b (A: b = wave + 4 i, B: b =
  // B_LD wave + j) holds rows 8 b .. 8 b + 7; this lane fills row
  // r = 8 b + lane / 8, LDS chunk lane % 8, i.e. global chunk
  // aswz<8>(r, lane % 8) = (lane % 8) ^ (lane / 8) ^ (b % 8).
  // Scales: this lane fills dword 64 wave + lane of each scale array. ----
  // Every source is a wave-uniform base plus a 32-bit per-lane offset, so the
  // loads take the scalar-base addressing form (one VGPR per address).
  const int cx = (lane & 7) ^ (lane >> 3);
  uint32_t aoff[A_LD];                              // byte offset of this lane's A chunk
#pragma unroll
  for (int i = 0; i < A_LD; ++i)
    aoff[i] = a_row(8 * (wave + 4 * i) + (lane >> 3)) * (uint32_t)p.K + ((cx ^ ((wave + 4 * i) & 7)) << 4);
  int bmat;
  const int bc = b_first(wave, &bmat);
  const uint32_t KB = W4 ? (uint32_t)p.K / 2 : (uint32_t)p.K;   // bytes of a weight row
  const uint8_t* bbase = b_codes(bmat) + (gN + bc) * (size_t)KB;
  uint32_t boff[B_LD];
#pragma unroll
  for (int j = 0; j < B_LD; ++j) {
    if constexpr (W4)   // row 16 b + lane / 4, LDS chunk lane % 4 = aswz<4>(row, global chunk)
      boff[j] = (uint32_t)(16 * j + (lane >> 2)) * KB + (uint32_t)(((lane & 3) ^ (lane >> 4)) << 4);
    else
      boff[j] = (uint32_t)(8 * j + (lane >> 3)) * KB + ((cx ^ ((B_LD * wave + j) & 7)) << 4);
  }
  const uint32_t asoff = a_row(64 * wave + lane) * (uint32_t)KS;
  const uint8_t* bsbase = b_scales(bmat) + (gN + bc) * (size_t)KS;
  const uint32_t bsoff = (uint32_t)lane * (uint32_t)KS;

  auto issue = [&](uint8_t* L, int kr) {
    const int k0 = k_lo + kr;
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(p.aq + (aoff[i] + (uint32_t)k0)),
                                       (lds_ptr_t)(L + (wave + 4 * i) * 1024), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < B_LD; ++j)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(bbase + (boff[j] + (uint32_t)(W4 ? k0 / 2 : k0))),
                                       (lds_ptr_t)(L + LDS_B + (B_LD * wave + j) * 1024), 16, 0,
                                       (BMV <= 128) ? 2 : 0);   // light tiles stream their weights
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(p.as + (asoff + (uint32_t)(k0 >> 5))),
                                     (lds_ptr_t)(L + LDS_SA + wave * 256), 4, 0, 0);
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(bsbase + (bsoff + (uint32_t)(k0 >> 5))),
                                     (lds_ptr_t)(L + LDS_SB + wave * 256), 4, 0, 0);
  };

  f32x16_t acc[MI][NI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  // B row (LDS) of fragment ni for this lane
  auto b_lrow = [&](int ni) -> int {
    if (DUAL) return (ni / NI_MAT) * 128 + wn * (128 / WN) + (ni % NI_MAT) * 32 + l32;
    return wn * (256 / WN) + ni * 32 + l32;
  };
  // Fragments of 64-K sub-step ks, plus the stage's scale dwords shifted so
  // that byte 2 ks is this lane's K block (h) of the sub-step.
  auto frags = [&](const uint8_t* L, int ks, i32x8_t* af, i32x8_t* bfr, uint32_t* sa, uint32_t* sb) {
    const int c0 = 4 * ks + lhi, c1 = c0 + 2;
    const int sh = 8 * lhi;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int row = wm * WROWS + mi * 32 + l32;
      const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(L + row * BK + aswz<8>(row, c0) * 16);
      const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(L + row * BK + aswz<8>(row, c1) * 16);
      af[mi] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      sa[mi] = *reinterpret_cast<const uint32_t*>(L + LDS_SA + row * 4) >> sh;
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int j = b_lrow(ni);
      const uint8_t* Lb = L + LDS_B + j * BKB;
      if constexpr (W4) {
        const u32x4_t q = *reinterpret_cast<const u32x4_t*>(Lb + aswz<4>(j, 2 * ks + lhi) * 16);
        bfr[ni] = i32x8_t{(int)q[0], (int)q[1], (int)q[2], (int)q[3], 0, 0, 0, 0};
      } else {
        const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(Lb + aswz<8>(j, c0) * 16);
        const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(Lb + aswz<8>(j, c1) * 16);
        bfr[ni] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      sb[ni] = *reinterpret_cast<const uint32_t*>(L + LDS_SB + j * 4) >> sh;
    }
  };
  auto mfmas = [&](const i32x8_t* af, const i32x8_t* bfr, const uint32_t* sa, const uint32_t* sb, auto KS_) {
    constexpr int ops = 2 * decltype(KS_)::value;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bfr[ni], acc[mi][ni], 0, W4 ? 4 : 0,
                                                                      ops, (int)sa[mi], ops, (int)sb[ni]);
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  // Pipeline over the two 64-K sub-steps of each stage (as in the bf16
  // kernel): sub-step 1's fragments are read while sub-step 0 multiplies; the
  // stage's last MFMAs run after the barrier that publishes the next stage and
  // cover the first fragment reads of the next stage.  The stage just read is
  // then refilled two steps ahead (past the end: the last stage again, never
  // read), so every wave issues the same loads per step and the vmcnt
  // thresholds are exact.
  // With three stages (light tiles) two steps of loads stay in flight: the
  // wait after a stage's first sub-step only needs the next stage, and the
  // stage just read is refilled NST steps ahead.
  i32x8_t fa0[MI], fb0[NI], fa1[MI], fb1[NI];
  uint32_t sa0[MI], sb0[NI], sa1[MI], sb1[NI];
  issue(L0, 0);
  issue(L1, min(1, nK - 1) * BK);
  if constexpr (NST > 2) issue(L2, min(2, nK - 1) * BK);
  wait_vmem_le<(NST - 1) * NVM>();
  __builtin_amdgcn_s_barrier();
  frags(L0, 0, fa0, fb0, sa0, sb0);

  auto step = [&](uint8_t* L, const uint8_t* Ln, int k) {
    frags(L, 1, fa1, fb1, sa1, sb1);
    mfmas(fa0, fb0, sa0, sb0, I0{});
    sched_interleave<NMF, NDS, 0>();
    __builtin_amdgcn_sched_barrier(0);
    wait_vmem_le_lds0<(NST - 2) * NVM>();
    __builtin_amdgcn_s_barrier();
    issue(L, min(k + NST, nK - 1) * BK);
    frags(Ln, 0, fa0, fb0, sa0, sb0);
    mfmas(fa1, fb1, sa1, sb1, I1{});
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

  // ---- epilogue ----
  if constexpr (DUAL) {
    // H = silu(gate) * up in fp32, quantised per row and 32 columns: a
    // fragment's 32 columns of one row live in the 32 lanes of a half-wave
    // (register v holds row 8 (v / 4) + 4 lhi + v % 4).  The block scale only
    // needs the largest exponent field, reduced for two rows at a time as
    // packed 16-bit integers.  The codes of 4 rows x 4 columns are transposed
    // inside each lane quad so that every lane stores one dword (4 columns of
    // one row); lane v of each half stores row v's scale byte.
    const int KSo = p.N >> 5;
    const int j4 = lane & 3;
    const uint32_t selA = (j4 & 1) ? 0x03070105u : 0x06020400u;
    const uint32_t selB = (j4 & 2) ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int nl = 0; nl < NI_MAT; ++nl) {
        const int cb0 = n0 + wn * (BN_MAT / WN) + nl * 32;     // first H column of the fragment
        float h[16];
        int code[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float g = acc[mi][nl][v];
          h[v] = g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * acc[mi][nl + NI_MAT][v];
        }
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          uint32_t m = ((__float_as_uint(h[v]) >> 23) & 0xffu) | (((__float_as_uint(h[v + 1]) >> 23) & 0xffu) << 16);
          m = half_wave_max_u16x2(m);
          code[v] = max((int)(m & 0xffffu) - 8, 0);
          code[v + 1] = max((int)(m >> 16) - 8, 0);
        }
        uint32_t rowq[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          int b = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(h[4 * g], code[4 * g]),
                                                  mx_scaled(h[4 * g + 1], code[4 * g + 1]), 0, false);
          b = __builtin_amdgcn_cvt_pk_fp8_f32(mx_scaled(h[4 * g + 2], code[4 * g + 2]),
                                              mx_scaled(h[4 * g + 3], code[4 * g + 3]), b, true);
          const uint32_t x = (uint32_t)__builtin_amdgcn_update_dpp(0, b, 0xB1, 0xF, 0xF, false);   // lane ^ 1
          const uint32_t t = __builtin_amdgcn_perm(x, (uint32_t)b, selA);
          const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0x4E, 0xF, 0xF, false);  // lane ^ 2
          rowq[g] = __builtin_amdgcn_perm(y, t, selB);
        }
        int sc = code[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) sc = (l32 == v) ? code[v] : sc;
        const int rbase = wm * WROWS + mi * 32 + lhi * 4;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r = rbase + 8 * g + j4;
          if (r < rows)
            *reinterpret_cast<uint32_t*>(p.hq_out + (size_t)(row0 + r) * p.N + cb0 + (l32 & ~3)) = rowq[g];
        }
        if (l32 < 16) {
          const int r = rbase + 8 * (l32 >> 2) + (l32 & 3);
          if (r < rows) p.hs_out[(size_t)(row0 + r) * KSo + (cb0 >> 5)] = (uint8_t)sc;
        }
      }
    }
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = n0 + wn * (256 / WN) + ni * 32 + l32;
        if (col >= p.N) continue;
        // K part 0 (or no split): Y rows; parts 1..: this slot's 128 x 256 block
        float* out = kpart == 0 ? p.y_out + (size_t)row0 * p.N + col
                                : p.y_part + ((size_t)(kpart - 1) * p.part_slots + slot) * (128 * 256) + (col - n0);
        const size_t ostride = kpart == 0 ? (size_t)p.N : 256;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WROWS + mi * 32 + (v >> 2) * 8 + lhi * 4 + (v & 3);
          if (r < rows) out[(size_t)r * ostride] = acc[mi][ni][v];
        }
      }
    }
  }
}

// SEG 1: heavy row tiles (more than 128 rows): 256-row LDS stages, two deep
//        with 8-bit weights; with 4-bit weights a stage is a quarter smaller,
//        so three fit in LDS (150 KB) and keep two steps of loads in flight.
// SEG 2: light row tiles (an expert's last tile, at most 128 rows): 128-row
//        stages, three deep (two steps of loads in flight; these tiles do little
//        MFMA work per stage and are bound by load latency).
template <bool DUAL, int SEG, bool W4>
__global__ __launch_bounds__(256, 1) void gemm_mx_kernel(MxParams p) {
  constexpr int BMMAX = SEG == 1 ? 256 : 128;
  constexpr int NST = (SEG == 1 && !W4) ? 2 : 3;
  constexpr int LDS_S = BMMAX * kMxBK + 256 * (W4 ? kMxBK / 2 : kMxBK) + 2048;
  __shared__ __attribute__((aligned(1024))) uint8_t L0[LDS_S];
  __shared__ __attribute__((aligned(1024))) uint8_t L1[LDS_S];
  __shared__ __attribute__((aligned(1024))) uint8_t L2[NST > 2 ? LDS_S : 16];
  constexpr int BN_MAT = DUAL ? 128 : 256;
  const int n_tiles = (p.N + BN_MAT - 1) / BN_MAT;
  int g, row0, rows, nt, slot = 0;
  if (!decode_tile<SEG>(p.sched, p.maxQ, p.E, n_tiles, &g, &row0, &rows, &nt, &slot)) return;
  // light down tiles may be split over K (blockIdx.y = K part)
  const int kparts = (!DUAL && SEG == 2) ? p.ksplit : 1;
  const int kpart = (!DUAL && SEG == 2) ? (int)blockIdx.y : 0;
  const int nK = p.K / kMxBK / kparts;
  const int k_lo = kpart * nK * kMxBK;
  if constexpr (SEG == 1) {
    mx_tile<DUAL, 256, BMMAX, NST, W4>(p, g, row0, rows, nt, L0, L1, L2, k_lo, nK, kpart, slot);
  } else {
    if (rows > 64) mx_tile<DUAL, 128, BMMAX, NST, W4>(p, g, row0, rows, nt, L0, L1, L2, k_lo, nK, kpart, slot);
    else mx_tile<DUAL, 64, BMMAX, NST, W4>(p, g, row0, rows, nt, L0, L1, L2, k_lo, nK, kpart, slot);
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
template <bool W4>
static hipError_t launch_grouped_ffn_mx_t(const GroupedArgs& a, hipStream_t s) {
  uint8_t* xq = a.mx_xq;
  uint8_t* xs = a.mx_xs;
  uint8_t* hq = (uint8_t*)a.h;
  uint8_t* hs = a.mx_hs;
  const SchedSpec sp = grouped_sched_spec(a);
  const int BM = sp.BM;
  const int maxQ = sp.maxQ;
  hipError_t err = hipSuccess;
  if (!a.sched_ready &&
      (err = launch_tile_schedule(a.offsets, a.E, BM, sp.shared_rows, a.routed_rows, maxQ, a.sched, s)) != hipSuccess)
    return err;
  if ((err = launch_mx_quantize(a.x, a.act_f32, a.T, a.d, xq, xs, s)) != hipSuccess) return err;

  MxParams p{};
  p.aq = xq; p.as = xs;
  p.sorted_assign = a.sorted_assign;
  p.W0 = (const uint8_t*)a.w.Wg; p.W1 = (const uint8_t*)a.w.Wu;
  p.S0 = a.w.mxg; p.S1 = a.w.mxu;
  p.Ws0 = (const uint8_t*)a.w.Wsg; p.Ws1 = (const uint8_t*)a.w.Wsu;
  p.Ss0 = a.w.mxsg; p.Ss1 = a.w.mxsu;
  p.sched = a.sched; p.maxQ = maxQ;
  p.k = a.assign_div; p.E = a.E; p.K = a.d; p.N = a.f; p.shared_row0 = a.routed_rows;
  p.hq_out = hq; p.hs_out = hs;
  p.ksplit = 1;
  // heavy tiles, then light tiles; the events (when requested) span both.
  // Layers of many small experts fork the light launch onto a second stream
  // (as the bf16 / fp8 grouped GEMMs do).
  const int groups = a.E + (a.has_shared ? 1 : 0);
  SideStream* side = (a.concurrent && groups >= kConcurrentMinGroups) ? side_stream(s) : nullptr;
  hipError_t ferr = hipSuccess;
  auto chk = [&](hipError_t e) { if (ferr == hipSuccess) ferr = e; };
  auto launch_split = [&](auto heavy, auto light, const MxParams& prm, int n_tiles, hipEvent_t eb, hipEvent_t ee,
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
      hipExtLaunchKernelGGL(light, dim3(gl), dim3(256), 0, s, nullptr, ee, 0, prm);
    } else {
      heavy<<<gh, 256, 0, s>>>(prm);
      light<<<gl, 256, 0, s>>>(prm);
    }
  };
  launch_split(gemm_mx_kernel<true, 1, W4>, gemm_mx_kernel<true, 2, W4>, p, a.f / 128, a.ev_begin, a.ev_end);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ferr != hipSuccess) return ferr;

  MxParams q{};
  q.aq = hq; q.as = hs;
  q.W0 = (const uint8_t*)a.w.Wd; q.S0 = a.w.mxd;
  q.Ws0 = (const uint8_t*)a.w.Wsd; q.Ss0 = a.w.mxsd;
  q.sched = a.sched; q.maxQ = maxQ;
  q.k = a.assign_div; q.E = a.E; q.K = a.f; q.N = a.d; q.shared_row0 = a.routed_rows;
  q.y_out = a.y;
  const int dn_tiles = (a.d + 255) / 256;
  q.ksplit = grouped_down_ksplit(a.d, a.f, a.E, a.has_shared, a.wkind, a.act_f32);
  q.part_slots = groups * dn_tiles;
  q.y_part = a.y_part;
  launch_split(gemm_mx_kernel<false, 1, W4>, gemm_mx_kernel<false, 2, W4>, q, dn_tiles, nullptr, nullptr, q.ksplit);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (ferr != hipSuccess) return ferr;
  if (q.ksplit > 1)
    return launch_down_split_reduce(a.sched, maxQ, a.E, dn_tiles, a.d, q.ksplit, q.part_slots, a.y_part, a.y, s);
  return hipSuccess;
}

hipError_t launch_grouped_ffn_mx(const GroupedArgs& a, hipStream_t s) {
  return a.wkind == W_MX4 ? launch_grouped_ffn_mx_t<true>(a, s) : launch_grouped_ffn_mx_t<false>(a, s);
}

}  // namespace moe
