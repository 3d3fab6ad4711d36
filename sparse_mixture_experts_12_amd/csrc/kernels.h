// Internal launch interface between the C-ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kDecodeMaxT = 8;

struct RouteArgs {
  const void* x;
  const void* W_g;
  const float* bias;
  int T, d, E, k, renormalize;
  int cap;          // -1: uncapped
  bool act_f32;
  float* logits;    // [T, E] or nullptr
  double* part;     // fp64 partial logits (router_partial_bytes); optional for T <= kDecodeMaxT
  int32_t* idx;     // [T, k]
  float* w;         // [T, k]
  int32_t* plan;    // decode plan or nullptr (T <= kDecodeMaxT only)
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
size_t router_partial_bytes(int T, int d, int E);

// Where and how to write the grouped GEMMs' tile schedule (see
// tile_schedule_kernel); sched == nullptr: not requested.
struct SchedSpec {
  int32_t* sched;
  int BM, shared_rows, shared_row0, maxQ;
  int light_max = 0;                 // a group's last tile is light at <= light_max rows (0: BM / 2)
};

struct PermuteArgs {
  const int32_t* idx;
  int n, E, cap;
  int32_t *counts, *offsets, *sorted_assign, *inv_perm, *n_dropped;
  int32_t* rank_ws;                  // permute_ws_bytes(n, E) bytes of scratch
  SchedSpec sched;                   // optional: also write the tile schedule
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t s);
// rank_ws bytes launch_permute needs for n assignments over E experts
size_t permute_ws_bytes(int n, int E);
// Tile schedule header size (ints): [0] heavy row tiles, [1] light row tiles.
constexpr int kSchedHead = 4;
hipError_t launch_tile_schedule(const int32_t* offsets, int E, int BM, int shared_rows, int shared_row0, int maxQ,
                                int32_t* sched, hipStream_t s, int light_max = 0);

// Expert weights of one group set: routed experts [E,...] plus the optional
// shared expert, addressed as group E.
struct ExpertWeights {
  const void *Wg, *Wu, *Wd;             // [E,d,f], [E,d,f], [E,f,d]
  const float *sg, *su, *sd;            // fp8 scales or nullptr
  const void *Wsg, *Wsu, *Wsd;          // shared expert or nullptr
  const float *ssg, *ssu, *ssd;
  // MXFP8: codes are output-major ([E,f,d], [E,f,d], [E,d,f]) and these are
  // their E8M0 block scales ([E,f,d/32], [E,f,d/32], [E,d,f/32]; shared [N, K/32])
  const uint8_t *mxg, *mxu, *mxd;
  const uint8_t *mxsg, *mxsu, *mxsd;
};

enum WKind { W_F32 = 0, W_BF16 = 1, W_FP8 = 2, W_MX = 3, W_MX4 = 4 };   // W_MX4: E2M1 codes, two per byte

struct GroupedArgs {
  const void* x;                 // [T, d] act
  const int32_t* sorted_assign;  // routed rows -> assignment id
  const int32_t* offsets;        // [E + 1]
  ExpertWeights w;
  int T, d, E, k, f;
  int routed_rows;               // rows before the shared expert's (T*k; E*C for expert choice)
  int assign_div;                // token of permuted row r = sorted_assign[r] / assign_div (k; 1)
  int has_shared;
  int max_group_rows;            // bound on any group's rows (capacity, T, the shared expert's T)
  int wkind;                     // WKind
  bool act_f32;
  float* y;                      // [routed_rows (+T), d] fp32
  void* h;                       // [routed_rows (+T), f] bf16 (or fp32 for act f32)
  int32_t* sched;                // schedule scratch
  bool sched_ready;              // the schedule (grouped_sched_spec) was already written with the permutation
  float* y_part;                 // down light tiles' K parts 1.. (grouped_down_part_bytes)
  uint8_t* mx_xq;                // W_MX: x codes [T, d] (scratch)
  uint8_t* mx_xs;                // W_MX: x scales [T, d/32]
  uint8_t* mx_hs;                // W_MX: H scales [rows, f/32]; h holds the H codes
  hipEvent_t ev_begin, ev_end;
  bool concurrent;               // may run heavy and light launches on a second stream (fork / join)
};
// Groups (experts + shared) from which the heavy and light launches of a
// grouped GEMM run on two streams.
constexpr int kConcurrentMinGroups = 64;
// A second stream and its fork / join events, created at the first use by a
// host thread on a device and kept until the process ends (default priority).
// nullptr if they cannot be created, or if that first use comes while
// `caller` is capturing a graph: the launches then stay on one stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool bad = false;
};
SideStream* side_stream(hipStream_t caller);
size_t grouped_sched_ints(int routed_rows, int T, int E, int has_shared);
// The schedule launch_grouped_ffn builds for a (its tile height and list size).
SchedSpec grouped_sched_spec(const GroupedArgs& a);
int grouped_max_row_tiles(int routed_rows, int T, int E, int has_shared, int BM);
int grouped_grid(int maxQ, int n_tiles);
hipError_t launch_grouped_ffn(const GroupedArgs& a, hipStream_t s);
int grouped_down_ksplit(int d, int f, int E, int has_shared, int wkind, int act_f32);
size_t grouped_down_part_bytes(int d, int f, int E, int has_shared, int wkind, int act_f32);
// Y rows of the light down tiles += their K parts 1 .. ksplit - 1, in order
hipError_t launch_down_split_reduce(const int32_t* sched, int maxQ, int E, int n_tiles, int N, int ksplit,
                                    int part_slots, const float* part, float* y, hipStream_t s);
hipError_t launch_grouped_ffn_mx(const GroupedArgs& a, hipStream_t s);
// OCP MXFP8 quantisation of rows x cols values (cols % 32 == 0) along rows
hipError_t launch_mx_quantize(const void* in, bool in_f32, long rows, int cols, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);

struct DecodeArgs {
  const void* x;                 // [T, d] act
  const int32_t* plan;           // from the small-T router
  const float* topk_w;           // [T, k]
  ExpertWeights w;
  int T, d, E, k, f, has_shared, wkind;
  bool act_f32;
  float* partial;                // scratch
  void* out;                     // [T, d] act
  hipEvent_t ev_begin, ev_end;
};
size_t decode_partial_bytes(int T, int d, int E, int k, int f, int has_shared, int wkind);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

struct CombineArgs {
  const float* y;
  const int32_t* inv_perm;
  const float* w;
  int T, d, k, has_shared;
  bool act_f32;
  void* out;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// Backward pass (token choice, bf16 activations and weights)
struct BwdGemmParams {          // grouped GEMMs of the backward
  const bf16_t* A0;        // GU/NT: padded rows [P, lda]; TN: activations [P, lda]
  const bf16_t* A1;        // NT: second K part (K >= K1), else nullptr
  int lda;
  const bf16_t* B0;        // GU: W_gate [E, K, N]; NT: weights [E, N, K]; TN: activations [P, ldb]
  const bf16_t* B1;        // GU: W_up; NT: second K part's weights; TN: nullptr
  const bf16_t* Bs0;       // shared expert's matrices (group E)
  const bf16_t* Bs1;
  int ldb;
  long bgs;                // GU/NT: elements of one group's weight matrix
  int K, K1;               // GU/NT: reduction length and the split point (K1 = K: no split)
  int M, N;                // TN: output rows (M) and columns (N); GU/NT: N = output columns
  const int32_t* sched;    // GU/NT row-tile schedule over the padded rows
  int maxQ, E, G;
  const int32_t* poff;     // [G + 1] padded group offsets
  float* C0;               // GU: G rows [P, N]; NT: [P, N]; TN: dW [G][M][N] (group g at C0 + g * cstride)
  float* C1;               // GU: U rows [P, N]
  float* Cs;               // TN: the shared group's output (group E), or nullptr
  long cstride;
  float* part;             // NT/NTS light tiles split over K: parts 1.. [ksplit - 1][part_slots][128][256]
  int ksplit;              // K parts of the light row tiles (0 or 1: none)
  int part_slots;          // light-segment slots (groups x column tiles)
};
// mode 0: G/U recompute, 1: NT, 2: NT with K split over two (A, B) pairs
hipError_t launch_bwd_rows(int mode, const BwdGemmParams& p, hipStream_t s);
hipError_t launch_bwd_wgrad(const BwdGemmParams& p, hipStream_t s);
struct BwdF32Params {           // backward GEMMs of fp32 layers (padded rows as above)
  const float* A0;               // rows: [P, lda] K-contiguous; wgrad: [P, lda], m contiguous
  const float* A1;               // rows: second K part (K >= K1), else nullptr
  int lda;
  const float *B0, *B1;          // rows: expert weights (group stride bgs); wgrad: [P, ldb]
  const float *Bs0, *Bs1;        // rows: shared expert's weights
  int ldb;
  long bgs;
  bool b_kc;                     // rows: B(k, n) = B[n ldb + k] (else B[k ldb + n])
  int K, K1, N, M;               // K: rows products' reduction; N: output columns; M: wgrad output rows
  const int32_t* poff;           // [G + 1] padded group offsets
  int G, E;
  float* C;                      // rows: [P, N]; wgrad: group g at C + g cstride ([M, N])
  float* Cs;                     // wgrad: the shared expert's [M, N]
  long cstride;
};
hipError_t launch_bwd_rows_f32(const BwdF32Params& p, long pmax, hipStream_t s);
hipError_t launch_bwd_wgrad_f32(const BwdF32Params& p, hipStream_t s);
// K parts of the dX GEMM's light row tiles, and the workspace their parts take
int backward_dx_ksplit(int d, int f, int G);
size_t backward_dx_part_bytes(int d, int f, int G);

struct BackwardArgs {
  const void* x;                 // [T, d] bf16
  const void* dout;              // [T, d] bf16
  const void* W_g;               // [d, E] bf16
  ExpertWeights w;
  int T, d, E, k, f, has_shared, renormalize;
  long routed;                   // routed rows: T k (token choice) or E C (expert choice)
  // forward routing (recomputed by the caller)
  const float* logits;           // [T, E]
  const int32_t* topk_idx;       // [T, k]   (token choice)
  const float* topk_w;           // [T, k]   (token choice)
  const int32_t* offsets;        // [E + 1]
  const int32_t* sorted_assign;  // [T k] assignment per row; expert choice: [E C] token per row
  const int32_t* inv_perm;       // [T k]   (token choice)
  // expert choice (ec_C > 0): the selection of launch_expert_choice
  int ec_C;
  const float* ec_scores;        // [E, T] full-softmax scores
  const int32_t* ec_pos;         // [T, E] row of (t, e) or -1
  const int32_t* ec_crow;        // [T, E] per token: rows of its experts, ascending expert order
  const float* ec_w;             // [T, E] the matching combine weights
  const int32_t* ec_count;       // [T] experts that took the token
  // scratch (padded row space of backward_pad_rows rows)
  int32_t* poff;                 // [G + 1]
  int32_t* ptok;                 // [P]
  float* pw;                     // [P]
  int32_t* apos;                 // [T k]; expert choice: [T, E] per token list entry
  float* gsc;                    // [P]
  int32_t* sched;                // backward_sched_ints
  bf16_t *Xp, *Dp;               // [P, d] (fp32 layers: float)
  float *G, *U, *dH;             // [P, f]
  bf16_t *dG, *dU, *Hw;          // [P, f] (fp32 layers: float)
  bool f32;                      // fp32 activations and weights
  // block-scaled layers: the expert inputs as the forward quantised them
  // (bf16 values, [T, d]; nullptr: x itself), and the activated rows' fp32
  // values Hf [P, f] with their MXFP8 codes hq [P, f] and scales hs [P, f / 32]
  const void* x_rows;
  float* Hf;
  uint8_t *hq, *hs;
  float* dXp;                    // [P, d]
  float* dl;                     // [T, E]
  float* rw_part;                // router_wgrad_ws_bytes
  float* dx_part;                // backward_dx_part_bytes
  // outputs (fp32)
  float *dx, *dW_g, *d_bias, *dW_gate, *dW_up, *dW_down, *dWs_gate, *dWs_up, *dWs_down;
  hipEvent_t ev_begin, ev_end;
};
long backward_pad_rows(long routed, int T, int E, int has_shared);
size_t backward_sched_ints(long routed, int T, int E, int has_shared);
size_t router_wgrad_ws_bytes(int T, int d, int E);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t s);
// block-scaled layers: MXFP8 rows -> bf16 values (same layout), and MXFP8 /
// MXFP4 weights [mats, N, K] -> bf16 values [mats, K, N]
hipError_t launch_dequant_mx_rows(const uint8_t* codes, const uint8_t* scales, long n, bf16_t* out, hipStream_t s);
hipError_t launch_dequant_mx_transpose(const void* codes, const uint8_t* scales, bool w4, int mats, int N, int K,
                                       bf16_t* out, hipStream_t s);
// fp8 weights -> bf16 values (code * per-column scale) for the backward's GEMMs
hipError_t launch_dequant_fp8(const void* codes, const float* scale, long n_mats, int R, int C, bf16_t* out,
                              hipStream_t s);
hipError_t launch_zero(float* p, long n, hipStream_t s);

// Router telemetry (optional side outputs of the layer call)
struct TelemetryArgs {
  const float* logits;           // [T, E] fp32 router logits
  const int32_t* idx;            // [T, k] chosen experts (before capacity)
  int T, E, k;
  void* ws;                      // telemetry_ws_bytes(T, E)
  int32_t* routed;               // [E] or nullptr
  float* prob_mean;              // [E] or nullptr
  float* lb_loss;                // [1] or nullptr
};
size_t telemetry_ws_bytes(int T, int E);
hipError_t launch_telemetry(const TelemetryArgs& a, hipStream_t s);

// Expert-choice routing: every expert takes its C best tokens
constexpr int kEcMaxT = 8192;
struct ExpertChoiceArgs {
  const float* logits;           // [T, E] fp32 router logits
  int T, E, C, renormalize;
  float* scores;                 // ws [E, T] fp32 full-softmax scores
  int32_t* pos;                  // [T, E] row of (t, e) or -1
  int32_t* crow;                 // [T, E] per token: rows of its experts, ascending expert order
  float* w;                      // [T, E] per token: the matching combine weights
  int32_t* ccount;               // [T] experts that took the token
  int32_t* sorted_tokens;        // [E*C] permuted row -> token
  int32_t* offsets;              // [E + 1] = e * C
  int32_t* counts;               // [E] or nullptr: C per expert
  int32_t* n_unchosen;           // [1] tokens no expert chose
};
hipError_t launch_expert_choice(const ExpertChoiceArgs& a, hipStream_t s);
struct EcCombineArgs {
  const float* y;                // [E*C (+T), d]
  const int32_t* crow;
  const float* w;
  const int32_t* ccount;
  int T, d, E, routed_rows, has_shared;
  bool act_f32;
  void* out;
};
hipError_t launch_ec_combine(const EcCombineArgs& a, hipStream_t s);

}  // namespace moe
