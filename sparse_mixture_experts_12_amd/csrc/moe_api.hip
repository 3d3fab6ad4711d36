// C ABI of the MoE layer library (declared in include/moe.h): argument
// validation, workspace layout and kernel sequencing.  No device memory is
// allocated here and the host never waits on the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

using namespace moe;

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t routed_rows_of(const moe_desc* d);

moe_status check_desc(const moe_desc* d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
  if (d->T < 0) return fail(MOE_ERR_INVALID_ARG, "T=%d < 0", d->T);
  if (d->d < 64 || d->d % 64) return fail(MOE_ERR_INVALID_ARG, "d=%d must be a positive multiple of 64", d->d);
  if (d->f < 64 || d->f % 64) return fail(MOE_ERR_INVALID_ARG, "f=%d must be a positive multiple of 64", d->f);
  if (d->E < 1 || d->E > kMaxExperts - 1) return fail(MOE_ERR_INVALID_ARG, "E=%d outside 1..%d", d->E, kMaxExperts - 1);
  const int kmax = d->E < kMaxTopK ? d->E : kMaxTopK;
  if (d->top_k < 1 || d->top_k > kmax) return fail(MOE_ERR_INVALID_ARG, "top_k=%d outside 1..%d", d->top_k, kmax);
  if (d->renormalize != 0 && d->renormalize != 1) return fail(MOE_ERR_INVALID_ARG, "renormalize must be 0 or 1");
  if (d->has_shared != 0 && d->has_shared != 1) return fail(MOE_ERR_INVALID_ARG, "has_shared must be 0 or 1");
  if (!(d->capacity_factor >= 0.f) || !isfinite(d->capacity_factor))
    return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite and >= 0");
  if (d->path < MOE_PATH_AUTO || d->path > MOE_PATH_FUSED_DECODE) return fail(MOE_ERR_INVALID_ARG, "bad path");
  if ((long long)d->T * d->top_k > (1LL << 24)) return fail(MOE_ERR_INVALID_ARG, "T*top_k too large");
  const int a = d->act_dtype, w = d->w_dtype;
  if (a != MOE_F32 && a != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "bad act_dtype %d", a);
  if (w != MOE_F32 && w != MOE_BF16 && w != MOE_FP8_E4M3 && w != MOE_MXFP8 && w != MOE_MXFP4)
    return fail(MOE_ERR_INVALID_ARG, "bad w_dtype %d", w);
  const bool mx = w == MOE_MXFP8 || w == MOE_MXFP4;
  const bool ok = (a == MOE_F32 && w == MOE_F32) || (a == MOE_BF16 && (w == MOE_BF16 || w == MOE_FP8_E4M3 || mx));
  if (!ok) return fail(MOE_ERR_UNSUPPORTED, "dtype pair act=%d w=%d not supported", a, w);
  if (mx) {
    if (d->d % 128 || d->f % 128)
      return fail(MOE_ERR_UNSUPPORTED, "MX layers take d and f multiples of 128 (d=%d f=%d)", d->d, d->f);
    if (d->path == MOE_PATH_FUSED_DECODE) return fail(MOE_ERR_UNSUPPORTED, "MX layers run on the grouped path");
  }
  if (d->routing != MOE_ROUTING_TOKEN_CHOICE && d->routing != MOE_ROUTING_EXPERT_CHOICE)
    return fail(MOE_ERR_INVALID_ARG, "bad routing %d", d->routing);
  if (mx) {   // the block-scaled kernels address code rows with 32-bit offsets
    const double rows = (double)routed_rows_of(d) + (double)d->T;
    if ((double)d->T * d->d >= 2147483648.0 || rows * d->f >= 2147483648.0)
      return fail(MOE_ERR_UNSUPPORTED, "MX layer too large (T*d and rows*f must stay below 2^31)");
  }
  if (d->routing == MOE_ROUTING_EXPERT_CHOICE) {
    if (d->path == MOE_PATH_FUSED_DECODE)
      return fail(MOE_ERR_UNSUPPORTED, "expert-choice routing runs on the grouped path");
    if (d->T > MOE_EXPERT_CHOICE_MAX_T)
      return fail(MOE_ERR_UNSUPPORTED, "expert-choice routing takes T <= %d (T=%d)", MOE_EXPERT_CHOICE_MAX_T, d->T);
  }
  if (d->path == MOE_PATH_FUSED_DECODE) {
    if (d->T > MOE_FUSED_DECODE_MAX_T)
      return fail(MOE_ERR_UNSUPPORTED, "fused decode path takes T <= %d (T=%d)", MOE_FUSED_DECODE_MAX_T, d->T);
    if (a != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "fused decode path takes bf16 activations");
  }
  return MOE_OK;
}

#define REQ(p, name)                                                                    \
  do {                                                                                  \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);                     \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s not 16-byte aligned", name); \
  } while (0)
#define OPT(p, name)                                                                             \
  do {                                                                                           \
    if ((p) && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s not 16-byte aligned", name); \
  } while (0)

moe_status check_router_weights(const moe_weights* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  REQ(w->W_g, "W_g");
  OPT(w->router_bias, "router_bias");
  return MOE_OK;
}

moe_status check_expert_weights(const moe_desc* d, const moe_weights* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  REQ(w->W_gate, "W_gate");
  REQ(w->W_up, "W_up");
  REQ(w->W_down, "W_down");
  const bool fp8 = d->w_dtype == MOE_FP8_E4M3;
  const bool mx = d->w_dtype == MOE_MXFP8 || d->w_dtype == MOE_MXFP4;
  if (fp8) {
    REQ(w->s_gate, "s_gate");
    REQ(w->s_up, "s_up");
    REQ(w->s_down, "s_down");
  }
  if (mx) {
    REQ(w->mx_gate, "mx_gate");
    REQ(w->mx_up, "mx_up");
    REQ(w->mx_down, "mx_down");
  }
  if (d->has_shared) {
    REQ(w->Ws_gate, "Ws_gate");
    REQ(w->Ws_up, "Ws_up");
    REQ(w->Ws_down, "Ws_down");
    if (fp8) {
      REQ(w->ss_gate, "ss_gate");
      REQ(w->ss_up, "ss_up");
      REQ(w->ss_down, "ss_down");
    }
    if (mx) {
      REQ(w->mxs_gate, "mxs_gate");
      REQ(w->mxs_up, "mxs_up");
      REQ(w->mxs_down, "mxs_down");
    }
  }
  return MOE_OK;
}

bool expert_choice(const moe_desc* d) { return d->routing == MOE_ROUTING_EXPERT_CHOICE; }

// Tokens every expert takes under expert-choice routing.
int ec_capacity_of(const moe_desc* d) {
  const double cf = d->capacity_factor > 0.f ? (double)d->capacity_factor : 1.0;
  const double c = ceil(cf * (double)d->T * (double)d->top_k / (double)d->E);
  const double cmax = d->T > 0 ? (double)d->T : 1.0;
  return c < 1.0 ? 1 : (int)(c > cmax ? cmax : c);
}

// Routed rows of the grouped FFN (before the shared expert's T rows).
size_t routed_rows_of(const moe_desc* d) {
  return expert_choice(d) ? (size_t)d->E * ec_capacity_of(d) : (size_t)d->T * d->top_k;
}

int capacity_of(const moe_desc* d) {
  if (expert_choice(d)) return ec_capacity_of(d);
  if (!(d->capacity_factor > 0.f)) return -1;
  const double c = ceil((double)d->capacity_factor * (double)d->T * (double)d->top_k / (double)d->E);
  return c < 1.0 ? 1 : (int)c;
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Layout {
  size_t part, idx, w, plan, counts, offsets, sorted, inv, ndrop, rank, sched, h, hs, xq, xs, y, ypart, partial, logits,
      tel;
  size_t ec_scores, ec_pos, ec_w, ec_crow, ec_count, ec_sorted, ec_offsets, total;
};

bool decode_capable(const moe_desc* d) {
  return d->T <= MOE_FUSED_DECODE_MAX_T && d->act_dtype == MOE_BF16 &&
         (d->w_dtype == MOE_BF16 || d->w_dtype == MOE_FP8_E4M3);
}

int wkind_of(const moe_desc* d);

Layout layout_of(const moe_desc* d) {
  Layout L{};
  const size_t T = d->T, k = d->top_k, E = d->E;
  const size_t routed = routed_rows_of(d);
  const size_t rows = routed + (d->has_shared ? T : 0);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += up256(bytes);
    return at;
  };
  L.part = take(router_partial_bytes(d->T, d->d, d->E));
  L.idx = take(T * k * 4);
  L.w = take(T * k * 4);
  L.plan = take((1 + E + T * k) * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted = take(T * k * 4);
  L.inv = take(T * k * 4);
  L.ndrop = take(4);
  L.rank = take(permute_ws_bytes(d->T * d->top_k, d->E));
  L.sched = take(grouped_sched_ints((int)routed, d->T, d->E, d->has_shared) * 4);
  const bool mx = d->w_dtype == MOE_MXFP8 || d->w_dtype == MOE_MXFP4;
  L.h = take(rows * d->f * (mx ? 1 : d->act_dtype == MOE_F32 ? 4 : 2));   // MXFP8: H codes
  L.hs = take(mx ? rows * (d->f / 32) : 0);                                  // MXFP8: H scales
  L.xq = take(mx ? T * d->d : 0);                                            // MXFP8: x codes
  L.xs = take(mx ? T * (d->d / 32) : 0);                                     // MXFP8: x scales
  L.y = take(rows * d->d * 4);
  L.ypart = take(grouped_down_part_bytes(d->d, d->f, d->E, d->has_shared, wkind_of(d), d->act_dtype == MOE_F32));
  L.partial = decode_capable(d) ? take(decode_partial_bytes(d->T, d->d, d->E, d->top_k, d->f, d->has_shared,
                                                           d->w_dtype == MOE_FP8_E4M3 ? W_FP8 : W_BF16))
                                : take(0);
  L.logits = take(T * E * 4);                         // router logits, for the telemetry outputs
  L.tel = take(telemetry_ws_bytes(d->T, d->E));
  const bool ec = expert_choice(d);
  L.ec_scores = take(ec ? E * T * 4 : 0);
  L.ec_pos = take(ec ? T * E * 4 : 0);
  L.ec_w = take(ec ? T * E * 4 : 0);
  L.ec_crow = take(ec ? T * E * 4 : 0);
  L.ec_count = take(ec ? T * 4 : 0);
  L.ec_sorted = take(ec ? routed * 4 : 0);
  L.ec_offsets = take(ec ? (E + 1) * 4 : 0);
  L.total = off;
  return L;
}

moe_status check_ws(const moe_desc* d, void* ws, size_t ws_bytes) {
  const size_t need = layout_of(d).total;
  if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws & 255u) return fail(MOE_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

ExpertWeights expert_weights(const moe_weights* w) {
  ExpertWeights x{};
  x.Wg = w->W_gate; x.Wu = w->W_up; x.Wd = w->W_down;
  x.sg = w->s_gate; x.su = w->s_up; x.sd = w->s_down;
  x.Wsg = w->Ws_gate; x.Wsu = w->Ws_up; x.Wsd = w->Ws_down;
  x.ssg = w->ss_gate; x.ssu = w->ss_up; x.ssd = w->ss_down;
  x.mxg = w->mx_gate; x.mxu = w->mx_up; x.mxd = w->mx_down;
  x.mxsg = w->mxs_gate; x.mxsu = w->mxs_up; x.mxsd = w->mxs_down;
  return x;
}

int wkind_of(const moe_desc* d) {
  return d->w_dtype == MOE_MXFP4 ? W_MX4 : d->w_dtype == MOE_MXFP8 ? W_MX : d->w_dtype == MOE_FP8_E4M3 ? W_FP8 : d->w_dtype == MOE_BF16 ? W_BF16 : W_F32;
}

hipEvent_t eb_of(const moe_stats* st) { return st ? st->ev_begin : nullptr; }
hipEvent_t ee_of(const moe_stats* st) { return st ? st->ev_end : nullptr; }

moe_status do_route(const moe_desc* d, const void* x, const moe_weights* w, int32_t* idx, float* tw, float* logits,
                    double* part, int32_t* plan, hipStream_t s) {
  RouteArgs a{};
  a.x = x; a.W_g = w->W_g; a.bias = w->router_bias;
  a.T = d->T; a.d = d->d; a.E = d->E; a.k = d->top_k; a.renormalize = d->renormalize;
  a.cap = expert_choice(d) ? -1 : capacity_of(d);     // token-choice capacity (decode plan)
  a.act_f32 = d->act_dtype == MOE_F32;
  a.logits = logits; a.part = part; a.idx = idx; a.w = tw; a.plan = plan;
  return hip_status(launch_route(a, s), "route");
}

moe_status do_permute(const moe_desc* d, const int32_t* idx, int32_t* counts, int32_t* offsets, int32_t* sorted,
                      int32_t* inv, int32_t* ndrop, int32_t* rank, hipStream_t s, SchedSpec sched = SchedSpec{}) {
  PermuteArgs a{};
  a.idx = idx; a.n = d->T * d->top_k; a.E = d->E; a.cap = capacity_of(d);
  a.counts = counts; a.offsets = offsets; a.sorted_assign = sorted; a.inv_perm = inv; a.n_dropped = ndrop;
  a.rank_ws = rank;
  a.sched = sched;
  return hip_status(launch_permute(a, s), "permute");
}

GroupedArgs grouped_args(const moe_desc* d, const void* x, const moe_weights* w, const int32_t* sorted,
                         const int32_t* offsets, float* y, char* ws, const Layout& L, hipEvent_t eb, hipEvent_t ee) {
  GroupedArgs a{};
  a.x = x; a.sorted_assign = sorted; a.offsets = offsets; a.w = expert_weights(w);
  a.T = d->T; a.d = d->d; a.E = d->E; a.k = d->top_k; a.f = d->f; a.has_shared = d->has_shared;
  a.routed_rows = (int)routed_rows_of(d);
  a.assign_div = expert_choice(d) ? 1 : d->top_k;
  {
    // a token takes an expert at most once, so no group exceeds T rows; capacity caps routed groups
    const int cap = capacity_of(d);
    a.max_group_rows = cap > 0 && cap < d->T ? cap : d->T;
    if (d->has_shared && d->T > a.max_group_rows) a.max_group_rows = d->T;
  }
  a.wkind = wkind_of(d);
  a.act_f32 = d->act_dtype == MOE_F32;
  a.y = y;
  a.h = ws + L.h;
  a.mx_hs = (uint8_t*)(ws + L.hs);
  a.mx_xq = (uint8_t*)(ws + L.xq);
  a.mx_xs = (uint8_t*)(ws + L.xs);
  a.sched = (int32_t*)(ws + L.sched);
  a.y_part = (float*)(ws + L.ypart);
  a.ev_begin = eb; a.ev_end = ee;
  return a;
}

// Set while moe_forward_noalloc runs: every launch stays on the caller's
// stream (no second stream or events are created on its behalf).
thread_local bool t_one_stream = false;

moe_status do_grouped(const moe_desc* d, const void* x, const moe_weights* w, const int32_t* sorted,
                      const int32_t* offsets, float* y, char* ws, const Layout& L, hipEvent_t eb, hipEvent_t ee,
                      hipStream_t s, bool sched_ready = false) {
  GroupedArgs a = grouped_args(d, x, w, sorted, offsets, y, ws, L, eb, ee);
  a.sched_ready = sched_ready;
  a.concurrent = !t_one_stream;
  return hip_status(launch_grouped_ffn(a, s), "grouped_ffn");
}

moe_status do_combine(const moe_desc* d, const float* y, const int32_t* inv, const float* tw, void* out,
                      hipStream_t s) {
  CombineArgs a{};
  a.y = y; a.inv_perm = inv; a.w = tw; a.T = d->T; a.d = d->d; a.k = d->top_k; a.has_shared = d->has_shared;
  a.act_f32 = d->act_dtype == MOE_F32;
  a.out = out;
  return hip_status(launch_combine(a, s), "combine");
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_desc* desc) {
  if (check_desc(desc) != MOE_OK) return 0;
  return layout_of(desc).total;
}

int32_t moe_capacity(const moe_desc* desc) {
  if (check_desc(desc) != MOE_OK) return -1;
  return capacity_of(desc);
}

moe_status moe_route(const moe_desc* desc, const void* x, const moe_weights* w, int32_t* topk_idx, float* topk_w,
                     float* logits, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (expert_choice(desc))
    return fail(MOE_ERR_UNSUPPORTED, "expert-choice routing runs through moe_forward only");
  if (desc->T == 0) return MOE_OK;
  REQ(x, "x");
  REQ(topk_idx, "topk_idx");
  REQ(topk_w, "topk_w");
  OPT(logits, "logits");
  if ((st = check_router_weights(w)) != MOE_OK) return st;
  double* part = nullptr;
  if (desc->T > kDecodeMaxT) {
    if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
    part = (double*)((char*)ws + layout_of(desc).part);
  } else if (ws && ws_bytes >= moe_workspace_size(desc)) {
    part = (double*)((char*)ws + layout_of(desc).part);   // wide routers split their logits over d
  }
  return do_route(desc, x, w, topk_idx, topk_w, logits, part, nullptr, stream);
}

moe_status moe_permute(const moe_desc* desc, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_assign, int32_t* inv_perm, int32_t* n_dropped, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (expert_choice(desc))
    return fail(MOE_ERR_UNSUPPORTED, "expert-choice routing runs through moe_forward only");
  if (desc->T == 0) return MOE_OK;
  REQ(counts, "counts");
  REQ(offsets, "offsets");
  REQ(n_dropped, "n_dropped");
  REQ(topk_idx, "topk_idx");
  REQ(sorted_assign, "sorted_assign");
  REQ(inv_perm, "inv_perm");
  if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
  const Layout L = layout_of(desc);
  return do_permute(desc, topk_idx, counts, offsets, sorted_assign, inv_perm, n_dropped,
                    (int32_t*)((char*)ws + L.rank), stream);
}

moe_status moe_grouped_ffn(const moe_desc* desc, const void* x, const moe_weights* w, const int32_t* sorted_assign,
                           const int32_t* offsets, float* y_sorted, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (expert_choice(desc))
    return fail(MOE_ERR_UNSUPPORTED, "expert-choice routing runs through moe_forward only");
  if (desc->T == 0) return MOE_OK;
  REQ(x, "x");
  REQ(sorted_assign, "sorted_assign");
  REQ(offsets, "offsets");
  REQ(y_sorted, "y_sorted");
  if ((st = check_expert_weights(desc, w)) != MOE_OK) return st;
  if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
  return do_grouped(desc, x, w, sorted_assign, offsets, y_sorted, (char*)ws, layout_of(desc), nullptr, nullptr,
                    stream);
}

moe_status moe_combine(const moe_desc* desc, const float* y_sorted, const int32_t* inv_perm, const float* topk_w,
                       void* out, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (expert_choice(desc))
    return fail(MOE_ERR_UNSUPPORTED, "expert-choice routing runs through moe_forward only");
  if (desc->T == 0) return MOE_OK;
  REQ(y_sorted, "y_sorted");
  REQ(inv_perm, "inv_perm");
  REQ(topk_w, "topk_w");
  REQ(out, "out");
  return do_combine(desc, y_sorted, inv_perm, topk_w, out, stream);
}

moe_status moe_forward(const moe_desc* desc, const void* x, const moe_weights* w, void* out, moe_stats* stats,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  const bool fused = !expert_choice(desc) && (desc->path == MOE_PATH_FUSED_DECODE ||
                                              (desc->path == MOE_PATH_AUTO && decode_capable(desc)));
  if (stats) stats->path_taken = fused ? MOE_PATH_FUSED_DECODE : MOE_PATH_GROUPED;
  if (desc->T == 0) return MOE_OK;
  REQ(x, "x");
  REQ(out, "out");
  if ((st = check_router_weights(w)) != MOE_OK) return st;
  if ((st = check_expert_weights(desc, w)) != MOE_OK) return st;
  if ((st = check_ws(desc, ws, ws_bytes)) != MOE_OK) return st;
  if (stats) {
    OPT(stats->d_n_dropped, "stats.d_n_dropped");
    OPT(stats->d_counts, "stats.d_counts");
    OPT(stats->d_routed, "stats.d_routed");
    OPT(stats->d_prob_mean, "stats.d_prob_mean");
    OPT(stats->d_lb_loss, "stats.d_lb_loss");
  }
  char* base = (char*)ws;
  const Layout L = layout_of(desc);
  int32_t* idx = (int32_t*)(base + L.idx);
  float* tw = (float*)(base + L.w);
  if (expert_choice(desc)) {
    if (stats && (stats->d_routed || stats->d_prob_mean || stats->d_lb_loss))
      return fail(MOE_ERR_UNSUPPORTED, "router telemetry describes token-choice routing");
    float* lg = (float*)(base + L.logits);
    if ((st = do_route(desc, x, w, idx, tw, lg, (double*)(base + L.part), nullptr, stream)) != MOE_OK) return st;
    ExpertChoiceArgs a{};
    a.logits = lg; a.T = desc->T; a.E = desc->E; a.C = ec_capacity_of(desc); a.renormalize = desc->renormalize;
    a.scores = (float*)(base + L.ec_scores);
    a.pos = (int32_t*)(base + L.ec_pos);
    a.w = (float*)(base + L.ec_w);
    a.crow = (int32_t*)(base + L.ec_crow);
    a.ccount = (int32_t*)(base + L.ec_count);
    a.sorted_tokens = (int32_t*)(base + L.ec_sorted);
    a.offsets = (int32_t*)(base + L.ec_offsets);
    a.counts = stats ? stats->d_counts : nullptr;
    a.n_unchosen = (stats && stats->d_n_dropped) ? stats->d_n_dropped : (int32_t*)(base + L.ndrop);
    if ((st = hip_status(launch_expert_choice(a, stream), "expert choice")) != MOE_OK) return st;
    float* y = (float*)(base + L.y);
    if ((st = do_grouped(desc, x, w, a.sorted_tokens, a.offsets, y, base, L, eb_of(stats), ee_of(stats), stream)) !=
        MOE_OK)
      return st;
    EcCombineArgs c{};
    c.y = y; c.crow = a.crow; c.w = a.w; c.ccount = a.ccount; c.T = desc->T; c.d = desc->d; c.E = desc->E;
    c.routed_rows = (int)routed_rows_of(desc); c.has_shared = desc->has_shared;
    c.act_f32 = desc->act_dtype == MOE_F32; c.out = out;
    return hip_status(launch_ec_combine(c, stream), "expert-choice combine");
  }
  const bool telemetry = stats && (stats->d_routed || stats->d_prob_mean || stats->d_lb_loss);
  float* logits = telemetry ? (float*)(base + L.logits) : nullptr;
  auto run_telemetry = [&]() -> moe_status {
    if (!telemetry) return MOE_OK;
    TelemetryArgs t{};
    t.logits = logits; t.idx = idx; t.T = desc->T; t.E = desc->E; t.k = desc->top_k;
    t.ws = base + L.tel;
    t.routed = stats->d_routed; t.prob_mean = stats->d_prob_mean; t.lb_loss = stats->d_lb_loss;
    return hip_status(launch_telemetry(t, stream), "telemetry");
  };
  hipEvent_t eb = stats ? stats->ev_begin : nullptr;
  hipEvent_t ee = stats ? stats->ev_end : nullptr;

  if (fused) {
    int32_t* plan = (int32_t*)(base + L.plan);
    if ((st = do_route(desc, x, w, idx, tw, logits, (double*)(base + L.part), plan, stream)) != MOE_OK) return st;
    if ((st = run_telemetry()) != MOE_OK) return st;
    DecodeArgs a{};
    a.x = x; a.plan = plan; a.topk_w = tw; a.w = expert_weights(w);
    a.T = desc->T; a.d = desc->d; a.E = desc->E; a.k = desc->top_k; a.f = desc->f;
    a.has_shared = desc->has_shared; a.wkind = wkind_of(desc); a.act_f32 = false;
    a.partial = (float*)(base + L.partial);
    a.out = out;
    a.ev_begin = eb; a.ev_end = ee;
    if ((st = hip_status(launch_decode(a, stream), "fused decode")) != MOE_OK) return st;
    if (stats && (stats->d_n_dropped || stats->d_counts)) {
      // the decode path does not build the permutation; derive the stats from it
      int32_t* counts = stats->d_counts ? stats->d_counts : (int32_t*)(base + L.counts);
      int32_t* nd = stats->d_n_dropped ? stats->d_n_dropped : (int32_t*)(base + L.ndrop);
      return do_permute(desc, idx, counts, (int32_t*)(base + L.offsets), (int32_t*)(base + L.sorted),
                        (int32_t*)(base + L.inv), nd, (int32_t*)(base + L.rank), stream);
    }
    return MOE_OK;
  }
  if ((st = do_route(desc, x, w, idx, tw, logits, (double*)(base + L.part), nullptr, stream)) != MOE_OK) return st;
  if ((st = run_telemetry()) != MOE_OK) return st;
  int32_t* counts = (stats && stats->d_counts) ? stats->d_counts : (int32_t*)(base + L.counts);
  int32_t* nd = (stats && stats->d_n_dropped) ? stats->d_n_dropped : (int32_t*)(base + L.ndrop);
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* sorted = (int32_t*)(base + L.sorted);
  int32_t* inv = (int32_t*)(base + L.inv);
  float* y = (float*)(base + L.y);
  // the permutation also writes the grouped GEMMs' tile schedule (one launch fewer)
  const SchedSpec sched = grouped_sched_spec(grouped_args(desc, x, w, sorted, offsets, y, base, L, eb, ee));
  if ((st = do_permute(desc, idx, counts, offsets, sorted, inv, nd, (int32_t*)(base + L.rank), stream, sched)) !=
      MOE_OK)
    return st;
  if ((st = do_grouped(desc, x, w, sorted, offsets, y, base, L, eb, ee, stream, true)) != MOE_OK) return st;
  return do_combine(desc, y, inv, tw, out, stream);
}

}  // extern "C"

// Scratch of the allocation-free entry point: one copy per GPU, created with
// the code object and held until the process ends.  Host code never passes
// `scratch` itself to a kernel (in host code it names a host-side stand-in);
// it uses the device address looked up per device below.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on the first call made
// with that device current.
moe_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d outside 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    if (!ptr || ((uintptr_t)ptr & 255u)) return fail(MOE_ERR_HIP, "scratch address %p not 256-byte aligned", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_desc* desc, const void* x, const moe_weights* w, void* out,
                                          moe_stats* stats, hipStream_t stream) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  const size_t need = layout_of(desc).total;
  if (need > MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_UNSUPPORTED, "layer needs %zu bytes of scratch; the allocation-free entry point holds %zu",
                need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = noalloc_scratch(&ws)) != MOE_OK) return st;
  t_one_stream = true;
  st = moe_forward(desc, x, w, out, stats, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
  t_one_stream = false;
  return st;
}

namespace {

moe_status check_backward_desc(const moe_desc* d) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  const bool bf = d->act_dtype == MOE_BF16 && (d->w_dtype == MOE_BF16 || d->w_dtype == MOE_FP8_E4M3 ||
                                               d->w_dtype == MOE_MXFP8 || d->w_dtype == MOE_MXFP4);
  const bool f32 = d->act_dtype == MOE_F32 && d->w_dtype == MOE_F32;
  if (!bf && !f32)
    return fail(MOE_ERR_UNSUPPORTED, "the backward takes bf16 activations with bf16, fp8, MXFP8 or MXFP4 weights, "
                "or fp32 layers");
  const double P = (double)backward_pad_rows((long)routed_rows_of(d), d->T, d->E, d->has_shared);
  if (P * (d->f > d->d ? d->f : d->d) >= 2147483648.0)
    return fail(MOE_ERR_UNSUPPORTED, "layer too large for the backward (padded rows * max(d, f) >= 2^31)");
  return MOE_OK;
}

struct BwdLayout {
  size_t part, idx, w, logits, counts, offsets, sorted, inv, ndrop, rank;
  size_t ec_scores, ec_pos, ec_w, ec_crow, ec_count;
  size_t wq_gate, wq_up, wq_down, wqs_gate, wqs_up, wqs_down;   // fp8 / MX layers: bf16 weight values
  size_t mx_xq, mx_xs, mx_xv, mx_hf, mx_hq, mx_hs;              // MX layers: quantised x and H
  size_t poff, ptok, pw, apos, gsc, sched, Xp, Dp, G, U, dH, dG, dU, Hw, dXp, dl, rw, dxp, total;
};

BwdLayout bwd_layout_of(const moe_desc* d) {
  BwdLayout L{};
  const size_t T = d->T, k = d->top_k, E = d->E, D = d->d, F = d->f;
  const bool ec = expert_choice(d);
  const size_t routed = routed_rows_of(d);
  const size_t P = (size_t)backward_pad_rows((long)routed, d->T, d->E, d->has_shared);
  const size_t Gn = E + (d->has_shared ? 1 : 0);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += up256(bytes);
    return at;
  };
  L.part = take(router_partial_bytes(d->T, d->d, d->E));
  L.idx = take(T * k * 4);
  L.w = take(T * k * 4);
  L.logits = take(T * E * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.sorted = take(routed * 4);                      // expert choice: the token of every row
  L.inv = take(ec ? 0 : T * k * 4);
  L.ndrop = take(4);
  L.rank = take(ec ? 0 : permute_ws_bytes(d->T * d->top_k, d->E));
  L.ec_scores = take(ec ? E * T * 4 : 0);
  L.ec_pos = take(ec ? T * E * 4 : 0);
  L.ec_w = take(ec ? T * E * 4 : 0);
  L.ec_crow = take(ec ? T * E * 4 : 0);
  L.ec_count = take(ec ? T * 4 : 0);
  const bool mxl = d->w_dtype == MOE_MXFP8 || d->w_dtype == MOE_MXFP4;
  const bool f8 = d->w_dtype == MOE_FP8_E4M3 || mxl;
  const bool f8s = f8 && d->has_shared;
  L.wq_gate = take(f8 ? E * D * F * 2 : 0);
  L.wq_up = take(f8 ? E * D * F * 2 : 0);
  L.wq_down = take(f8 ? E * D * F * 2 : 0);
  L.wqs_gate = take(f8s ? D * F * 2 : 0);
  L.wqs_up = take(f8s ? D * F * 2 : 0);
  L.wqs_down = take(f8s ? D * F * 2 : 0);
  L.mx_xq = take(mxl ? T * D : 0);
  L.mx_xs = take(mxl ? T * D / 32 : 0);
  L.mx_xv = take(mxl ? T * D * 2 : 0);
  L.mx_hf = take(mxl ? P * F * 4 : 0);
  L.mx_hq = take(mxl ? P * F : 0);
  L.mx_hs = take(mxl ? P * F / 32 : 0);
  L.poff = take((Gn + 1) * 4);
  L.ptok = take(P * 4);
  L.pw = take(P * 4);
  L.apos = take((ec ? T * E : T * k) * 4);
  L.gsc = take(P * 4);
  L.sched = take(backward_sched_ints((long)routed, d->T, d->E, d->has_shared) * 4);
  const size_t ea = d->act_dtype == MOE_F32 ? 4 : 2;    // gathered rows and the SwiGLU backward's outputs
  L.Xp = take(P * D * ea);
  L.Dp = take(P * D * ea);
  L.G = take(P * F * 4);
  L.U = take(P * F * 4);
  L.dH = take(P * F * 4);
  L.dG = take(P * F * ea);
  L.dU = take(P * F * ea);
  L.Hw = take(P * F * ea);
  L.dXp = take(P * D * 4);
  L.dl = take(T * E * 4);
  L.rw = take(router_wgrad_ws_bytes(d->T, d->d, d->E));
  L.dxp = take(backward_dx_part_bytes(d->d, d->f, (int)Gn));
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t moe_backward_workspace_size(const moe_desc* desc) {
  if (check_backward_desc(desc) != MOE_OK) return 0;
  return bwd_layout_of(desc).total;
}

moe_status moe_backward(const moe_desc* desc, const void* x, const moe_weights* w, const void* dout,
                        const moe_grads* g, void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_backward_desc(desc);
  if (st != MOE_OK) return st;
  if (!g) return fail(MOE_ERR_INVALID_ARG, "grads is NULL");
  REQ(g->dW_g, "grads.dW_g");
  REQ(g->dW_gate, "grads.dW_gate");
  REQ(g->dW_up, "grads.dW_up");
  REQ(g->dW_down, "grads.dW_down");
  OPT(g->d_bias, "grads.d_bias");
  if (desc->has_shared) {
    REQ(g->dWs_gate, "grads.dWs_gate");
    REQ(g->dWs_up, "grads.dWs_up");
    REQ(g->dWs_down, "grads.dWs_down");
  }
  if ((st = check_router_weights(w)) != MOE_OK) return st;
  if ((st = check_expert_weights(desc, w)) != MOE_OK) return st;
  const size_t E = desc->E, D = desc->d, F = desc->f;
  if (desc->T == 0) {   // an empty batch: zero weight gradients
    hipError_t e = launch_zero(g->dW_g, (long)(D * E), stream);
    if (e == hipSuccess) e = launch_zero(g->d_bias, (long)E, stream);
    if (e == hipSuccess) e = launch_zero(g->dW_gate, (long)(E * D * F), stream);
    if (e == hipSuccess) e = launch_zero(g->dW_up, (long)(E * D * F), stream);
    if (e == hipSuccess) e = launch_zero(g->dW_down, (long)(E * D * F), stream);
    if (desc->has_shared) {
      if (e == hipSuccess) e = launch_zero(g->dWs_gate, (long)(D * F), stream);
      if (e == hipSuccess) e = launch_zero(g->dWs_up, (long)(D * F), stream);
      if (e == hipSuccess) e = launch_zero(g->dWs_down, (long)(D * F), stream);
    }
    return hip_status(e, "zero gradients");
  }
  REQ(x, "x");
  REQ(dout, "dout");
  REQ(g->dx, "grads.dx");
  const BwdLayout L = bwd_layout_of(desc);
  if (ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, L.total);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)ws & 255u) return fail(MOE_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  char* base = (char*)ws;
  int32_t* idx = (int32_t*)(base + L.idx);
  float* tw = (float*)(base + L.w);
  float* logits = (float*)(base + L.logits);
  if ((st = do_route(desc, x, w, idx, tw, logits, (double*)(base + L.part), nullptr, stream)) != MOE_OK) return st;
  int32_t* offsets = (int32_t*)(base + L.offsets);
  int32_t* sorted = (int32_t*)(base + L.sorted);
  int32_t* inv = (int32_t*)(base + L.inv);
  BackwardArgs a{};
  if (expert_choice(desc)) {                      // the forward's selection, recomputed
    ExpertChoiceArgs e{};
    e.logits = logits; e.T = desc->T; e.E = desc->E; e.C = ec_capacity_of(desc); e.renormalize = desc->renormalize;
    e.scores = (float*)(base + L.ec_scores);
    e.pos = (int32_t*)(base + L.ec_pos);
    e.w = (float*)(base + L.ec_w);
    e.crow = (int32_t*)(base + L.ec_crow);
    e.ccount = (int32_t*)(base + L.ec_count);
    e.sorted_tokens = sorted;
    e.offsets = offsets;
    e.counts = nullptr;
    e.n_unchosen = (int32_t*)(base + L.ndrop);
    if ((st = hip_status(launch_expert_choice(e, stream), "expert choice")) != MOE_OK) return st;
    a.ec_C = e.C; a.ec_scores = e.scores; a.ec_pos = e.pos; a.ec_crow = e.crow; a.ec_w = e.w; a.ec_count = e.ccount;
  } else if ((st = do_permute(desc, idx, (int32_t*)(base + L.counts), offsets, sorted, inv,
                              (int32_t*)(base + L.ndrop), (int32_t*)(base + L.rank), stream)) != MOE_OK) {
    return st;
  }
  a.x = x; a.dout = dout; a.W_g = w->W_g; a.w = expert_weights(w);
  if (desc->w_dtype == MOE_FP8_E4M3) {            // the GEMMs run on the weights' values in bf16
    ExpertWeights v{};
    v.Wg = base + L.wq_gate; v.Wu = base + L.wq_up; v.Wd = base + L.wq_down;
    hipError_t e = launch_dequant_fp8(w->W_gate, w->s_gate, (long)E, (int)D, (int)F, (bf16_t*)v.Wg, stream);
    if (e == hipSuccess) e = launch_dequant_fp8(w->W_up, w->s_up, (long)E, (int)D, (int)F, (bf16_t*)v.Wu, stream);
    if (e == hipSuccess) e = launch_dequant_fp8(w->W_down, w->s_down, (long)E, (int)F, (int)D, (bf16_t*)v.Wd, stream);
    if (desc->has_shared) {
      v.Wsg = base + L.wqs_gate; v.Wsu = base + L.wqs_up; v.Wsd = base + L.wqs_down;
      if (e == hipSuccess) e = launch_dequant_fp8(w->Ws_gate, w->ss_gate, 1, (int)D, (int)F, (bf16_t*)v.Wsg, stream);
      if (e == hipSuccess) e = launch_dequant_fp8(w->Ws_up, w->ss_up, 1, (int)D, (int)F, (bf16_t*)v.Wsu, stream);
      if (e == hipSuccess) e = launch_dequant_fp8(w->Ws_down, w->ss_down, 1, (int)F, (int)D, (bf16_t*)v.Wsd, stream);
    }
    if ((st = hip_status(e, "fp8 weight values")) != MOE_OK) return st;
    a.w = v;
  } else if (desc->w_dtype == MOE_MXFP8 || desc->w_dtype == MOE_MXFP4) {
    // the GEMMs run on the weights' values in bf16 (exact: at most 4 significant
    // bits times a power of two), laid out input-major as for bf16 layers; the
    // expert inputs and the activated rows are quantised as the forward did
    const bool w4 = desc->w_dtype == MOE_MXFP4;
    ExpertWeights v{};
    v.Wg = base + L.wq_gate; v.Wu = base + L.wq_up; v.Wd = base + L.wq_down;
    hipError_t e = launch_dequant_mx_transpose(w->W_gate, w->mx_gate, w4, (int)E, (int)F, (int)D, (bf16_t*)v.Wg, stream);
    if (e == hipSuccess)
      e = launch_dequant_mx_transpose(w->W_up, w->mx_up, w4, (int)E, (int)F, (int)D, (bf16_t*)v.Wu, stream);
    if (e == hipSuccess)
      e = launch_dequant_mx_transpose(w->W_down, w->mx_down, w4, (int)E, (int)D, (int)F, (bf16_t*)v.Wd, stream);
    if (desc->has_shared) {
      v.Wsg = base + L.wqs_gate; v.Wsu = base + L.wqs_up; v.Wsd = base + L.wqs_down;
      if (e == hipSuccess)
        e = launch_dequant_mx_transpose(w->Ws_gate, w->mxs_gate, w4, 1, (int)F, (int)D, (bf16_t*)v.Wsg, stream);
      if (e == hipSuccess)
        e = launch_dequant_mx_transpose(w->Ws_up, w->mxs_up, w4, 1, (int)F, (int)D, (bf16_t*)v.Wsu, stream);
      if (e == hipSuccess)
        e = launch_dequant_mx_transpose(w->Ws_down, w->mxs_down, w4, 1, (int)D, (int)F, (bf16_t*)v.Wsd, stream);
    }
    uint8_t* xq = (uint8_t*)(base + L.mx_xq);
    uint8_t* xs = (uint8_t*)(base + L.mx_xs);
    if (e == hipSuccess) e = launch_mx_quantize(x, false, desc->T, desc->d, xq, xs, stream);
    if (e == hipSuccess) e = launch_dequant_mx_rows(xq, xs, (long)desc->T * desc->d, (bf16_t*)(base + L.mx_xv), stream);
    if ((st = hip_status(e, "block-scaled weight and input values")) != MOE_OK) return st;
    a.w = v;
    a.x_rows = base + L.mx_xv;
    a.Hf = (float*)(base + L.mx_hf);
    a.hq = (uint8_t*)(base + L.mx_hq);
    a.hs = (uint8_t*)(base + L.mx_hs);
  }
  a.T = desc->T; a.d = desc->d; a.E = desc->E; a.k = desc->top_k; a.f = desc->f;
  a.has_shared = desc->has_shared; a.renormalize = desc->renormalize;
  a.routed = (long)routed_rows_of(desc);
  a.f32 = desc->act_dtype == MOE_F32;
  a.logits = logits; a.topk_idx = idx; a.topk_w = tw; a.offsets = offsets; a.sorted_assign = sorted; a.inv_perm = inv;
  a.poff = (int32_t*)(base + L.poff); a.ptok = (int32_t*)(base + L.ptok); a.pw = (float*)(base + L.pw);
  a.apos = (int32_t*)(base + L.apos); a.gsc = (float*)(base + L.gsc); a.sched = (int32_t*)(base + L.sched);
  a.Xp = (bf16_t*)(base + L.Xp); a.Dp = (bf16_t*)(base + L.Dp);
  a.G = (float*)(base + L.G); a.U = (float*)(base + L.U); a.dH = (float*)(base + L.dH);
  a.dG = (bf16_t*)(base + L.dG); a.dU = (bf16_t*)(base + L.dU); a.Hw = (bf16_t*)(base + L.Hw);
  a.dXp = (float*)(base + L.dXp); a.dl = (float*)(base + L.dl); a.rw_part = (float*)(base + L.rw);
  a.dx_part = (float*)(base + L.dxp);
  a.dx = g->dx; a.dW_g = g->dW_g; a.d_bias = g->d_bias; a.dW_gate = g->dW_gate; a.dW_up = g->dW_up;
  a.dW_down = g->dW_down; a.dWs_gate = g->dWs_gate; a.dWs_up = g->dWs_up; a.dWs_down = g->dWs_down;
  a.ev_begin = g->ev_begin; a.ev_end = g->ev_end;
  return hip_status(launch_backward(a, stream), "backward");
}

moe_status moe_quantize_mxfp8(const void* in, int32_t in_dtype, int64_t rows, int32_t cols, uint8_t* codes,
                              uint8_t* scales, hipStream_t stream) {
  if (in_dtype != MOE_F32 && in_dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "bad in_dtype %d", in_dtype);
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows=%lld < 0", (long long)rows);
  if (cols < 32 || cols % 32) return fail(MOE_ERR_INVALID_ARG, "cols=%d must be a positive multiple of 32", cols);
  if (rows > (1LL << 40) / cols) return fail(MOE_ERR_INVALID_ARG, "rows*cols too large");
  if (rows == 0) return MOE_OK;
  REQ(in, "in");
  REQ(codes, "codes");
  if (!scales) return fail(MOE_ERR_INVALID_ARG, "scales is NULL");
  return hip_status(launch_mx_quantize(in, in_dtype == MOE_F32, (long)rows, cols, codes, scales, stream),
                    "mx quantize");
}

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

}  // extern "C"
