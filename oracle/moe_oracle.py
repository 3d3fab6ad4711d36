"""CPU oracle for the routed Mixture-of-Experts SwiGLU feed-forward layer (forward and backward).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this module.  It shares no code with the HIP library and
imports nothing from it; both sides only receive the same seeded inputs.

The oracle is plain, slow and obviously correct: numpy in fp64, Python loops
over tokens and assignments, numpy's fp64 matrix product as the only library
step.  Inputs are the already-rounded tensors the GPU receives (fp32 values,
bf16 values widened exactly to fp32, or fp8 e4m3fn byte codes plus fp32 scale
factors); they are widened exactly to fp64 here.

Sources (page titles; sections named on each page):
  [MIX]  "MoE Model Architectures", Mixtral 8x7B: "Sparse MoE Block" and
         "Expert FFN" -- router gate, softmax over experts, top-k, divide the
         top-k weights by their sum, per-expert SwiGLU w2(silu(w1 x) * w3 x),
         experts with no tokens skipped, weighted outputs summed per token.
  [DSK]  same page, DeepSeek-V3: "DeepSeekMoE Architecture" (shared experts
         always computed with weight 1 and added to the routed output) and
         "Auxiliary-Loss-Free Load Balancing" (per-expert bias inside the
         router's linear map).
  [SWT]  same page, Switch Transformers "Top-1 Routing" (capacity: an expert
         takes at most `expert_capacity` tokens, overflow tokens are dropped).
  [MINI] "Faster writing: run only the chosen experts; uncap the large
         profile" (#3): only chosen experts need computing; capacity_factor 0
         means uncapped; the dropped-routing share is reported.
  [BUG]  "Current Bug: CuTeDSLMoERunner produces wrong output", root-cause
         section: expert_offsets over the permuted rows, the inclusive form
         [4, 8, 8] and the leading-zero form [0, 4, 8, 8] for counts [4, 4, 0].

Readings where the pages are silent:
  * router logit = fp32 rounding (RNE) of the fp64 sum x.W_g (+ bias), so a
    GPU that accumulates in fp64 selects the same experts (certificate below);
  * experts are selected on those fp32 logits, larger first, equal logits
    ordered by the lower expert index (the same order as the probabilities,
    which fp64 rounding or underflow could merge);
  * capacity C = max(1, ceil(cf * T * k / E)) with cf the fp32 capacity
    factor; priority is assignment order a = t*k + j; dropped assignments add
    nothing and the remaining weights are not renormalised again;
  * the shared expert has weight 1, is not counted in k and has no capacity;
  * block-scaled (MXFP8) layers quantise the token rows entering the experts
    and the activated rows before the down projection, 32 values per scale
    along the reduction axis, with the OCP MX shared-exponent rule and
    round-to-nearest-even, saturating E4M3 elements; the activated rows are
    rounded to fp32 before that decision (the GPU produces them in fp32).
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence

import numpy as np

U64 = 2.0 ** -53          # unit roundoff of fp64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# fp8 e4m3fn codes -> values (OCP 8-bit floating point format, "fn" variant:
# 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
# exponent 1111 with mantissa 111 is NaN, exponent 0000 is subnormal).
# ----------------------------------------------------------------------------
def _e4m3fn_value(c: int) -> float:
    sign = -1.0 if (c >> 7) & 1 else 1.0
    exp = (c >> 3) & 0xF
    man = c & 0x7
    if exp == 15 and man == 7:
        return math.nan
    if exp == 0:                        # subnormal: 0.mmm x 2^-6
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_E4M3FN_VALUES = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def fp8_e4m3fn_decode(codes) -> np.ndarray:
    """Value of every code: the 256 values above, looked up by code."""
    return _E4M3FN_VALUES[np.asarray(codes, dtype=np.uint8)]


def dequantize(codes, scale, channel_axis: int) -> np.ndarray:
    """Per-output-channel scaled fp8 weight: w[..., c] = value(q[..., c]) * s[c]."""
    v = fp8_e4m3fn_decode(codes)
    shape = [1] * v.ndim
    shape[channel_axis] = -1
    return v * _f64(scale).reshape(shape)


# ----------------------------------------------------------------------------
# Router  ([MIX] gate; [DSK] router bias)
# ----------------------------------------------------------------------------
def router_logits(x, W_g, bias=None, round32: bool = True) -> np.ndarray:
    """logits[t, e] = fp32( sum_i x[t, i] * W_g[i, e] (+ bias[e]) ), fp64 sum.
    round32=False keeps the fp64 sum (smooth in x and W_g, for derivative checks)."""
    s = _f64(x) @ _f64(W_g)
    if bias is not None:
        s = s + _f64(bias)[None, :]
    return s.astype(np.float32) if round32 else s


def softmax_rows(logits32) -> np.ndarray:
    """Softmax over the experts of each token, fp64 ([MIX] softmax over dim 1)."""
    l = _f64(logits32)
    p = np.empty_like(l)
    for t in range(l.shape[0]):
        m = max(l[t])
        e = np.array([math.exp(v - m) for v in l[t]])
        p[t] = e / math.fsum(e)
    return p


def topk_select(logits32, k: int) -> np.ndarray:
    """Per token, the k experts of largest fp32 router logit, largest first;
    equal logits ordered by the lower expert index ([MIX] topk of the softmax).
    Softmax is strictly increasing in the logit, so these are the top-k
    probabilities; ranking the fp32 logits themselves keeps apart experts whose
    fp64 probabilities round (or underflow) to the same value."""
    l = _f64(logits32)
    T, E = l.shape
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-l[t, e], e))
        idx[t] = order[:k]
    return idx


def routing_weights(probs, idx, renormalize: bool) -> np.ndarray:
    """Top-k probabilities, divided by their sum when renormalising (the step
    after the top-k in [MIX] "Sparse MoE Block"; [DSK] does the same)."""
    T, k = idx.shape
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        sel = [probs[t, e] for e in idx[t]]
        den = math.fsum(sel) if renormalize else 1.0
        w[t] = [v / den for v in sel]
    return w


# ----------------------------------------------------------------------------
# Capacity and token-to-expert permutation ([SWT] capacity, [MINI] cf 0 =
# uncapped, [MIX] per-expert gather order, [BUG] expert_offsets)
# ----------------------------------------------------------------------------
def capacity(T: int, k: int, E: int, capacity_factor) -> Optional[int]:
    cf = float(np.float32(capacity_factor))
    if not cf > 0.0:
        return None
    return max(1, math.ceil(cf * T * k / E))


def permute(idx, E: int, cap: Optional[int]) -> dict:
    """Group assignments a = t*k + j by expert, keeping ascending a inside an
    expert (the order in which the per-expert loop of [MIX] finds them), and
    drop an assignment once its expert already holds `cap` earlier ones.

    counts[e]        kept assignments of expert e
    offsets[E + 1]   exclusive prefix of counts with a leading 0 ([BUG] form)
    sorted_assign    kept assignment ids, expert-major, ascending a inside
    inv_perm[a]      position of a in sorted_assign, or -1 when dropped
    n_dropped        number of dropped assignments
    """
    T, k = idx.shape
    flat = [int(v) for v in np.asarray(idx).reshape(-1)]
    buckets = [[] for _ in range(E)]
    dropped = 0
    for a, e in enumerate(flat):
        if cap is None or len(buckets[e]) < cap:
            buckets[e].append(a)
        else:
            dropped += 1
    counts = np.array([len(b) for b in buckets], dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    sorted_assign = np.array([a for b in buckets for a in b], dtype=np.int32)
    inv_perm = np.full(T * k, -1, dtype=np.int32)
    for pos, a in enumerate(sorted_assign):
        inv_perm[a] = pos
    return dict(counts=counts, offsets=offsets, sorted_assign=sorted_assign,
                inv_perm=inv_perm, n_dropped=dropped)


# ----------------------------------------------------------------------------
# Expert FFN ([MIX] "Expert FFN": w2(silu(w1 x) * w3 x), no biases).  Weights
# are stored input-major: W_gate = w1 and W_up = w3 as [d, f], W_down = w2 as
# [f, d], so a row vector x maps to x @ W.
# ----------------------------------------------------------------------------
def silu(z) -> np.ndarray:
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X, W_gate, W_up, W_down, quant_h=None) -> np.ndarray:
    """SwiGLU expert; quant_h (optional) maps the activated rows H to the
    values the down projection sees (block-scaled layers quantise them)."""
    X = _f64(X)
    G = X @ _f64(W_gate)
    U = X @ _f64(W_up)
    H = silu(G) * U
    if quant_h is not None:
        H = quant_h(H)
    return H @ _f64(W_down)


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------
ExpertFn = Callable[[int], Sequence[np.ndarray]]


def forward(x, W_g, bias, k: int, renormalize: bool, capacity_factor,
            expert: ExpertFn, E: int, shared: Optional[Sequence[np.ndarray]] = None,
            tokens: Optional[Sequence[int]] = None, quant_x=None, quant_h=None,
            round_logits: bool = True) -> dict:
    """Routed MoE SwiGLU layer.

    expert(e) returns (W_gate[d,f], W_up[d,f], W_down[f,d]) of expert e as
    arrays widened to fp64 by the caller's choice (fp8 callers pass the
    dequantized values).  `shared` is the shared expert's triple or None.
    Routing and permutation are computed for every token; the expert FFN and
    the weighted sum only for `tokens` (all when None), so large layers can be
    checked on a sample.  out rows follow the order of `tokens`.
    quant_x / quant_h (optional) map the token rows entering the experts and
    the activated intermediate rows to the values a block-scaled layer sees;
    routing always uses the unquantised x.  round_logits=False skips the fp32
    rounding of the router logits (derivative checks only).
    """
    x = _f64(x)
    T = x.shape[0]
    logits = router_logits(x, W_g, bias, round_logits)
    probs = softmax_rows(logits)
    idx = topk_select(logits, k)
    w = routing_weights(probs, idx, renormalize)
    cap = capacity(T, k, E, capacity_factor)
    perm = permute(idx, E, cap)

    toks = list(range(T)) if tokens is None else [int(t) for t in tokens]
    want = set(toks)
    y_assign = {}                       # a -> expert output row (fp64)
    offs, sa = perm["offsets"], perm["sorted_assign"]
    for e in range(E):
        rows = [int(a) for a in sa[offs[e]:offs[e + 1]] if int(a) // k in want]
        if not rows:                    # experts without tokens do no work ([MIX])
            continue
        X = x[[a // k for a in rows]]
        Y = expert_ffn(X if quant_x is None else quant_x(X), *expert(e), quant_h=quant_h)
        for a, y in zip(rows, Y):
            y_assign[a] = y

    out = np.zeros((len(toks), x.shape[1]), dtype=np.float64)
    for r, t in enumerate(toks):
        acc = np.zeros(x.shape[1], dtype=np.float64)
        for j in range(k):              # weighted sum in slot order
            a = t * k + j
            if perm["inv_perm"][a] >= 0:
                acc = acc + w[t, j] * y_assign[a]
        out[r] = acc
    if shared is not None:              # [DSK]: shared output + routed output
        X = x[toks]
        out = out + expert_ffn(X if quant_x is None else quant_x(X), *shared, quant_h=quant_h)
    return dict(logits=logits, probs=probs, topk_idx=idx, topk_w=w, capacity=cap,
                out=out, tokens=np.array(toks, dtype=np.int64), **perm)


# ----------------------------------------------------------------------------
# Routing certificate: the selection and slot order are the same for every
# fp64 summation order when adjacent fp64 logit sums among the top k+1 are
# separated by more than both sums' worst-case error plus two fp32 ulps.
# ----------------------------------------------------------------------------
def logit_error_bound(x, W_g, bias=None) -> np.ndarray:
    """Worst-case distance between the exact router sum x.W_g (+ b) and its
    value computed in fp64 with any order of the d (+1) additions: the
    recursive-summation bound gamma_n * sum |terms| with gamma_n = n u /
    (1 - n u), n = d + 1 and u = 2^-53 (products of bf16 or fp32 values are
    exact in fp64, so only the additions round)."""
    x, W = _f64(x), _f64(W_g)
    d = x.shape[1]
    gamma = (d + 1) * U64 / (1.0 - (d + 1) * U64)
    bound = gamma * (np.abs(x) @ np.abs(W))
    if bias is not None:
        bound = bound + gamma * np.abs(_f64(bias))[None, :]
    return bound


def routing_certificate(x, W_g, bias, k: int) -> dict:
    """ok[t]: token t's top-k (and slot order) on fp32-rounded logits is the
    same for every fp64 summation order.  The fp64 sums s computed here and
    any other order's sums are each within `bound` of the exact value, so two
    experts keep their order (or tie) in every order when their computed gap
    exceeds twice both bounds plus two fp32 ulps: the ulps cover two sums on
    either side of one fp32 rounding boundary, which one order may round
    apart and another together (a tie, broken by the expert index)."""
    x, W = _f64(x), _f64(W_g)
    T = x.shape[0]
    E = W.shape[1]
    s = x @ W
    if bias is not None:
        s = s + _f64(bias)[None, :]
    bound = logit_error_bound(x, W, bias)
    ok = np.ones(T, dtype=bool)
    margin = np.full(T, np.inf)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-s[t, e], e))[:min(k + 1, E)]
        for a, b in zip(order[:-1], order[1:]):
            ulp = float(np.spacing(np.float32(max(abs(s[t, a]), abs(s[t, b])))))
            need = 2.0 * (bound[t, a] + bound[t, b]) + 2.0 * ulp
            gap = s[t, a] - s[t, b]
            margin[t] = min(margin[t], gap - need)
            if not gap > need:
                ok[t] = False
    return dict(ok=ok, margin=margin, bound=bound)


# ----------------------------------------------------------------------------
# Router telemetry: per-expert load and the Switch load-balancing loss
# ([SWT] "Load Balancing Loss"; [DSK] "Auxiliary-Loss-Free Load Balancing").
# ----------------------------------------------------------------------------
def router_telemetry(logits32, idx, E: int) -> dict:
    """Load statistics of one routing, from the fp32 logits and the chosen
    experts (before any capacity limit).

      routed[e]    number of (token, slot) assignments that chose expert e
      prob_mean[e] mean over the tokens of expert e's full softmax probability
      lb_loss      E * sum_e prob_mean[e] * routed[e] / T

    [SWT] defines the loss as E times the sum over experts of the product of
    the mean router probability and the fraction of tokens routed to the
    expert, with the fraction taken as the token-mean of the one-hot of the
    chosen index.  For k slots per token the same one-hot mean, summed over
    the slots, is routed[e] / T, which is the reading used here.  [DSK] steers
    load with a per-expert bias instead of a loss; the pages give no update
    rule, so only its input, the per-expert load, is reported."""
    probs = softmax_rows(logits32)
    T = probs.shape[0]
    routed = np.zeros(E, dtype=np.int64)
    for t in range(T):
        for e in idx[t]:
            routed[int(e)] += 1
    if T == 0:
        return {"routed": routed, "prob_mean": np.zeros(E), "lb_loss": 0.0}
    prob_mean = np.array([math.fsum(probs[:, e]) / T for e in range(E)])
    lb_loss = E * math.fsum(prob_mean[e] * routed[e] / T for e in range(E))
    return {"routed": routed, "prob_mean": prob_mean, "lb_loss": lb_loss}


# ----------------------------------------------------------------------------
# Expert-choice routing ("MoE Model Architectures", Design Patterns, Pattern 3:
# every expert selects its top tokens instead of tokens selecting experts).
# ----------------------------------------------------------------------------
def expert_choice_capacity(T: int, k: int, E: int, capacity_factor) -> int:
    """Tokens each expert takes: C = ceil(cf * T * k / E) (cf = 0 -> 1, so the
    number of (token, expert) pairs matches token choice), at least 1 and at
    most T."""
    cf = float(np.float32(capacity_factor))
    c = math.ceil((cf if cf > 0 else 1.0) * T * k / E)
    return max(1, min(T, c))


def expert_choice_routing(logits32, k: int, capacity_factor, renormalize: bool, round_scores: bool = True) -> dict:
    """Scores are the full softmax of the fp32 logits, rounded to fp32.  Expert
    e takes the C tokens of largest score (equal scores -> lower token index);
    its rows are those tokens in ascending order.  A token's weight for expert
    e is its score (divided by the sum of its scores over the experts that
    chose it when renormalising); tokens no expert chose get nothing.
    round_scores=False keeps the fp64 scores (for differentiating the layer).

    Returns capacity, offsets[E+1], sorted_tokens[E*C] (row -> token),
    pos[T, E] (row of (t, e) or -1) and weight[T, E] (0 where not chosen)."""
    probs = softmax_rows(logits32)
    s32 = probs.astype(np.float32) if round_scores else probs
    T, E = probs.shape
    C = expert_choice_capacity(T, k, E, capacity_factor) if T > 0 else 0
    pos = np.full((T, E), -1, dtype=np.int64)
    sorted_tokens = []
    offsets = [0]
    for e in range(E):
        best = sorted(range(T), key=lambda t: (-float(s32[t, e]), t))[:C]
        for t in sorted(best):
            pos[t, e] = len(sorted_tokens)
            sorted_tokens.append(t)
        offsets.append(len(sorted_tokens))
    weight = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        chosen = [e for e in range(E) if pos[t, e] >= 0]
        den = math.fsum(float(s32[t, e]) for e in chosen) if (renormalize and chosen) else 1.0
        for e in chosen:
            weight[t, e] = float(s32[t, e]) / den
    return dict(capacity=C, offsets=np.array(offsets, dtype=np.int64),
                sorted_tokens=np.array(sorted_tokens, dtype=np.int64), pos=pos, weight=weight, scores=s32)


def expert_choice_forward(x, W_g, bias, k: int, renormalize: bool, capacity_factor,
                          expert: ExpertFn, E: int, shared: Optional[Sequence[np.ndarray]] = None,
                          tokens: Optional[Sequence[int]] = None, quant_x=None, quant_h=None,
                          round_logits: bool = True) -> dict:
    """The layer with expert-choice routing: out[t] = sum over the experts that
    chose t, in ascending expert order, of weight[t, e] * FFN_e(x[t]), plus the
    shared expert.  Routing for every token; FFN and sum for `tokens`.
    quant_x / quant_h as in forward(); round_logits=False keeps the fp64
    logits and scores (for differentiating the layer)."""
    qx = (lambda X: X) if quant_x is None else quant_x
    x = _f64(x)
    T = x.shape[0]
    logits = router_logits(x, W_g, bias, round_logits)
    r = expert_choice_routing(logits, k, capacity_factor, renormalize, round_logits)
    toks = list(range(T)) if tokens is None else [int(t) for t in tokens]
    want = set(toks)
    y = {}
    for e in range(E):
        rows = [int(t) for t in r["sorted_tokens"][r["offsets"][e]:r["offsets"][e + 1]] if int(t) in want]
        if not rows:
            continue
        Y = expert_ffn(qx(x[rows]), *expert(e), quant_h=quant_h)
        for t, yy in zip(rows, Y):
            y[(t, e)] = yy
    out = np.zeros((len(toks), x.shape[1]), dtype=np.float64)
    for i, t in enumerate(toks):
        acc = np.zeros(x.shape[1], dtype=np.float64)
        for e in range(E):
            if r["pos"][t, e] >= 0:
                acc = acc + r["weight"][t, e] * y[(t, e)]
        out[i] = acc
    if shared is not None:
        out = out + expert_ffn(qx(x[toks]), *shared, quant_h=quant_h)
    return dict(logits=logits, out=out, tokens=np.array(toks, dtype=np.int64), **r)



# ----------------------------------------------------------------------------
# Backward of the token-choice layer (gradients of a scalar loss L, given
# dout = dL/dout).  Pages: "MoE Model Architectures", Mixtral "Sparse MoE
# Block" / "Expert FFN" (the forward these are the derivatives of) and
# DeepSeek-V3 "DeepSeekMoE Architecture" (shared expert, weight 1); "Testing
# using claude to graft ETHOS onto modded-nanogpt base", "Key Implementation
# Details" (a backward that recomputes the forward values and accumulates
# every weight gradient over the tokens that chose the expert); "Faster
# writing: run only the chosen experts; uncap the large profile", "Test plan"
# (the chosen-experts dispatch must give the same slot gradients as running
# every expert).
#
# The expert selection (top-k, capacity) is piecewise constant: gradients flow
# through the routing weights and the expert FFNs with the selection held
# fixed.  Readings where the pages are silent: the router logits' fp32
# rounding is differentiated as the identity; dropped assignments carry no
# gradient; the router bias gets the gradient of an additive logit term.
# ----------------------------------------------------------------------------
def dsilu(z) -> np.ndarray:
    """d/dz of z * sigmoid(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    z = _f64(z)
    s = 1.0 / (1.0 + np.exp(-z))
    return s * (1.0 + z * (1.0 - s))


def expert_ffn_backward(X, W_gate, W_up, W_down, dY, quant_h=None) -> dict:
    """Y = (silu(X Wg) * (X Wu)) Wd; given dY = dL/dY returns dX, dWg, dWu, dWd
    and H (the activated rows).  quant_h (block-scaled layers): the down
    projection sees quant_h(H), differentiated as the identity (straight
    through), so dW_down uses the quantised rows and dH passes unchanged."""
    X, dY = _f64(X), _f64(dY)
    Wg, Wu, Wd = _f64(W_gate), _f64(W_up), _f64(W_down)
    G = X @ Wg
    U = X @ Wu
    H = silu(G) * U
    if quant_h is not None:
        H = quant_h(H)
    dH = dY @ Wd.T
    dG = dH * U * dsilu(G)
    dU = dH * silu(G)
    return dict(dX=dG @ Wg.T + dU @ Wu.T, dW_gate=X.T @ dG, dW_up=X.T @ dU, dW_down=H.T @ dY, H=H)


def routing_weights_backward(probs, idx, g, renormalize: bool) -> np.ndarray:
    """dL/dlogits from g[t, j] = dL/dw[t, j].
    renormalised: w_j = exp(l_ij) / sum over the chosen l, a softmax over the
    chosen logits, so dl_(i_m) = w_m (g_m - sum_j g_j w_j), zero elsewhere;
    not renormalised: w_j = p_(i_j) with p the softmax over all E logits, so
    dl_e = p_e ([e chosen] g_(j(e)) - sum_j g_j p_(i_j))."""
    p = _f64(probs)
    T, k = idx.shape
    dl = np.zeros_like(p)
    for t in range(T):
        sel = [int(e) for e in idx[t]]
        if renormalize:
            den = math.fsum(p[t, e] for e in sel)
            w = [p[t, e] / den for e in sel]
            s = math.fsum(g[t, j] * w[j] for j in range(k))
            for j, e in enumerate(sel):
                dl[t, e] = w[j] * (g[t, j] - s)
        else:
            s = math.fsum(g[t, j] * p[t, e] for j, e in enumerate(sel))
            for e in range(p.shape[1]):
                dl[t, e] = -p[t, e] * s
            for j, e in enumerate(sel):
                dl[t, e] += p[t, e] * g[t, j]
    return dl


def backward(x, W_g, bias, k: int, renormalize: bool, capacity_factor, expert: ExpertFn, E: int,
             shared: Optional[Sequence[np.ndarray]], dout, round_logits: bool = True,
             quant_x=None, quant_h=None) -> dict:
    """Gradients of the token-choice layer of forward() for dL/dout = dout:
    dx [T,d], dW_g [d,E], d_bias [E], dW_gate/dW_up [E,d,f], dW_down [E,f,d],
    the shared expert's dWs_* (or None), and the intermediates d_logits [T,E]
    and g [T,k] = dL/dw (0 for dropped assignments).  quant_x / quant_h as in
    forward(), each differentiated as the identity (straight through)."""
    qx = (lambda X: X) if quant_x is None else quant_x
    x, W_g, dout = _f64(x), _f64(W_g), _f64(dout)
    T, d = x.shape
    logits = router_logits(x, W_g, bias, round_logits)
    probs = softmax_rows(logits)
    idx = topk_select(logits, k)
    w = routing_weights(probs, idx, renormalize)
    perm = permute(idx, E, capacity(T, k, E, capacity_factor))
    f = _f64(expert(0)[0]).shape[1]
    dx = np.zeros((T, d))
    dWg_e = np.zeros((E, d, f))
    dWu_e = np.zeros((E, d, f))
    dWd_e = np.zeros((E, f, d))
    g = np.zeros((T, k))
    offs, sa = perm["offsets"], perm["sorted_assign"]
    for e in range(E):
        rows = [int(a) for a in sa[offs[e]:offs[e + 1]]]
        if not rows:                                  # no tokens: zero gradient
            continue
        toks = [a // k for a in rows]
        Wg, Wu, Wd = expert(e)
        X = qx(x[toks])
        Y = expert_ffn(X, Wg, Wu, Wd, quant_h=quant_h)   # the unweighted expert outputs
        wt = np.array([w[a // k, a % k] for a in rows])
        b = expert_ffn_backward(X, Wg, Wu, Wd, wt[:, None] * dout[toks], quant_h=quant_h)
        dWg_e[e], dWu_e[e], dWd_e[e] = b["dW_gate"], b["dW_up"], b["dW_down"]
        for i, a in enumerate(rows):
            t, j = a // k, a % k
            dx[t] += b["dX"][i]
            g[t, j] = float(np.dot(dout[t], Y[i]))    # dL/dw of a kept assignment
    dl = routing_weights_backward(probs, idx, g, renormalize)
    dx += dl @ W_g.T
    out = dict(dx=dx, dW_g=x.T @ dl, d_bias=dl.sum(axis=0), dW_gate=dWg_e, dW_up=dWu_e, dW_down=dWd_e,
               d_logits=dl, g=g, dWs_gate=None, dWs_up=None, dWs_down=None)
    if shared is not None:
        b = expert_ffn_backward(qx(x), *shared, dout, quant_h=quant_h)
        out["dx"] = dx + b["dX"]
        out.update(dWs_gate=b["dW_gate"], dWs_up=b["dW_up"], dWs_down=b["dW_down"])
    return out


# ----------------------------------------------------------------------------
# Backward of the expert-choice layer.  Pages: "MoE Model Architectures",
# Design Patterns, Pattern 3 "Expert Choice Routing" (the forward: experts
# take their best tokens; a token's output sums the experts that took it) and
# Switch Transformers "Top-1 Routing" (scores are the router softmax); the
# backward pages as for token choice above.  The selection (which tokens each
# expert took) is held fixed, as the top-k is for token choice; the fp32
# rounding of the scores is differentiated as the identity.
# ----------------------------------------------------------------------------
def expert_choice_weights_backward(probs, pos, g, renormalize: bool) -> np.ndarray:
    """dL/dlogits from g[t, e] = dL/dweight[t, e] of the experts that took t
    (pos[t, e] >= 0).  renormalised: the weights are a softmax over the
    logits of the experts that took t, so dl_e = w_e (g_e - sum_i g_i w_i)
    for those experts and zero elsewhere; not renormalised: weight = p_e,
    the softmax over all E logits, so dl_e = p_e ([e took t] g_e - sum_i g_i p_i)
    for every e.  A token no expert took gets zero."""
    p = _f64(probs)
    T, E = p.shape
    dl = np.zeros_like(p)
    for t in range(T):
        chosen = [e for e in range(E) if pos[t, e] >= 0]
        if not chosen:
            continue
        if renormalize:
            den = math.fsum(p[t, e] for e in chosen)
            w = {e: p[t, e] / den for e in chosen}
            s = math.fsum(g[t, e] * w[e] for e in chosen)
            for e in chosen:
                dl[t, e] = w[e] * (g[t, e] - s)
        else:
            s = math.fsum(g[t, e] * p[t, e] for e in chosen)
            for e in range(E):
                dl[t, e] = -p[t, e] * s
            for e in chosen:
                dl[t, e] += p[t, e] * g[t, e]
    return dl


def expert_choice_backward(x, W_g, bias, k: int, renormalize: bool, capacity_factor, expert: ExpertFn, E: int,
                           shared: Optional[Sequence[np.ndarray]], dout, round_logits: bool = True,
                           quant_x=None, quant_h=None) -> dict:
    """Gradients of expert_choice_forward() for dL/dout = dout, with the keys
    of backward(); g is [T, E] (dL/dweight[t, e], zero where e did not take t).
    quant_x / quant_h as in backward()."""
    qx = (lambda X: X) if quant_x is None else quant_x
    x, W_g, dout = _f64(x), _f64(W_g), _f64(dout)
    T, d = x.shape
    logits = router_logits(x, W_g, bias, round_logits)
    probs = softmax_rows(logits)
    r = expert_choice_routing(logits, k, capacity_factor, renormalize, round_logits)
    f = _f64(expert(0)[0]).shape[1]
    dx = np.zeros((T, d))
    dWg_e = np.zeros((E, d, f))
    dWu_e = np.zeros((E, d, f))
    dWd_e = np.zeros((E, f, d))
    g = np.zeros((T, E))
    offs, st = r["offsets"], r["sorted_tokens"]
    for e in range(E):
        toks = [int(t) for t in st[offs[e]:offs[e + 1]]]
        if not toks:
            continue
        Wg, Wu, Wd = expert(e)
        X = qx(x[toks])
        Y = expert_ffn(X, Wg, Wu, Wd, quant_h=quant_h)   # the unweighted expert outputs
        wt = np.array([r["weight"][t, e] for t in toks])
        b = expert_ffn_backward(X, Wg, Wu, Wd, wt[:, None] * dout[toks], quant_h=quant_h)
        dWg_e[e], dWu_e[e], dWd_e[e] = b["dW_gate"], b["dW_up"], b["dW_down"]
        for i, t in enumerate(toks):
            dx[t] += b["dX"][i]
            g[t, e] = float(np.dot(dout[t], Y[i]))
    dl = expert_choice_weights_backward(probs, r["pos"], g, renormalize)
    dx += dl @ W_g.T
    out = dict(dx=dx, dW_g=x.T @ dl, d_bias=dl.sum(axis=0), dW_gate=dWg_e, dW_up=dWu_e, dW_down=dWd_e,
               d_logits=dl, g=g, dWs_gate=None, dWs_up=None, dWs_down=None, capacity=r["capacity"], pos=r["pos"])
    if shared is not None:
        b = expert_ffn_backward(qx(x), *shared, dout, quant_h=quant_h)
        out["dx"] = dx + b["dX"]
        out.update(dWs_gate=b["dW_gate"], dWs_up=b["dW_up"], dWs_down=b["dW_down"])
    return out


# ----------------------------------------------------------------------------
# MXFP8 block scaling (OCP Microscaling): E4M3 elements, one E8M0 power-of-two
# scale per 32 consecutive elements along the reduction dimension.  Page:
# "Current Bug: CuTeDSLMoERunner produces wrong output", "Root Cause: scale_a
# layout doesn't match expert_offsets" (a grouped MoE whose activations carry
# per-token block scale factors, found per expert through its row offsets; its
# NVFP4 blocks are the same idea for another chip).  The block size, element
# format and shared-exponent rule are the OCP MX ones, which the gfx950 scaled
# matrix instructions consume.
# ----------------------------------------------------------------------------
MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8               # exponent of the largest normal: 448 = 1.75 * 2^8

_E4M3_POS_CODES = np.arange(0x7F, dtype=np.uint8)             # +0 .. +448, values rise with the code
_E4M3_POS_VALS = fp8_e4m3fn_decode(_E4M3_POS_CODES)


def e4m3_encode(v) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to the even code (RNE); magnitudes
    beyond 448 saturate to 448; the sign bit is the input's (so a negative
    value that rounds to zero gives -0, code 0x80)."""
    v = _f64(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    i = np.clip(np.searchsorted(_E4M3_POS_VALS, a, side="left"), 1, len(_E4M3_POS_VALS) - 1)
    lo, hi = _E4M3_POS_VALS[i - 1], _E4M3_POS_VALS[i]
    d_lo, d_hi = a - lo, hi - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (i % 2 == 0)), i, i - 1)   # code i is even <=> i % 2 == 0
    code = np.where(a == 0.0, 0, code).astype(np.uint8)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def mx_quantize(v, block: int = MX_BLOCK):
    """Per block of `block` consecutive values along the last axis: shared
    exponent s = floor(log2(max |v|)) - 8, clamped to [-127, 127] (an all-zero
    block takes -127); elements = e4m3_encode(v / 2^s).  Returns (codes uint8,
    scales uint8 with code s + 127)."""
    v = _f64(v)
    K = v.shape[-1]
    assert K % block == 0
    b = v.reshape(-1, K // block, block)
    amax = np.abs(b).max(axis=2)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    e[nz] = np.frexp(amax[nz])[1] - 1 - E4M3_EMAX          # frexp: amax = m 2^x, m in [0.5, 1)
    e = np.clip(e, -127, 127)
    codes = e4m3_encode(b / np.exp2(e.astype(np.float64))[:, :, None])
    return codes.reshape(v.shape), (e + 127).astype(np.uint8).reshape(v.shape[:-1] + (K // block,))


def mx_dequantize(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    s = np.asarray(scales, dtype=np.uint8).astype(np.float64)
    f = np.exp2(s - 127.0)
    return fp8_e4m3fn_decode(c) * np.repeat(f, block, axis=-1)


def mx_roundtrip(v, as_fp32: bool = False) -> np.ndarray:
    """The values a block-scaled operand carries: quantise and decode.  With
    as_fp32 the input is rounded to fp32 first (an fp32 producer decides)."""
    v = _f64(v)
    if as_fp32:
        v = v.astype(np.float32).astype(np.float64)
    return mx_dequantize(*mx_quantize(v))


# ----------------------------------------------------------------------------
# MXFP4 block scaling (OCP Microscaling): E2M1 elements -- a sign, two exponent
# bits (bias 1) and one mantissa bit, i.e. 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their
# negatives -- with the same E8M0 scale per 32 values as MXFP8 and the same
# rule for it: s = floor(log2 max|v|) - emax, emax = 2 for E2M1.  The pages
# show the 4-bit block-scaled idea only as NVFP4 on another chip ("Current Bug:
# CuTeDSLMoERunner produces wrong output", Root Cause); here it is the expert
# weights' format, with the activations in MXFP8.
# ----------------------------------------------------------------------------
E2M1_MAX = 6.0
E2M1_EMAX = 2               # 6 = 1.5 * 2^2


def _e2m1_value(c: int) -> float:
    sign = -1.0 if c & 8 else 1.0
    e, m = (c >> 1) & 3, c & 1
    mag = 0.5 * m if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)   # e = 0: subnormal, m / 2
    return sign * mag


_E2M1_VALUES = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
_E2M1_POS_VALS = _E2M1_VALUES[:8]          # codes 0..7: +0 .. +6, rising with the code


def e2m1_decode(codes) -> np.ndarray:
    """Values of E2M1 codes (the low four bits of each byte)."""
    return _E2M1_VALUES[np.asarray(codes, dtype=np.uint8) & 0x0F]


def e2m1_encode(v) -> np.ndarray:
    """Nearest E2M1 value, ties to the even code; magnitudes beyond 6 saturate
    to 6; the sign bit is the input's (a negative value that rounds to zero
    gives -0, code 8).  One code (0..15) per byte."""
    v = _f64(v)
    a = np.minimum(np.abs(v), E2M1_MAX)
    i = np.clip(np.searchsorted(_E2M1_POS_VALS, a, side="left"), 1, len(_E2M1_POS_VALS) - 1)
    lo, hi = _E2M1_POS_VALS[i - 1], _E2M1_POS_VALS[i]
    d_lo, d_hi = a - lo, hi - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (i % 2 == 0)), i, i - 1)
    code = np.where(a == 0.0, 0, code).astype(np.uint8)
    return (code | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def mx4_quantize(v, block: int = MX_BLOCK):
    """Per block of `block` consecutive values along the last axis: shared
    exponent s = floor(log2(max |v|)) - 2, clamped to [-127, 127] (an all-zero
    block takes -127); elements = e2m1_encode(v / 2^s).  Returns (codes uint8,
    one E2M1 code per byte, scales uint8 with code s + 127)."""
    v = _f64(v)
    K = v.shape[-1]
    assert K % block == 0
    b = v.reshape(-1, K // block, block)
    amax = np.abs(b).max(axis=2)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    e[nz] = np.frexp(amax[nz])[1] - 1 - E2M1_EMAX
    e = np.clip(e, -127, 127)
    codes = e2m1_encode(b / np.exp2(e.astype(np.float64))[:, :, None])
    return codes.reshape(v.shape), (e + 127).astype(np.uint8).reshape(v.shape[:-1] + (K // block,))


def mx4_dequantize(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    """codes: one E2M1 code per byte (as mx4_quantize returns them)."""
    s = np.asarray(scales, dtype=np.uint8).astype(np.float64)
    return e2m1_decode(codes) * np.repeat(np.exp2(s - 127.0), block, axis=-1)
