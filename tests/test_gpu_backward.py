"""GPU parity of moe_backward against the CPU oracle, through the C ABI.

Bar: every gradient within max|gpu - oracle| / max|oracle| <= 2e-2 (the bf16
bar), experts without tokens exactly zero, results bitwise reproducible.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import OracleInputs, assert_close, device_inputs, ec_boundary_is_clear, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_mixture_experts_12_amd import _lib as ops
else:  # collected on CPU hosts but never run there (marker)
    ops = None

C = synth.CONFIGS
TOL = 2e-2          # bf16 (and fp8-weight) layers
TOL_F32 = 1e-5      # fp32 layers
TOL_MX = 6e-2       # block-scaled layers (the forward's MXFP8 bar: H is requantised)


def _tol(cfg):
    return TOL_F32 if cfg.act == "f32" else TOL_MX if cfg.wdt in ("mxfp8", "mxfp4") else TOL

CASES = {
    "prefill": C["mixtral_prefill"].with_(T=300, d=256, f=512, seed=40),
    "renorm_off_shared_cap": C["fine_grained"].with_(T=120, d=256, E=16, k=4, f=256, renormalize=False,
                                                     capacity_factor=1.0, seed=41),
    "finegrained_shared": C["fine_grained"].with_(T=96, d=512, E=32, f=256, seed=42),
    "big_tiles_shared": C["fine_grained"].with_(T=700, d=256, E=4, k=2, f=384, seed=43),
    "one_expert": C["mixtral_prefill"].with_(T=50, d=256, f=256, E=1, k=1, seed=44),
    "k_equals_E": C["mixtral_prefill"].with_(T=40, d=256, f=256, E=4, k=4, seed=45),
    "T1": C["mixtral_prefill"].with_(T=1, d=256, f=256, seed=46),
    "d64_f64": C["mixtral_prefill"].with_(T=90, d=64, f=64, seed=47),
    "tight_capacity": C["mixtral_prefill"].with_(T=64, d=256, E=8, f=128, capacity_factor=0.5, seed=48),
    # one-step weight-gradient tiles (<= 64 rows per group) whose 256 x 256 tiles alternate between whole
    # and partial (f = 384: partial columns for dW_gate/dW_up, partial rows for dW_down), plus empty groups
    "wgrad_mixed_tiles": C["fine_grained"].with_(T=128, d=512, E=16, k=2, f=384, seed=49),
    # 65 one-step groups x 15 tiles per weight-gradient launch (~122 tiles per XCD): every persistent
    # work-group runs several one-step tiles in a row, whole tiles prefetching partial ones (f = 640)
    "wgrad_prefetch_partial": C["fine_grained"].with_(T=64, d=1280, E=64, k=2, f=640, seed=50),
    # fp8 e4m3 weights with per-output-channel scales (capacity drops, shared expert)
    "fp8_capacity_shared": C["fp8_capacity"].with_(T=160, d=256, E=16, k=4, f=256, shared=True, seed=57),
    "fp8_uncapped": C["fp8_capacity"].with_(T=96, d=512, E=8, k=2, f=192, capacity_factor=0.0, seed=58),
    # fp32 layers (the tiny configuration and a capped, shared-expert, renormalisation-off variant)
    "f32_tiny": C["tiny_f32"],
    "f32_shared_cap_renorm_off": C["tiny_f32"].with_(T=96, E=16, k=4, f=256, shared=True, renormalize=False,
                                                     capacity_factor=1.0, seed=60),
    # block-scaled weights (MXFP8 x and H, MXFP8 or MXFP4 weights), straight-through quantisation
    "mx8_finegrained_shared": C["fine_grained_mxfp8"].with_(T=96, d=512, E=32, f=256, seed=62),
    "mx4_prefill": C["mixtral_prefill_mxfp4"].with_(T=300, d=256, f=512, seed=63),
    "mx8_capacity_renorm_off": C["mixtral_prefill_mxfp8"].with_(T=120, d=256, E=8, f=256, capacity_factor=0.8,
                                                                renormalize=False, seed=64),
}

WG_TILE_COST = 96      # the weight-gradient kernel's per-tile cost term (rows + this)


def _wgrad_prefetch_pairs(counts, T, has_shared, M, N, n_cu):
    """Host replay of the persistent weight-gradient launch's tile split: the
    pairs (t, t + nslots) one work-group runs back to back where tile t is
    whole and the next tile has one K step (so its loads are issued before
    tile t's stores), returned as (next tile is partial) flags."""
    groups = [int(c) for c in counts] + ([T] if has_shared else [])
    padded = [(r + 63) // 64 * 64 for r in groups]
    poff = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    G = len(groups)
    tm_n, tn_n = (M + 255) // 256, (N + 255) // 256
    per_g = tm_n * tn_n
    total = G * per_g
    W = per_g * (int(poff[G]) + G * WG_TILE_COST)

    def gstart(g):
        return per_g * (int(poff[g]) + g * WG_TILE_COST)

    def first_tile(w):
        g = max(i for i in range(G + 1) if gstart(i) <= w)
        if g >= G:
            return G * per_g
        cost = int(poff[g + 1] - poff[g]) + WG_TILE_COST
        return g * per_g + min(per_g, -(-(w - gstart(g)) // cost))

    def tile_of(t):
        g, r = divmod(t, per_g)
        strip, rs = divmod(r, 4 * tn_n)
        gm = min(4, tm_n - strip * 4)
        return g, strip * 4 + rs % gm, rs // gm, int(poff[g + 1] - poff[g]) // 64

    grid = 8 * ((n_cu + 7) // 8)
    nslots = grid // 8
    flags = []
    for xcd in range(8):
        t0 = 0 if xcd == 0 else first_tile(W * xcd // 8)
        t1 = total if xcd == 7 else first_tile(W * (xcd + 1) // 8)
        for t in range(t0, t1):
            if t + nslots >= t1:
                continue
            _, tm, tn, _ = tile_of(t)
            if tm * 256 + 256 > M or tn * 256 + 256 > N:
                continue
            _, tm2, tn2, nk2 = tile_of(t + nslots)
            if nk2 == 1:
                flags.append(tm2 * 256 + 256 > M or tn2 * 256 + 256 > N)
    return flags


def _dout(cfg, seed=7):
    g = torch.Generator(device="cpu").manual_seed(seed)
    dt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    return torch.randn((cfg.T, cfg.d), generator=g).to(dt).cuda()


def _alloc_grads(cfg):
    z = lambda *s: torch.full(s, float("nan"), dtype=torch.float32, device="cuda")
    g = {"dx": z(cfg.T, cfg.d), "dW_g": z(cfg.d, cfg.E), "d_bias": z(cfg.E),
         "dW_gate": z(cfg.E, cfg.d, cfg.f), "dW_up": z(cfg.E, cfg.d, cfg.f), "dW_down": z(cfg.E, cfg.f, cfg.d)}
    if cfg.shared:
        g.update(dWs_gate=z(cfg.d, cfg.f), dWs_up=z(cfg.d, cfg.f), dWs_down=z(cfg.f, cfg.d))
    return g


def run_backward(inp, dout, routing=None):
    cfg = inp["cfg"]
    desc = ops.desc_from_cfg(cfg, routing=ops.ROUTING_TOKEN_CHOICE if routing is None else routing)
    ws = ops.alloc_backward_workspace(desc)
    g = _alloc_grads(cfg)
    ops.backward(desc, inp["x"], ops.weights_struct(inp), dout, ops.grads_struct(g), ws)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity_small(name):
    cfg = CASES[name]
    print(f"[backward] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    assert ov.certificate()["ok"].all()
    dout = _dout(cfg)
    g = run_backward(inp, dout)
    ref = oracle.backward(ov.x, ov.W_g, ov.bias, cfg.k, cfg.renormalize, np.float32(cfg.capacity_factor),
                          ov.expert, cfg.E, ov.shared(), to64(dout), **ov.quant_hooks())
    errs = {}
    tol = _tol(cfg)
    for key in ("dx", "dW_g", "dW_gate", "dW_up", "dW_down"):
        errs[key] = assert_close(to64(g[key]), ref[key], tol, f"{name} {key}")
    if inp["bias"] is not None:
        errs["d_bias"] = assert_close(to64(g["d_bias"]), ref["d_bias"], tol, f"{name} d_bias")
    if cfg.shared:
        for key in ("dWs_gate", "dWs_up", "dWs_down"):
            errs[key] = assert_close(to64(g[key]), ref[key], tol, f"{name} {key}")
    r = ov.forward(tokens=np.arange(min(cfg.T, 1)))
    if name == "wgrad_prefetch_partial":
        # the case exists to run the prefetch of a partial one-step tile: check on the host that the
        # launch's own tile split (dW_gate / dW_up: M = d, N = f; dW_down: M = f, N = d) contains it
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        flags = (_wgrad_prefetch_pairs(r["counts"], cfg.T, cfg.shared, cfg.d, cfg.f, n_cu) +
                 _wgrad_prefetch_pairs(r["counts"], cfg.T, cfg.shared, cfg.f, cfg.d, n_cu))
        assert any(flags) and not all(flags), f"prefetched tiles: {len(flags)}, partial: {sum(flags)}"
        print(f"[backward] {name}: {len(flags)} prefetched one-step tiles, {sum(flags)} of them partial",
              flush=True)
    empty = np.nonzero(r["counts"] == 0)[0]
    for e in empty:                                     # experts without tokens: exactly zero
        for key in ("dW_gate", "dW_up", "dW_down"):
            assert torch.count_nonzero(g[key][e]) == 0, (key, e)
    print(f"[backward] {name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()) +
          f" empty_experts={len(empty)}", flush=True)


@pytest.mark.parametrize("name", ["prefill", "renorm_off_shared_cap", "fp8_capacity_shared", "f32_tiny",
                                  "mx8_finegrained_shared", "mx4_prefill"])
def test_backward_bitwise_deterministic(name):
    inp = device_inputs(CASES[name])
    dout = _dout(CASES[name])
    a = run_backward(inp, dout)
    b = run_backward(inp, dout)
    for key in a:
        assert torch.equal(a[key], b[key]), key


def test_backward_empty_batch_writes_zero_weight_gradients():
    cfg = CASES["finegrained_shared"].with_(T=0)
    inp = device_inputs(CASES["finegrained_shared"])
    desc = ops.desc_from_cfg(cfg)
    g = _alloc_grads(cfg)
    x = torch.empty((0, cfg.d), dtype=torch.bfloat16, device="cuda")
    ops.backward(desc, x, ops.weights_struct(inp), x, ops.grads_struct(g), torch.empty(256, dtype=torch.uint8,
                                                                                        device="cuda"))
    torch.cuda.synchronize()
    for key, t in g.items():
        if key != "dx":
            assert torch.count_nonzero(t) == 0, key


# ---------------------------------------------------------------------------
# Full-size layers: dx on sampled tokens and weight-gradient columns of a few
# experts, each recomputed by the oracle's own functions on that slice (SwiGLU
# is separable by intermediate column, so a column's gradient only needs that
# column of W_gate / W_up and that row of W_down).
# ---------------------------------------------------------------------------
def _token_dx(ov, cfg, ref_fwd, dout64, t):
    k = cfg.k
    x_t = ov.x[t:t + 1]
    gj = np.zeros(k)
    dx = np.zeros(cfg.d)
    for j in range(k):
        a = t * k + j
        if ref_fwd["inv_perm"][a] < 0:
            continue
        e = int(ref_fwd["topk_idx"][t, j])
        W = ov.expert(e)
        y = oracle.expert_ffn(x_t, *W)[0]
        gj[j] = float(np.dot(dout64[t], y))
        dx += oracle.expert_ffn_backward(x_t, *W, ref_fwd["topk_w"][t, j] * dout64[t:t + 1])["dX"][0]
    dl = oracle.routing_weights_backward(ref_fwd["probs"][t:t + 1], ref_fwd["topk_idx"][t:t + 1], gj[None, :],
                                         cfg.renormalize)
    dx += (dl @ ov.W_g.T)[0]
    if cfg.shared:
        dx += oracle.expert_ffn_backward(x_t, *ov.shared(), dout64[t:t + 1])["dX"][0]
    return dx


@pytest.mark.parametrize("name,ntok,ncol", [("mixtral_prefill", 6, 4), ("fine_grained", 4, 3)])
def test_backward_parity_full_size(name, ntok, ncol):
    cfg = C[name]
    print(f"[backward-full] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    cache = {}
    expert = ov.expert
    ov.expert = lambda e: cache[e] if e in cache else cache.setdefault(e, expert(e))
    dout = _dout(cfg)
    dout64 = to64(dout)
    g = run_backward(inp, dout)
    ref_fwd = ov.forward(tokens=np.arange(1))
    rng = np.random.default_rng(3)
    toks = np.sort(rng.choice(cfg.T, size=ntok, replace=False))
    # also the token owning each expert's last row: its padded group's last
    # (light, possibly K-split) row tile; with many experts, those of the
    # heaviest, a median and the lightest non-empty expert
    offs, sa = ref_fwd["offsets"], ref_fwd["sorted_assign"]
    counts = ref_fwd["counts"]
    nonempty = [e for e in range(cfg.E) if counts[e] > 0]
    if cfg.E > 16:
        by_load = sorted(nonempty, key=lambda e: (counts[e], e))
        nonempty = sorted({by_load[-1], by_load[len(by_load) // 2], by_load[0]})
    tails = [int(sa[offs[e + 1] - 1]) // cfg.k for e in nonempty]
    toks = np.unique(np.concatenate([toks, np.array(tails, dtype=toks.dtype)]))
    got = to64(g["dx"][torch.from_numpy(toks).cuda()])
    want = np.stack([_token_dx(ov, cfg, ref_fwd, dout64, int(t)) for t in toks])
    e_dx = assert_close(got, want, TOL, f"{name} dx (sampled tokens)")
    # weight-gradient columns of the busiest expert, a middle one and (if any) an empty one
    counts = ref_fwd["counts"]
    experts = [int(np.argmax(counts)), int(np.argsort(counts)[len(counts) // 2])]
    empty = np.nonzero(counts == 0)[0]
    offs, sa = ref_fwd["offsets"], ref_fwd["sorted_assign"]
    cols = np.sort(rng.choice(cfg.f, size=ncol, replace=False))
    errs = []
    for e in experts:
        rows = sa[offs[e]:offs[e + 1]]
        toks_e = rows // cfg.k
        wt = np.array([ref_fwd["topk_w"][a // cfg.k, a % cfg.k] for a in rows])
        Wg, Wu, Wd = ov.expert(e)
        b = oracle.expert_ffn_backward(ov.x[toks_e], Wg[:, cols], Wu[:, cols], Wd[cols, :],
                                       wt[:, None] * dout64[toks_e])
        ci = torch.from_numpy(cols).cuda()
        errs.append(assert_close(to64(g["dW_gate"][e][:, ci]), b["dW_gate"], TOL, f"{name} dW_gate[{e}]"))
        errs.append(assert_close(to64(g["dW_up"][e][:, ci]), b["dW_up"], TOL, f"{name} dW_up[{e}]"))
        errs.append(assert_close(to64(g["dW_down"][e][ci, :]), b["dW_down"], TOL, f"{name} dW_down[{e}]"))
    for e in empty[:2]:
        for key in ("dW_gate", "dW_up", "dW_down"):
            assert torch.count_nonzero(g[key][int(e)]) == 0, (key, e)
    print(f"[backward-full] {name}: dx rel_err={e_dx:.3e} on {len(toks)} tokens (tails of experts {nonempty}) "
          f"dW rel_err max={max(errs):.3e} experts={experts} empty={len(empty)}", flush=True)


def test_backward_hip_graph_capture_replay():
    """moe_backward enqueues no host reads or memsets: captured once, replayed
    with unrelated eager work in between, every replay equals the eager call."""
    cfg = CASES["renorm_off_shared_cap"]
    inp = device_inputs(cfg)
    dout = _dout(cfg)
    eager = run_backward(inp, dout)
    desc = ops.desc_from_cfg(cfg)
    ws = ops.alloc_backward_workspace(desc)
    g = _alloc_grads(cfg)
    gs = ops.grads_struct(g)
    w = ops.weights_struct(inp)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        ops.backward(desc, inp["x"], w, dout, gs, ws)
    for rep in range(3):
        for t in g.values():
            t.fill_(float("nan"))
        junk = torch.randn(1000, device="cuda").sum()          # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for key in g:
            assert torch.equal(g[key], eager[key]), (rep, key)
        del junk


# ---------------------------------------------------------------------------
# Expert-choice layers (moe_desc.routing = expert choice): every expert takes
# its C best tokens, a token's slots are the 0..E experts that took it
# ---------------------------------------------------------------------------
EC_CASES = {
    "ec_prefill": C["mixtral_prefill"].with_(T=300, d=256, f=512, seed=51),
    "ec_renorm_off_shared": C["fine_grained"].with_(T=96, d=512, E=32, f=256, renormalize=False, seed=52),
    # C = ceil(0.5 T k / E): about half the tokens are taken by no expert
    "ec_low_capacity_shared": C["fine_grained"].with_(T=120, d=256, E=16, k=2, f=256, capacity_factor=0.5,
                                                      seed=53),
    "ec_every_token": C["mixtral_prefill"].with_(T=40, d=256, f=256, E=4, k=2, capacity_factor=2.0, seed=54),
    # C = T: every token is in all 96 experts' lists (longer than a wave)
    "ec_long_lists": C["fine_grained"].with_(T=40, d=256, E=96, k=8, f=128, capacity_factor=12.0, seed=55),
    "ec_small_batch": C["mixtral_prefill"].with_(T=5, d=256, f=256, E=8, k=2, seed=56),
    "ec_fp8_shared": C["fp8_capacity"].with_(T=128, d=256, E=16, k=4, f=256, shared=True, seed=59),
    "ec_f32_shared": C["tiny_f32"].with_(T=80, E=16, k=4, f=256, shared=True, seed=61),
    "ec_mx4_shared": C["fine_grained_mxfp4"].with_(T=96, d=512, E=32, f=256, seed=65),
}


def _ec_routing(ov, cfg):
    logits = oracle.router_logits(ov.x, ov.W_g, ov.bias)
    r = oracle.expert_choice_routing(logits, cfg.k, np.float32(cfg.capacity_factor), cfg.renormalize)
    r["logits"] = logits
    assert ec_boundary_is_clear(r)
    return r


@pytest.mark.parametrize("name", list(EC_CASES))
def test_backward_expert_choice_parity(name):
    cfg = EC_CASES[name]
    print(f"[backward-ec] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    r = _ec_routing(ov, cfg)
    dout = _dout(cfg)
    g = run_backward(inp, dout, ops.ROUTING_EXPERT_CHOICE)
    ref = oracle.expert_choice_backward(ov.x, ov.W_g, ov.bias, cfg.k, cfg.renormalize,
                                        np.float32(cfg.capacity_factor), ov.expert, cfg.E, ov.shared(), to64(dout),
                                        **ov.quant_hooks())
    assert np.array_equal(ref["pos"], r["pos"])
    errs = {}
    tol = _tol(cfg)
    for key in ("dx", "dW_g", "dW_gate", "dW_up", "dW_down"):
        errs[key] = assert_close(to64(g[key]), ref[key], tol, f"{name} {key}")
    if inp["bias"] is not None:
        errs["d_bias"] = assert_close(to64(g["d_bias"]), ref["d_bias"], tol, f"{name} d_bias")
    if cfg.shared:
        for key in ("dWs_gate", "dWs_up", "dWs_down"):
            errs[key] = assert_close(to64(g[key]), ref[key], tol, f"{name} {key}")
    taken = (r["pos"] >= 0).sum(axis=1)
    untaken = np.nonzero(taken == 0)[0]
    if len(untaken):                                    # tokens no expert took: only the shared expert's dx
        hk = ov.quant_hooks()
        xu = hk["quant_x"](ov.x[untaken]) if hk else ov.x[untaken]
        want = (oracle.expert_ffn_backward(xu, *ov.shared(), to64(dout)[untaken], quant_h=hk.get("quant_h"))["dX"]
                if cfg.shared else np.zeros((len(untaken), cfg.d)))
        assert_close(to64(g["dx"])[untaken], want, tol, f"{name} dx of untaken tokens")
    g2 = run_backward(inp, dout, ops.ROUTING_EXPERT_CHOICE)
    for key in g:
        assert torch.equal(g[key], g2[key]), key        # bitwise reproducible
    print(f"[backward-ec] {name}: C={r['capacity']} untaken_tokens={len(untaken)} max_list={taken.max()} " +
          " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)


def _token_dx_ec(ov, cfg, r, probs, dout64, t):
    x_t = ov.x[t:t + 1]
    gt = np.zeros((1, cfg.E))
    dx = np.zeros(cfg.d)
    for e in np.nonzero(r["pos"][t] >= 0)[0]:
        W = ov.expert(int(e))
        gt[0, e] = float(np.dot(dout64[t], oracle.expert_ffn(x_t, *W)[0]))
        dx += oracle.expert_ffn_backward(x_t, *W, r["weight"][t, e] * dout64[t:t + 1])["dX"][0]
    dl = oracle.expert_choice_weights_backward(probs[t:t + 1], r["pos"][t:t + 1], gt, cfg.renormalize)
    dx += (dl @ ov.W_g.T)[0]
    if cfg.shared:
        dx += oracle.expert_ffn_backward(x_t, *ov.shared(), dout64[t:t + 1])["dX"][0]
    return dx


@pytest.mark.parametrize("name,ntok,ncol", [("mixtral_prefill", 4, 4), ("fine_grained", 3, 3)])
def test_backward_expert_choice_full_size(name, ntok, ncol):
    """Full-size expert-choice layers: dx of sampled tokens (plus the tokens in
    the first and last rows of the first, a middle and the last expert) and
    weight-gradient columns of two experts, each from the oracle's functions."""
    cfg = C[name]
    print(f"[backward-ec-full] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    cache = {}
    expert = ov.expert
    ov.expert = lambda e: cache[e] if e in cache else cache.setdefault(e, expert(e))
    r = _ec_routing(ov, cfg)
    probs = oracle.softmax_rows(r["logits"])
    dout = _dout(cfg)
    dout64 = to64(dout)
    g = run_backward(inp, dout, ops.ROUTING_EXPERT_CHOICE)
    rng = np.random.default_rng(5)
    offs, st = r["offsets"], r["sorted_tokens"]
    edges = [int(st[i]) for e in (0, cfg.E // 2, cfg.E - 1) for i in (int(offs[e]), int(offs[e + 1]) - 1)]
    toks = np.unique(np.concatenate([rng.choice(cfg.T, size=ntok, replace=False), np.array(edges)]))
    got = to64(g["dx"][torch.from_numpy(toks).cuda()])
    want = np.stack([_token_dx_ec(ov, cfg, r, probs, dout64, int(t)) for t in toks])
    e_dx = assert_close(got, want, TOL, f"{name} expert-choice dx (sampled tokens)")
    cols = np.sort(rng.choice(cfg.f, size=ncol, replace=False))
    ci = torch.from_numpy(cols).cuda()
    errs = []
    for e in (0, cfg.E - 1):
        rows = st[offs[e]:offs[e + 1]]
        wt = np.array([r["weight"][t, e] for t in rows])
        Wg, Wu, Wd = ov.expert(e)
        b = oracle.expert_ffn_backward(ov.x[rows], Wg[:, cols], Wu[:, cols], Wd[cols, :], wt[:, None] * dout64[rows])
        errs.append(assert_close(to64(g["dW_gate"][e][:, ci]), b["dW_gate"], TOL, f"{name} dW_gate[{e}]"))
        errs.append(assert_close(to64(g["dW_up"][e][:, ci]), b["dW_up"], TOL, f"{name} dW_up[{e}]"))
        errs.append(assert_close(to64(g["dW_down"][e][ci, :]), b["dW_down"], TOL, f"{name} dW_down[{e}]"))
    print(f"[backward-ec-full] {name}: C={r['capacity']} dx rel_err={e_dx:.3e} on {len(toks)} tokens, "
          f"dW rel_err max={max(errs):.3e}", flush=True)


def test_backward_fp8_full_size_every_element():
    """The full fp8_capacity layer (T = 512, 128 experts of d = 2048, f = 768,
    capacity 1.25): every gradient element against the oracle's backward on the
    weights' values (code x channel scale)."""
    cfg = C["fp8_capacity"]
    print("[backward-full] fp8_capacity", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    assert ov.certificate()["ok"].all()
    dout = _dout(cfg)
    g = run_backward(inp, dout)
    ref = oracle.backward(ov.x, ov.W_g, ov.bias, cfg.k, cfg.renormalize, np.float32(cfg.capacity_factor),
                          ov.expert, cfg.E, ov.shared(), to64(dout))
    errs = {key: assert_close(to64(g[key]), ref[key], TOL, f"fp8_capacity {key}")
            for key in ("dx", "dW_g", "dW_gate", "dW_up", "dW_down")}
    if inp["bias"] is not None:
        errs["d_bias"] = assert_close(to64(g["d_bias"]), ref["d_bias"], TOL, "fp8_capacity d_bias")
    print("[backward-full] fp8_capacity: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
