"""GPU parity of the HIP library against the CPU oracle, through the C ABI.

Bars: top-k indices, expert counts/offsets, permutation, inverse permutation
and drop counts bit-exact; routing weights within 1e-6 relative; outputs within
max|gpu - oracle| / max|oracle| of 1e-5 (fp32), 2e-2 (bf16), 6e-2 (fp8).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import TOL, OracleInputs, assert_close, device_inputs, ec_boundary_is_clear, rel_err, to64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from sparse_mixture_experts_12_amd import _lib as ops
else:  # collected on CPU hosts but never run there (marker)
    ops = None

C = synth.CONFIGS

# Small layers the oracle finishes in seconds, spanning several tiles and a
# ragged last tile; each mirrors one workload's dtype/routing features.
SMALL = {
    "tiny_f32": C["tiny_f32"],
    "tiny_f32_ragged": C["tiny_f32"].with_(T=77, seed=3),
    # fp32: the shared expert's 64- and 32-row tiles with capacity drops (16-column
    # kernel), and a layer whose gate/up GEMM has enough 64 x 64 tiles for the
    # 64-column kernel while its down GEMM takes the 16-column one with K = 1024
    "f32_shared_cap": C["tiny_f32"].with_(T=96, E=16, k=4, f=256, shared=True, capacity_factor=1.25, seed=30),
    "f32_wide": C["tiny_f32"].with_(T=512, d=512, f=1024, seed=31),
    # fp32, K not a multiple of 128: a last K step of 64 in both GEMMs (gate/up K = 192, down K = 320)
    "f32_k192": C["tiny_f32"].with_(T=40, d=192, f=320, E=4, k=2, seed=32),
    "bf16_prefill": C["mixtral_prefill"].with_(T=300, d=512, f=1024),
    "bf16_prefill_ragged": C["mixtral_prefill"].with_(T=133, d=256, f=768, seed=5),
    "bf16_finegrained_shared": C["fine_grained"].with_(T=96, d=512, E=32, f=256),
    "fp8_capacity": C["fp8_capacity"].with_(T=200, d=256, E=16, f=128),
    "fp8_capacity_tight": C["fp8_capacity"].with_(T=64, d=256, E=8, f=128, capacity_factor=0.5, seed=2),
    "bf16_renorm_off": C["mixtral_prefill"].with_(T=70, d=256, f=256, renormalize=False, seed=4),
    "bf16_k_equals_E": C["mixtral_prefill"].with_(T=40, d=256, f=256, E=4, k=4, seed=6),
    "bf16_one_expert": C["mixtral_prefill"].with_(T=50, d=256, f=256, E=1, k=1, seed=7),
    "bf16_top1_switch": C["mixtral_prefill"].with_(T=90, d=256, f=256, E=16, k=1, capacity_factor=1.0),
    "bf16_big_tiles": C["mixtral_prefill"].with_(T=600, d=256, f=512, E=4, k=2, seed=8),
    # 256-row tiles whose last tiles hold 108..139 rows: the 128- and 256-row bodies
    "bf16_big_tiles_mid": C["mixtral_prefill"].with_(T=760, d=256, f=512, E=4, k=2, seed=3),
    "bf16_big_tiles_shared": C["fine_grained"].with_(T=700, d=256, E=4, k=2, f=256, seed=10),
    # last tiles at the bf16 light bound: 64 rows (light, full 64-row body), 65 rows (heavy launch,
    # 128-row body), 128 rows (128-row body full) and 129 rows (256-row body)
    "bf16_last_64": C["mixtral_prefill"].with_(T=311, d=128, f=256, seed=45),
    "bf16_last_65": C["mixtral_prefill"].with_(T=311, d=128, f=256, seed=42),
    "bf16_last_128": C["mixtral_prefill"].with_(T=476, d=128, f=256, seed=42),
    "bf16_last_129": C["mixtral_prefill"].with_(T=443, d=128, f=256, seed=40),
    "fp8_big_tiles_shared": C["fp8_capacity"].with_(T=700, d=256, E=4, k=2, f=256, capacity_factor=0.0,
                                                     shared=True, seed=9),
    # range edges: many experts and top-32, d = f = 64, E = 1023 (+ shared), one token on the grouped path
    "bf16_k32_E64": C["mixtral_prefill"].with_(T=50, d=128, f=128, E=64, k=32, seed=18),
    "bf16_d64_f64": C["mixtral_prefill"].with_(T=90, d=64, f=64, seed=19),
    "bf16_E1023_shared": C["fine_grained"].with_(T=40, d=64, f=64, E=1023, k=8, seed=20),
    "f32_T1": C["tiny_f32"].with_(T=1, seed=21),
    "decode_T2_E300_k16": C["mixtral_decode"].with_(T=2, d=128, f=128, E=300, k=16, seed=22),
    "decode_T1": C["mixtral_decode"].with_(d=512, f=1024),
    # enough work-groups (2 experts x 100 column slices) for the single fused
    # decode kernel; the other small decode cases take the row-split kernels
    "decode_T1_fused": C["mixtral_decode"].with_(d=256, f=6400, seed=26),
    "decode_T8": C["mixtral_decode_b8"].with_(d=512, f=1024),
    "decode_T5_shared_fp8": C["fp8_capacity_decode"].with_(T=5, d=256, E=16, f=256, shared=True),
    "decode_T3_fp8_cap": C["fp8_capacity_decode"].with_(T=3, d=256, E=8, f=128, k=4, capacity_factor=0.5),
    # block-scaled (MXFP8) layers: 64/128/256-row tile bodies, ragged tails, the
    # shared expert, capacity drops, a half-used last down-projection tile (d % 256 = 128)
    "mx_prefill": C["mixtral_prefill_mxfp8"].with_(T=300, d=512, f=1024),
    "mx_ragged": C["mixtral_prefill_mxfp8"].with_(T=133, d=256, f=768, seed=5),
    "mx_big_tiles": C["mixtral_prefill_mxfp8"].with_(T=760, d=384, f=512, E=4, k=2, seed=3),
    "mx_finegrained_shared": C["fine_grained_mxfp8"].with_(T=96, d=512, E=32, f=256),
    "mx_big_tiles_shared": C["fine_grained_mxfp8"].with_(T=700, d=256, E=4, k=2, f=384, seed=10),
    "mx_capacity": C["mixtral_prefill_mxfp8"].with_(T=200, d=256, E=16, k=8, f=128, capacity_factor=1.25,
                                                     seed=23),
    "mx_T1": C["mixtral_prefill_mxfp8"].with_(T=1, d=256, f=256, seed=24),
    "mx_long_k": C["mixtral_prefill_mxfp8"].with_(T=70, d=2048, f=1280, E=4, k=1, seed=25),
    # 97 expert groups: the light launches run on the library's second stream
    "mx_many_experts": C["fine_grained_mxfp8"].with_(T=64, d=256, E=96, k=4, f=256, seed=27),
    # MXFP4 weights (E2M1, two per byte) with MXFP8 activations: 64/128/256-row
    # bodies and ragged tails, the shared expert, capacity drops, a half-used
    # last down tile (d % 256 = 128), many groups on the second stream
    "mx4_prefill": C["mixtral_prefill_mxfp4"].with_(T=300, d=512, f=1024),
    "mx4_big_tiles": C["mixtral_prefill_mxfp4"].with_(T=760, d=384, f=512, E=4, k=2, seed=3),
    "mx4_finegrained_shared": C["fine_grained_mxfp4"].with_(T=96, d=512, E=32, f=256),
    "mx4_capacity": C["mixtral_prefill_mxfp4"].with_(T=200, d=256, E=16, k=8, f=128, capacity_factor=1.25,
                                                      seed=23),
    "mx4_many_experts": C["fine_grained_mxfp4"].with_(T=64, d=256, E=96, k=4, f=256, seed=28),
    "mx4_T1": C["mixtral_prefill_mxfp4"].with_(T=1, d=256, f=256, seed=29),
}


def run_forward(inp, path=ops.PATH_AUTO if ops else 0, stats=None):
    cfg = inp["cfg"]
    desc = ops.desc_from_cfg(cfg, path=path)
    ws = ops.alloc_workspace(desc)
    dt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    out = torch.empty((cfg.T, cfg.d), dtype=dt, device="cuda")
    taken = ops.forward(desc, inp["x"], ops.weights_struct(inp), out, ws, stats=stats)
    torch.cuda.synchronize()
    return out, taken


# ---------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------
ROUTE_CASES = {**{k: v for k, v in C.items()},
               "prefill_renorm_off": C["mixtral_prefill"].with_(renormalize=False),
               "fine_grained_T9": C["fine_grained"].with_(T=9),
               "fine_grained_T5": C["fine_grained"].with_(T=5),
               "k_equals_E": C["mixtral_prefill"].with_(T=33, E=4, k=4),
               "E_1": C["mixtral_prefill"].with_(T=17, E=1, k=1),
               # edges of the accepted ranges: E = 1023 with top-32, d = 64
               "E_1023_k32": C["fine_grained"].with_(T=70, d=128, E=1023, k=32),
               "d_64": C["mixtral_prefill"].with_(T=100, d=64, E=16, k=4, seed=3),
               # more than 256 tiles of 16 x 16 with E <= 16: the LDS-staged 256 x 16 partial tiles
               "lds_few_experts": C["mixtral_prefill"].with_(T=4200, d=512, E=16, k=4, seed=11),
               # 16 x 16 partial tiles with ragged token and expert tiles and a K slice of 320
               # (waves take 3, 3, 2 and 2 chunks of 32), in bf16 and fp32
               "tile_ragged": C["mixtral_prefill"].with_(T=50, d=320, E=100, k=6, seed=12),
               "tile_ragged_f32": C["tiny_f32"].with_(T=45, d=192, E=12, k=3, seed=13)}


@pytest.mark.parametrize("name", list(ROUTE_CASES))
def test_route_parity(name):
    cfg = ROUTE_CASES[name]
    print(f"[route] {name}", flush=True)
    inp = device_inputs(cfg, router_only=True)
    desc = ops.desc_from_cfg(cfg)
    T, k, E = cfg.T, cfg.k, cfg.E
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ws = ops.alloc_workspace(desc)
    ops.route(desc, inp["x"], ops.weights_struct(inp), idx, w, logits, ws)
    torch.cuda.synchronize()
    ov = OracleInputs(inp)
    ref_logits = oracle.router_logits(ov.x, ov.W_g, ov.bias)
    probs = oracle.softmax_rows(ref_logits)
    ref_idx = oracle.topk_select(ref_logits, k)
    ref_w = oracle.routing_weights(probs, ref_idx, cfg.renormalize)
    cert = ov.certificate()
    assert cert["ok"].all(), f"routing not certified for tokens {np.nonzero(~cert['ok'])[0][:10]}"
    g_logits = logits.cpu().numpy()
    # fp64 sums of different order round to the same fp32 value (1 ulp at most)
    ulps = np.abs(g_logits.view(np.int32).astype(np.int64) - ref_logits.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    assert (ulps == 0).mean() > 0.999
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=1e-6, atol=0)
    if cfg.renormalize:
        np.testing.assert_allclose(w.cpu().numpy().astype(np.float64).sum(1), 1.0, atol=1e-6)


# Exactly tied logits: odd expert columns of W_g copy the even ones, so every
# expert ties with its neighbour (identical fp64 sums in every path).  The
# selection must put the lower index first (the fixed tie rule), in each top-k
# path: the small-T block ranks (whole W_g or split into slices), the wave
# argmax rounds (E > 128, or 1024 tokens and more), and the wave ranks.
TIE_CASES = {
    "small_split_E128": C["fp8_capacity_decode"].with_(T=3),
    "small_whole_E64": C["mixtral_decode"].with_(T=2, d=256, E=64, k=6, seed=31),
    "small_split_E600": C["mixtral_decode"].with_(T=3, d=128, E=600, k=16, seed=32),
    "large_E128": C["mixtral_prefill"].with_(T=40, d=256, E=128, k=8, seed=33),
    "large_E600_renorm_off": C["mixtral_prefill"].with_(T=40, d=128, E=600, k=16, renormalize=False, seed=34),
    "large_T1100_E8": C["mixtral_prefill"].with_(T=1100, d=128, E=8, k=2, seed=35),
}


@pytest.mark.parametrize("name", list(TIE_CASES))
def test_route_exact_ties(name):
    cfg = TIE_CASES[name]
    print(f"[route-ties] {name}", flush=True)
    inp = device_inputs(cfg, router_only=True)
    inp["W_g"][:, 1::2] = inp["W_g"][:, 0::2]
    desc = ops.desc_from_cfg(cfg)
    T, k, E = cfg.T, cfg.k, cfg.E
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    ops.route(desc, inp["x"], ops.weights_struct(inp), idx, w, logits, ops.alloc_workspace(desc))
    torch.cuda.synchronize()
    g_logits = logits.cpu().numpy()
    assert np.array_equal(g_logits[:, 1::2], g_logits[:, 0::2]), "tied columns gave different logits"
    ov = OracleInputs(inp)
    ref_logits = oracle.router_logits(ov.x, ov.W_g, ov.bias)
    ulps = np.abs(g_logits.view(np.int32).astype(np.int64) - ref_logits.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    # the selection on the GPU's own logits: ties broken by the lower index
    gi = idx.cpu().numpy()
    np.testing.assert_array_equal(gi, oracle.topk_select(g_logits, k))
    assert (gi[:, 0] % 2 == 0).all()                     # the first of a tied pair is the even expert
    ref_w = oracle.routing_weights(oracle.softmax_rows(g_logits.astype(np.float64)), gi, cfg.renormalize)
    np.testing.assert_allclose(w.cpu().numpy(), ref_w, rtol=1e-6, atol=0)


def test_small_t_route_without_workspace():
    """A wide router (d * E > 65536) at T <= 8 splits its logits over d when
    given the workspace and runs one work-group without it: same results."""
    cfg = C["fine_grained"].with_(T=5)
    inp = device_inputs(cfg, router_only=True)
    desc = ops.desc_from_cfg(cfg)
    outs = []
    for ws in (ops.alloc_workspace(desc), None):
        idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
        w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
        logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
        ops.route(desc, inp["x"], ops.weights_struct(inp), idx, w, logits, ws)
        torch.cuda.synchronize()
        outs.append((idx.cpu(), w.cpu(), logits.cpu()))
    np.testing.assert_array_equal(outs[0][0].numpy(), outs[1][0].numpy())
    ulps = np.abs(outs[0][2].numpy().view(np.int32).astype(np.int64) - outs[1][2].numpy().view(np.int32).astype(np.int64))
    assert ulps.max() <= 1
    np.testing.assert_allclose(outs[0][1].numpy(), outs[1][1].numpy(), rtol=1e-6, atol=0)


def test_route_without_logits_output():
    cfg = C["mixtral_prefill"].with_(T=100)
    inp = device_inputs(cfg, router_only=True)
    desc = ops.desc_from_cfg(cfg)
    ws = ops.alloc_workspace(desc)
    idx = torch.empty((cfg.T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
    ops.route(desc, inp["x"], ops.weights_struct(inp), idx, w, None, ws)
    torch.cuda.synchronize()
    ov = OracleInputs(inp)
    logits = oracle.router_logits(ov.x, ov.W_g, ov.bias)
    np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk_select(logits, cfg.k))


# ---------------------------------------------------------------------------
# Permutation
# ---------------------------------------------------------------------------
def _perm_gpu(idx_np, E, cf):
    T, k = idx_np.shape
    desc = ops.make_desc(T, 64, E, k, 64, capacity_factor=cf)
    ws = ops.alloc_workspace(desc)
    dev = lambda n: torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    counts, offsets, sa, inv, nd = dev(E), dev(E + 1), dev(T * k), dev(T * k), dev(1)
    ops.permute(desc, torch.from_numpy(idx_np).cuda(), counts, offsets, sa, inv, nd, ws)
    torch.cuda.synchronize()
    return {"counts": counts.cpu().numpy()[:E], "offsets": offsets.cpu().numpy(),
            "sorted_assign": sa.cpu().numpy()[:T * k], "inv_perm": inv.cpu().numpy()[:T * k],
            "n_dropped": int(nd.cpu()[0]), "cap": ops.capacity(desc)}


def _check_perm(idx_np, E, cf):
    T, k = idx_np.shape
    g = _perm_gpu(idx_np, E, cf)
    cap = oracle.capacity(T, k, E, np.float32(cf))
    assert g["cap"] == (-1 if cap is None else cap)
    r = oracle.permute(idx_np, E, cap)
    np.testing.assert_array_equal(g["counts"], r["counts"])
    np.testing.assert_array_equal(g["offsets"], r["offsets"])
    kept = int(r["offsets"][-1])
    np.testing.assert_array_equal(g["sorted_assign"][:kept], r["sorted_assign"])
    assert (g["sorted_assign"][kept:] == -1).all()
    np.testing.assert_array_equal(g["inv_perm"], r["inv_perm"])
    assert g["n_dropped"] == r["n_dropped"]
    return r


def test_permute_worked_example():
    idx = np.array([[0, 1]] * 4, dtype=np.int32)
    r = _check_perm(idx, 3, 0.0)
    assert r["offsets"].tolist() == [0, 4, 8, 8]


# T*k up to 4096 runs the single-work-group permutation, beyond it the
# multi-block one (4097, 16385: a one-assignment last block), which sums the
# block counts inside its scatter launch up to 64 blocks (65536 assignments)
# and in a launch of its own beyond; 2^21 x 8 = 2^24 is the largest T*k the
# library accepts.
@pytest.mark.parametrize("T,k,E,cf,skew", [
    (1, 2, 8, 0.0, 0), (64, 2, 8, 0.0, 0), (4096, 2, 8, 0.0, 0), (2048, 8, 256, 0.0, 1),
    (512, 8, 128, 1.25, 1), (1, 8, 128, 1.25, 0), (333, 3, 7, 1.0, 1), (1000, 1, 1, 0.0, 0),
    (700, 4, 1023, 0.0, 0), (129, 2, 64, 0.3, 1), (2049, 8, 256, 1.0, 2),
    (4096, 1, 4, 0.0, 0), (4097, 1, 5, 0.0, 0), (16385, 1, 5, 0.0, 0), (5000, 4, 1023, 0.7, 1),
    (32768, 2, 3, 0.8, 1), (32769, 2, 3, 0.8, 1),
    (2 ** 21, 8, 256, 1.25, 1)])
def test_permute_parity(T, k, E, cf, skew):
    print(f"[permute] T={T} k={k} E={E} cf={cf} skew={skew}", flush=True)
    rng = np.random.default_rng(T * 7 + E)
    if skew == 0:
        p = None
    else:
        p = 1.0 / np.arange(1, E + 1) ** (1.1 * skew)
        p /= p.sum()
    if T * k <= 100000:
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    else:       # large: experts drawn independently per slot (repeats inside a token are fine here)
        idx = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    _check_perm(idx, E, cf)


def test_permute_all_to_one_expert_with_capacity():
    T, k, E = 300, 1, 4
    idx = np.zeros((T, k), dtype=np.int32)
    r = _check_perm(idx, E, 1.0)
    assert r["n_dropped"] == T - 75


# ---------------------------------------------------------------------------
# Grouped FFN, given the oracle's permutation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny_f32", "tiny_f32_ragged", "f32_shared_cap", "f32_wide", "f32_k192",
                                  "bf16_prefill", "bf16_prefill_ragged",
                                  "bf16_finegrained_shared", "fp8_capacity", "fp8_capacity_tight",
                                  "bf16_one_expert", "bf16_big_tiles", "bf16_big_tiles_mid",
                                  "bf16_big_tiles_shared", "bf16_last_64", "bf16_last_65", "bf16_last_128",
                                  "bf16_last_129", "fp8_big_tiles_shared", "mx_prefill", "mx_big_tiles",
                                  "mx_big_tiles_shared", "mx_capacity", "mx4_prefill", "mx4_big_tiles",
                                  "mx4_finegrained_shared", "mx4_capacity"])
def test_grouped_ffn_parity(name):
    cfg = SMALL[name]
    print(f"[grouped_ffn] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    ref = ov.forward()
    T, k, d = cfg.T, cfg.k, cfg.d
    rows = T * k + (T if cfg.shared else 0)
    y = torch.full((rows, d), float("nan"), dtype=torch.float32, device="cuda")
    desc = ops.desc_from_cfg(cfg)
    ws = ops.alloc_workspace(desc)
    sa = np.full(T * k, -1, dtype=np.int32)
    sa[:len(ref["sorted_assign"])] = ref["sorted_assign"]
    ops.grouped_ffn(desc, inp["x"], ops.weights_struct(inp), torch.from_numpy(sa).cuda(),
                    torch.from_numpy(ref["offsets"]).cuda(), y, ws)
    torch.cuda.synchronize()
    yg = to64(y)
    kept = int(ref["offsets"][-1])
    # oracle rows in permuted order
    yref = np.zeros((kept, d))
    for e in range(cfg.E):
        lo, hi = ref["offsets"][e], ref["offsets"][e + 1]
        if hi > lo:
            toks = ref["sorted_assign"][lo:hi] // k
            yref[lo:hi] = ov.ffn(ov.x[toks], e)
    assert_close(yg[:kept], yref, TOL[cfg.wdt], f"{name} routed rows")
    assert np.isnan(yg[kept:T * k]).all(), "rows past the kept ones must stay untouched"
    if cfg.shared:
        assert_close(yg[T * k:], ov.ffn(ov.x), TOL[cfg.wdt], f"{name} shared rows")


# ---------------------------------------------------------------------------
# Combine, given the oracle's expert outputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("act,shared,cf", [("bf16", False, 0.0), ("f32", False, 0.0), ("bf16", True, 0.0),
                                            ("bf16", False, 0.5)])
def test_combine_parity(act, shared, cf):
    rng = np.random.default_rng(11)
    T, k, E, d = 57, 3, 9, 320
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    cap = oracle.capacity(T, k, E, np.float32(cf))
    perm = oracle.permute(idx, E, cap)
    w = rng.random((T, k)).astype(np.float32)
    rows = T * k + (T if shared else 0)
    y = rng.normal(size=(rows, d)).astype(np.float32)
    ref = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            p = perm["inv_perm"][t * k + j]
            if p >= 0:
                ref[t] += float(w[t, j]) * y[p].astype(np.float64)
        if shared:
            ref[t] += y[T * k + t]
    desc = ops.make_desc(T, d, E, k, 64, act=act, wdt=act, has_shared=shared, capacity_factor=cf)
    out = torch.empty((T, d), dtype=torch.float32 if act == "f32" else torch.bfloat16, device="cuda")
    ops.combine(desc, torch.from_numpy(y).cuda(), torch.from_numpy(perm["inv_perm"]).cuda(),
                torch.from_numpy(w).cuda(), out)
    torch.cuda.synchronize()
    assert_close(to64(out), ref, 1e-6 if act == "f32" else 2 ** -8, "combine")


# ---------------------------------------------------------------------------
# Whole layer, small sizes, every element
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(SMALL))
def test_forward_parity_small(name):
    cfg = SMALL[name]
    print(f"[forward] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    assert ov.certificate()["ok"].all()
    dev_nd = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev_counts = torch.zeros(cfg.E, dtype=torch.int32, device="cuda")
    st = ops.Stats(d_n_dropped=dev_nd.data_ptr(), d_counts=dev_counts.data_ptr())
    out, taken = run_forward(inp, stats=st)
    ref = ov.forward()
    decode = cfg.T <= 8 and cfg.act == "bf16" and cfg.wdt not in ("mxfp8", "mxfp4")
    want_path = ops.PATH_FUSED_DECODE if decode else ops.PATH_GROUPED
    assert taken == want_path
    e = assert_close(to64(out), ref["out"], TOL[cfg.wdt], name)
    print(f"[forward] {name}: rel_err={e:.3e}", flush=True)
    assert int(dev_nd.cpu()[0]) == ref["n_dropped"]
    np.testing.assert_array_equal(dev_counts.cpu().numpy(), ref["counts"])


@pytest.mark.parametrize("name", ["decode_T1", "decode_T1_fused", "decode_T8", "decode_T5_shared_fp8",
                                  "decode_T3_fp8_cap"])
def test_fused_decode_matches_grouped(name):
    cfg = SMALL[name]
    inp = device_inputs(cfg)
    a, pa = run_forward(inp, path=ops.PATH_FUSED_DECODE)
    b, pb = run_forward(inp, path=ops.PATH_GROUPED)
    assert pa == ops.PATH_FUSED_DECODE and pb == ops.PATH_GROUPED
    assert_close(to64(a), to64(b), TOL[cfg.wdt], f"{name} fused vs grouped")


@pytest.mark.parametrize("name", ["bf16_prefill", "decode_T8", "fp8_capacity", "tiny_f32", "bf16_E1023_shared"])
def test_bitwise_deterministic(name):
    inp = device_inputs(SMALL[name])
    a, _ = run_forward(inp)
    b, _ = run_forward(inp)
    assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


# bf16_E1023_shared, mx_many_experts: 64 or more expert groups, so the grouped
# GEMMs' light launches run on the library's second stream (fork / join
# captured into the graph)
@pytest.mark.parametrize("name", ["bf16_prefill_ragged", "decode_T1", "mx_ragged", "bf16_E1023_shared",
                                  "mx_many_experts"])
def test_hip_graph_capture_replay(name):
    cfg = SMALL[name]
    inp = device_inputs(cfg)
    eager, _ = run_forward(inp)
    desc = ops.desc_from_cfg(cfg)
    ws = ops.alloc_workspace(desc)
    out = torch.zeros_like(eager)
    w = ops.weights_struct(inp)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ops.forward(desc, inp["x"], w, out, ws)
    for rep in range(3):
        out.zero_()
        junk = torch.randn(1000, device="cuda").sum()       # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        del junk


def test_graph_capture_first_call_of_a_thread():
    """A many-group layer whose first call in a host thread is made under graph
    capture: the library creates no stream or event during the capture (it
    keeps that call on the capturing stream) and the replays match eager."""
    import threading
    cfg = SMALL["bf16_E1023_shared"]
    inp = device_inputs(cfg)
    eager, _ = run_forward(inp)
    desc = ops.desc_from_cfg(cfg)
    ws = ops.alloc_workspace(desc)
    out = torch.zeros_like(eager)
    w = ops.weights_struct(inp)
    box = {}

    def capture():
        try:
            s = torch.cuda.Stream()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                ops.forward(desc, inp["x"], w, out, ws)
            box["g"] = g
        except Exception as e:                              # reported in the main thread
            box["err"] = e

    th = threading.Thread(target=capture)
    th.start()
    th.join()
    assert "err" not in box, box.get("err")
    for rep in range(3):
        out.zero_()
        box["g"].replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"


# ---------------------------------------------------------------------------
# Whole layer at the workloads' full sizes: routing and permutation on every
# token; outputs on sampled tokens plus, for every non-empty expert, the tokens
# owning its first and last permuted rows, and tokens on the shared expert's
# row-tile boundaries, all recomputed by the oracle.
# ---------------------------------------------------------------------------
FULL = ["tiny_f32", "mixtral_decode", "mixtral_decode_b8", "mixtral_prefill", "fine_grained",
        "fp8_capacity", "fp8_capacity_decode", "mixtral_prefill_mxfp8", "fine_grained_mxfp8",
        "mixtral_prefill_mxfp4", "fine_grained_mxfp4"]
SAMPLE = {"mixtral_prefill": 12, "fine_grained": 3, "fp8_capacity": 24, "mixtral_prefill_mxfp8": 12,
          "fine_grained_mxfp8": 3, "mixtral_prefill_mxfp4": 12, "fine_grained_mxfp4": 3}
TILE = 32          # the smallest row-tile height any grouped GEMM body uses


def _edge_tokens(offsets, sorted_assign, k, E):
    """Tokens owning each non-empty expert's first and last permuted rows."""
    out = []
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            out += [int(sorted_assign[lo]) // k, int(sorted_assign[hi - 1]) // k]
    return out


def _tile_edge_rows(lo, hi, tile=TILE):
    """First and last row of every `tile`-row block of rows [lo, hi)."""
    rows = set()
    for r in range(lo, hi, tile):
        rows.update((r, min(r + tile, hi) - 1))
    return sorted(rows)


@pytest.mark.parametrize("name", FULL)
def test_forward_parity_full_size(name):
    cfg = C[name]
    print(f"[forward-full] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    assert ov.certificate()["ok"].all()
    dev_nd = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev_counts = torch.zeros(cfg.E, dtype=torch.int32, device="cuda")
    st = ops.Stats(d_n_dropped=dev_nd.data_ptr(), d_counts=dev_counts.data_ptr())
    out, taken = run_forward(inp, stats=st)
    n = SAMPLE.get(name)
    toks = None
    if n is not None:
        routing = ov.forward(tokens=np.arange(0))
        picks = [np.random.default_rng(0).choice(cfg.T, size=n, replace=False),
                 _edge_tokens(routing["offsets"], routing["sorted_assign"], cfg.k, cfg.E)]
        if cfg.shared:
            picks.append(_tile_edge_rows(0, cfg.T))
        toks = np.unique(np.concatenate([np.asarray(p, dtype=np.int64) for p in picks]))
    ref = ov.forward(tokens=toks)
    got = to64(out) if toks is None else to64(out)[toks]
    e = assert_close(got, ref["out"], TOL[cfg.wdt], name)
    covered = sum(1 for i in range(cfg.E) if ref["counts"][i] > 0)
    print(f"[forward-full] {name}: path={taken} rel_err={e:.3e} tokens_checked={len(ref['out'])}/{cfg.T} "
          f"experts_covered={covered}/{covered} dropped={ref['n_dropped']} "
          f"empty_experts={(ref['counts'] == 0).sum()}", flush=True)
    np.testing.assert_array_equal(dev_counts.cpu().numpy(), ref["counts"])
    assert int(dev_nd.cpu()[0]) == ref["n_dropped"]
    if name == "fine_grained":
        assert (ref["counts"] == 0).sum() >= 1, "the Zipf bias should leave some expert without tokens"


# Grouped FFN at full size, expert by expert: the rows on every 64-row tile
# boundary of every non-empty expert (so every row tile of every expert, heavy,
# light or split over K, is compared on every output column) and of the shared
# expert, against the oracle's FFN of that expert alone.  Expert-choice layers
# feed the same kernels the oracle's expert-choice selection (E*C rows, token t
# given as assignment t*k).
GROUPED_FULL = ["mixtral_prefill", "fine_grained", "fp8_capacity", "mixtral_prefill_mxfp8",
                "fine_grained_mxfp8", "mixtral_prefill_mxfp4", "fine_grained_mxfp4", "fine_grained_expert_choice"]


@pytest.mark.parametrize("name", GROUPED_FULL)
def test_grouped_ffn_every_expert_full_size(name):
    ec = name.endswith("_expert_choice")
    cfg = C[name[:-len("_expert_choice")] if ec else name]
    print(f"[grouped-full] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    T, k, d, E = cfg.T, cfg.k, cfg.d, cfg.E
    if ec:
        r = oracle.expert_choice_routing(oracle.router_logits(ov.x, ov.W_g, ov.bias), k,
                                         np.float32(cfg.capacity_factor), cfg.renormalize)
        offsets = r["offsets"].astype(np.int32)
        assert offsets[-1] == T * k, "the expert-choice rows must fill the T*k routed rows"
        sa = (r["sorted_tokens"] * k).astype(np.int32)
    else:
        r = ov.forward(tokens=np.arange(0))
        offsets = r["offsets"]
        sa = np.full(T * k, -1, dtype=np.int32)
        sa[:len(r["sorted_assign"])] = r["sorted_assign"]
    rows = T * k + (T if cfg.shared else 0)
    y = torch.full((rows, d), float("nan"), dtype=torch.float32, device="cuda")
    desc = ops.desc_from_cfg(cfg)
    ws = ops.alloc_workspace(desc)
    ops.grouped_ffn(desc, inp["x"], ops.weights_struct(inp), torch.from_numpy(sa).cuda(),
                    torch.from_numpy(offsets).cuda(), y, ws)
    torch.cuda.synchronize()
    kept = int(offsets[-1])
    assert bool(torch.isnan(y[kept:T * k]).all()), "rows past the kept ones must stay untouched"
    worst, n_rows, covered = 0.0, 0, 0
    nonempty = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    for e in nonempty:
        rr = _tile_edge_rows(int(offsets[e]), int(offsets[e + 1]))
        toks = sa[rr] // k
        got = to64(y[torch.tensor(rr, device="cuda")])
        worst = max(worst, assert_close(got, ov.ffn(ov.x[toks], e), TOL[cfg.wdt], f"{name} expert {e} rows {rr[:4]}"))
        n_rows += len(rr)
        covered += 1
    if cfg.shared:
        tt = _tile_edge_rows(0, T)
        got = to64(y[torch.tensor([T * k + t for t in tt], device="cuda")])
        worst = max(worst, assert_close(got, ov.ffn(ov.x[tt]), TOL[cfg.wdt], f"{name} shared rows"))
        n_rows += len(tt)
    print(f"[grouped-full] {name}: experts covered {covered}/{len(nonempty)} (+shared={cfg.shared}), "
          f"rows checked {n_rows}/{kept + (T if cfg.shared else 0)}, worst rel_err={worst:.3e}", flush=True)


# ---------------------------------------------------------------------------
# Router telemetry side outputs of moe_forward, against the oracle
# ---------------------------------------------------------------------------
TEL_CASES = ["tiny_f32_ragged", "bf16_prefill_ragged", "bf16_finegrained_shared", "fp8_capacity_tight",
             "bf16_top1_switch", "decode_T1", "decode_T8", "decode_T3_fp8_cap", "fine_grained", "mixtral_prefill"]


@pytest.mark.parametrize("name", TEL_CASES)
def test_router_telemetry_parity(name):
    cfg = SMALL[name] if name in SMALL else C[name]
    print(f"[telemetry] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    plain, _ = run_forward(inp)

    def run():
        routed = torch.full((cfg.E,), -7, dtype=torch.int32, device="cuda")
        pm = torch.full((cfg.E,), float("nan"), dtype=torch.float32, device="cuda")
        loss = torch.full((4,), float("nan"), dtype=torch.float32, device="cuda")
        st = ops.Stats(d_routed=routed.data_ptr(), d_prob_mean=pm.data_ptr(), d_lb_loss=loss.data_ptr())
        out, _ = run_forward(inp, stats=st)
        return out, routed.cpu().numpy(), pm.cpu().numpy(), loss.cpu().numpy()

    out, routed, pm, loss = run()
    ref = ov.forward(tokens=np.arange(min(cfg.T, 2)))     # routing of every token; FFN of two
    tel = oracle.router_telemetry(ref["logits"], ref["topk_idx"], cfg.E)
    np.testing.assert_array_equal(routed, tel["routed"])
    np.testing.assert_allclose(pm.astype(np.float64), tel["prob_mean"], rtol=1e-6, atol=1e-12)
    assert loss[0] == pytest.approx(tel["lb_loss"], rel=1e-6)
    assert np.isnan(loss[1:]).all()                       # nothing written past the loss
    # the side outputs change nothing else and are bitwise reproducible
    assert torch.equal(out, plain)
    out2, routed2, pm2, loss2 = run()
    assert torch.equal(out2, out)
    np.testing.assert_array_equal(routed2, routed)
    np.testing.assert_array_equal(pm2.view(np.int32), pm.view(np.int32))
    np.testing.assert_array_equal(loss2[:1].view(np.int32), loss[:1].view(np.int32))
    print(f"[telemetry] {name}: loss={loss[0]:.6f} oracle={tel['lb_loss']:.6f} "
          f"max_load={routed.max()} idle_experts={(routed == 0).sum()}", flush=True)


# ---------------------------------------------------------------------------
# Expert-choice routing (moe_desc.routing = expert choice), against the oracle
# ---------------------------------------------------------------------------
EC_CASES = {
    "ec_bf16": C["mixtral_prefill"].with_(T=300, d=256, f=512, seed=12),
    "ec_bf16_renorm_off_shared": C["fine_grained"].with_(T=96, d=512, E=32, f=256, renormalize=False, seed=13),
    "ec_fp8_cf": C["fp8_capacity"].with_(T=200, d=256, E=16, f=128, seed=14),
    "ec_f32": C["tiny_f32"].with_(T=77, seed=15),
    "ec_all_tokens": C["mixtral_prefill"].with_(T=40, d=256, f=256, E=4, k=2, capacity_factor=2.0, seed=16),
    "ec_small_batch": C["mixtral_prefill"].with_(T=5, d=256, f=256, E=8, k=2, seed=17),
    "ec_mx_shared": C["fine_grained_mxfp8"].with_(T=96, d=512, E=32, f=256, seed=26),
    "ec_mx4_shared": C["fine_grained_mxfp4"].with_(T=96, d=512, E=32, f=256, seed=30),
    "mixtral_prefill": C["mixtral_prefill"],
    "fine_grained": C["fine_grained"],
}
EC_SAMPLE = {"mixtral_prefill": 8, "fine_grained": 3}


@pytest.mark.parametrize("name", list(EC_CASES))
def test_expert_choice_parity(name):
    cfg = EC_CASES[name]
    print(f"[expert-choice] {name}", flush=True)
    inp = device_inputs(cfg)
    ov = OracleInputs(inp)
    desc = ops.desc_from_cfg(cfg, routing=ops.ROUTING_EXPERT_CHOICE)
    ws = ops.alloc_workspace(desc)
    dt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    counts = torch.full((cfg.E,), -1, dtype=torch.int32, device="cuda")
    nd = torch.full((1,), -1, dtype=torch.int32, device="cuda")

    def run():
        out = torch.empty((cfg.T, cfg.d), dtype=dt, device="cuda")
        st = ops.Stats(d_n_dropped=nd.data_ptr(), d_counts=counts.data_ptr())
        taken = ops.forward(desc, inp["x"], ops.weights_struct(inp), out, ws, stats=st)
        torch.cuda.synchronize()
        return out, taken

    out, taken = run()
    assert taken == ops.PATH_GROUPED
    n = EC_SAMPLE.get(name)
    toks = None
    if n is not None:
        r = oracle.expert_choice_routing(oracle.router_logits(ov.x, ov.W_g, ov.bias), cfg.k,
                                         np.float32(cfg.capacity_factor), cfg.renormalize)
        edges = [int(r["sorted_tokens"][i]) for e in range(cfg.E)
                 for i in (int(r["offsets"][e]), int(r["offsets"][e + 1]) - 1)]
        toks = np.unique(np.concatenate([np.random.default_rng(1).choice(cfg.T, size=n, replace=False),
                                         np.array(edges, dtype=np.int64)]))
    ref = oracle.expert_choice_forward(ov.x, ov.W_g, ov.bias, cfg.k, cfg.renormalize,
                                       np.float32(cfg.capacity_factor), ov.expert, cfg.E, shared=ov.shared(),
                                       tokens=toks, **ov.quant_hooks())
    assert ec_boundary_is_clear(ref)
    Cap = ref["capacity"]
    assert ops.capacity(desc) == Cap
    assert counts.cpu().numpy().tolist() == [Cap] * cfg.E
    unchosen = int(((ref["pos"] >= 0).sum(axis=1) == 0).sum())
    assert int(nd.cpu()[0]) == unchosen
    got = to64(out) if toks is None else to64(out)[toks]
    e = assert_close(got, ref["out"], TOL[cfg.wdt], name)
    out2, _ = run()
    assert torch.equal(out2, out)                       # bitwise reproducible
    print(f"[expert-choice] {name}: C={Cap} unchosen_tokens={unchosen} rel_err={e:.3e} "
          f"tokens_checked={len(got)}/{cfg.T}", flush=True)


# ---------------------------------------------------------------------------
# MXFP8 quantiser (moe_quantize_mxfp8): codes and scales bit-exact
# ---------------------------------------------------------------------------
def _mx_rows(rng, rows, cols):
    v = rng.normal(0, 1, (rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, 1)))
    special = [np.zeros(32),                                         # all-zero block
               -np.zeros(32),
               rng.normal(0, 1, 32) * 1e-37,                         # scale exponent clamped at -127
               np.array([448.0, 464.0, 480.0, 500.0, -511.0] + [1.0] * 27),   # saturation (block max 511)
               2.0 ** np.arange(-10, 22),                            # powers of two across the E4M3 range
               -(2.0 ** -20) * np.arange(32),                        # negatives that round to -0
               (np.arange(32) + 0.5) * 2.0 ** -4]                    # ties
    nb = cols // 32
    for i, blk in enumerate(special):
        r, b = divmod(i, nb)
        if r < rows:
            v[r, 32 * b:32 * b + 32] = blk
    return v


@pytest.mark.parametrize("dtype,rows,cols", [("bf16", 37, 256), ("f32", 37, 256), ("bf16", 4096, 4096),
                                              ("f32", 5, 32), ("bf16", 300, 2048 + 96)])
def test_mx_quantize_parity(dtype, rows, cols):
    print(f"[mx_quantize] {dtype} {rows}x{cols}", flush=True)
    rng = np.random.default_rng(rows * 31 + cols)
    v = _mx_rows(rng, rows, cols)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    xt = torch.from_numpy(v.astype(np.float32)).to(tdt).cuda()
    q = torch.full((rows, cols), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, cols // 32), 0x5A, dtype=torch.uint8, device="cuda")
    ops.quantize_mxfp8(xt, q, s)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quantize(to64(xt))
    np.testing.assert_array_equal(s.cpu().numpy(), rs)
    np.testing.assert_array_equal(q.cpu().numpy(), rq)


def test_mx_quantize_empty_and_errors():
    q = torch.zeros(64, dtype=torch.uint8, device="cuda")
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    ops.quantize_mxfp8(x, q, q)                           # rows == 0 enqueues nothing
    bad = torch.zeros((2, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ops.MoEError):
        ops.quantize_mxfp8(bad, q, q)
