"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test checks the oracle against something the oracle does not compute the
same way: a value printed on the pages (tests/golden), a library routine
(torch / scipy), a closed form, an invariant of the method, or brute force on
tiny inputs.  A plausible slip in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a wrong tie rule) fails at least one of them.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

RNG = np.random.default_rng(1234)


def bf16_values(shape, std, rng=RNG):
    """Random values exactly representable in bf16 (as float64)."""
    t = torch.from_numpy(rng.normal(0.0, std, size=shape).astype(np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def read_golden(golden_dir, name):
    rows = {}
    with open(os.path.join(golden_dir, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows[key] = [int(v) for v in vals]
    return rows


# --------------------------------------------------------------------------
# Permutation / expert_offsets
# --------------------------------------------------------------------------
def test_offsets_worked_example_from_pages(golden_dir):
    g = read_golden(golden_dir, "expert_offsets_worked_example.txt")
    E = g["E"][0]
    # four tokens, each choosing experts 0 and 1 -> counts [4, 4, 0]
    idx = np.array([[0, 1]] * 4, dtype=np.int32)
    p = oracle.permute(idx, E, None)
    assert p["counts"].tolist() == g["counts"]
    assert p["offsets"].tolist() == g["offsets_leading_zero"]
    assert p["offsets"][1:].tolist() == g["offsets_inclusive"]
    rows0 = list(range(p["offsets"][0], p["offsets"][1]))
    rows1 = list(range(p["offsets"][1], p["offsets"][2]))
    assert rows0 == g["rows_expert0"] and rows1 == g["rows_expert1"]
    assert p["offsets"][2] == p["offsets"][3]          # empty expert 2
    # expert 0's rows hold the slot-0 assignments in token order
    assert [int(a) for a in p["sorted_assign"][:4]] == [0, 2, 4, 6]
    assert p["n_dropped"] == 0


def _brute_permute(flat, E, cap):
    n = len(flat)
    rank = [sum(1 for b in range(a) if flat[b] == flat[a]) for a in range(n)]
    kept = [cap is None or rank[a] < cap for a in range(n)]
    order = sorted((a for a in range(n) if kept[a]), key=lambda a: (flat[a], a))
    counts = [sum(1 for a in range(n) if kept[a] and flat[a] == e) for e in range(E)]
    return order, counts, n - sum(kept)


@pytest.mark.parametrize("T,k,E,cap", [(7, 2, 5, None), (13, 3, 4, 4), (1, 4, 8, 1),
                                        (20, 1, 3, 2), (0, 2, 4, None), (9, 4, 4, None)])
def test_permute_brute_force(T, k, E, cap):
    rng = np.random.default_rng(T * 100 + k)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    p = oracle.permute(idx, E, cap)
    order, counts, nd = _brute_permute(idx.reshape(-1).tolist(), E, cap)
    assert p["sorted_assign"].tolist() == order
    assert p["counts"].tolist() == counts
    assert p["n_dropped"] == nd
    assert p["offsets"].tolist() == [0] + list(np.cumsum(counts))
    # inverse permutation
    for pos, a in enumerate(order):
        assert p["inv_perm"][a] == pos
    assert int((p["inv_perm"] < 0).sum()) == nd
    assert p["offsets"][-1] == T * k - nd


def test_capacity_special_cases():
    assert oracle.capacity(512, 8, 128, 1.25) == 40
    assert oracle.capacity(1, 8, 128, 1.25) == 1
    assert oracle.capacity(100, 2, 8, 0.0) is None
    # every token on expert 0: the first C assignments in token order are kept
    T, k, E = 10, 1, 4
    idx = np.zeros((T, k), dtype=np.int32)
    C = oracle.capacity(T, k, E, 1.0)           # ceil(10/4) = 3
    assert C == 3
    p = oracle.permute(idx, E, C)
    assert p["sorted_assign"].tolist() == [0, 1, 2]
    assert p["n_dropped"] == 7
    assert p["inv_perm"].tolist() == [0, 1, 2] + [-1] * 7
    # one token: its k experts are distinct, nothing can be dropped
    idx1 = np.array([[3, 1, 2, 0]], dtype=np.int32)
    p1 = oracle.permute(idx1, 4, oracle.capacity(1, 4, 4, 1.25))
    assert p1["n_dropped"] == 0 and p1["sorted_assign"].tolist() == [3, 1, 2, 0]


# --------------------------------------------------------------------------
# Router logits, softmax, top-k, weights
# --------------------------------------------------------------------------
def test_router_logits_exact_rounding():
    T, d, E = 5, 24, 7
    x = bf16_values((T, d), 1.0)
    W = bf16_values((d, E), 0.02)
    b = np.float32(RNG.normal(size=E)).astype(np.float64)
    got = oracle.router_logits(x, W, b)
    assert got.dtype == np.float32 and got.shape == (T, E)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(x[t, i]) * Fraction(W[i, e]) for i in range(d)) + Fraction(b[e])
            # bf16 products of this spread sum exactly in fp64, so one rounding to fp32 remains
            assert Fraction(float(exact)) == exact
            assert got[t, e] == np.float32(float(exact))


def test_softmax_matches_scipy_and_topk_weights():
    from scipy.special import softmax
    l = np.float32(RNG.normal(size=(9, 6)) * 3)
    p = oracle.softmax_rows(l)
    np.testing.assert_allclose(p, softmax(l.astype(np.float64), axis=1), rtol=1e-14, atol=0)
    for k in (1, 2, 6):
        idx = oracle.topk_select(l, k)
        w_on = oracle.routing_weights(p, idx, True)
        w_off = oracle.routing_weights(p, idx, False)
        np.testing.assert_allclose(w_on.sum(1), 1.0, rtol=0, atol=1e-15)
        np.testing.assert_array_equal(w_off, np.take_along_axis(p, idx.astype(np.int64), 1))
        if k == 1:
            assert np.all(w_on == 1.0)             # top-1 (Switch) weight is exactly 1
        if k == 6:
            np.testing.assert_allclose(w_on, w_off, rtol=1e-14)


def test_softmax_closed_forms():
    l = np.array([[0.5, 0.5, -np.inf]], dtype=np.float32)
    p = oracle.softmax_rows(l)
    assert p[0, 0] == p[0, 1] == 0.5 and p[0, 2] == 0.0
    l2 = np.array([[np.float32(2.0), np.float32(2.0) - np.float32(math.log(3.0))]], dtype=np.float32)
    p2 = oracle.softmax_rows(l2)
    r = math.exp(float(l2[0, 0]) - float(l2[0, 1]))
    np.testing.assert_allclose(p2[0], [r / (1 + r), 1 / (1 + r)], rtol=1e-15)
    np.testing.assert_allclose(p2[0], [0.75, 0.25], rtol=1e-7)


def _brute_topk(l, k):
    E = len(l)
    fr = [Fraction(float(v)) for v in l]
    best = None
    for sub in itertools.combinations(range(E), k):
        key = (sum(fr[e] for e in sub), tuple(-e for e in sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return set(best[1])


@pytest.mark.parametrize("trial", range(40))
def test_topk_brute_force_with_ties(trial):
    rng = np.random.default_rng(trial)
    E = int(rng.integers(1, 9))
    k = int(rng.integers(1, E + 1))
    # few distinct values so ties are common
    l = np.float32(rng.integers(-3, 3, size=E) * 0.25 + (0 if trial % 2 else rng.normal(size=E)))
    idx = oracle.topk_select(l[None, :], k)[0].tolist()
    assert set(idx) == _brute_topk(l, k)
    for a, b in zip(idx[:-1], idx[1:]):            # slots: larger first, ties lower index first
        assert l[a] > l[b] or (l[a] == l[b] and a < b)


# --------------------------------------------------------------------------
# fp8 e4m3fn decoding vs torch's float8_e4m3fn type
# --------------------------------------------------------------------------
def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.fp8_e4m3fn_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_dequantize_channel_axis():
    q = torch.tensor([[1.0, 2.0, -0.5], [4.0, 0.25, 448.0]]).to(torch.float8_e4m3fn)
    s = np.array([0.5, 2.0, 1.0 / 448.0], dtype=np.float32)
    w = oracle.dequantize(q.view(torch.uint8).numpy(), s, 1)
    np.testing.assert_array_equal(w, q.to(torch.float64).numpy() * s.astype(np.float64)[None, :])


# --------------------------------------------------------------------------
# Expert FFN and the whole layer
# --------------------------------------------------------------------------
def torch_dense_swiglu(x, wg, wu, wd):
    X = torch.from_numpy(np.asarray(x, np.float64))
    G = X @ torch.from_numpy(np.asarray(wg, np.float64))
    U = X @ torch.from_numpy(np.asarray(wu, np.float64))
    return (torch.nn.functional.silu(G) * U) @ torch.from_numpy(np.asarray(wd, np.float64))


def test_silu_against_torch_and_identity():
    z = np.linspace(-40, 40, 1001)
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(oracle.silu(z), ref, rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=1e-14, atol=1e-14)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def _layer(T, d, E, k, f, shared=False, seed=0):
    rng = np.random.default_rng(seed)
    x = bf16_values((T, d), 1.0, rng)
    Wg = bf16_values((d, E), 0.3, rng)
    ex = [(bf16_values((d, f), 0.2, rng), bf16_values((d, f), 0.2, rng),
           bf16_values((f, d), 0.2, rng)) for _ in range(E)]
    sh = (bf16_values((d, f), 0.2, rng), bf16_values((d, f), 0.2, rng),
          bf16_values((f, d), 0.2, rng)) if shared else None
    return x, Wg, ex, sh


def test_single_expert_top1_is_dense_swiglu():
    T, d, f = 13, 24, 40                        # d != f catches a transposed operand
    x, Wg, ex, _ = _layer(T, d, 1, 1, f)
    r = oracle.forward(x, Wg, None, 1, True, 0.0, lambda e: ex[e], 1)
    assert np.all(r["topk_w"] == 1.0)
    ref = torch_dense_swiglu(x, *ex[0]).numpy()
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("renorm", [True, False])
def test_gather_chosen_equals_all_experts(renorm):
    T, d, E, k, f = 17, 16, 6, 2, 24
    x, Wg, ex, _ = _layer(T, d, E, k, f, seed=3)
    r = oracle.forward(x, Wg, None, k, renorm, 0.0, lambda e: ex[e], E)
    full = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            full[t, r["topk_idx"][t, j]] = r["topk_w"][t, j]
    # every expert on every token, weighted by 0 where not chosen
    all_out = sum(full[:, e:e + 1] * torch_dense_swiglu(x, *ex[e]).numpy() for e in range(E))
    np.testing.assert_allclose(r["out"], all_out, rtol=1e-12, atol=1e-12)


def test_expert_permutation_invariance():
    T, d, E, k, f = 11, 16, 7, 3, 20
    x, Wg, ex, _ = _layer(T, d, E, k, f, seed=5)
    bias = np.float32(np.random.default_rng(9).normal(size=E))
    cert = oracle.routing_certificate(x, Wg, bias, k)
    assert cert["ok"].all()
    r0 = oracle.forward(x, Wg, bias, k, True, 0.0, lambda e: ex[e], E)
    pi = np.random.default_rng(11).permutation(E)
    r1 = oracle.forward(x, Wg[:, pi], bias[pi], k, True, 0.0, lambda e: ex[pi[e]], E)
    np.testing.assert_array_equal(pi[r1["topk_idx"]], r0["topk_idx"])
    np.testing.assert_allclose(r1["topk_w"], r0["topk_w"], rtol=1e-15)
    np.testing.assert_allclose(r1["out"], r0["out"], rtol=1e-13, atol=1e-13)


def test_shared_expert_is_additive():
    T, d, E, k, f = 9, 16, 5, 2, 24
    x, Wg, ex, sh = _layer(T, d, E, k, f, shared=True, seed=7)
    a = oracle.forward(x, Wg, None, k, True, 0.0, lambda e: ex[e], E, shared=sh)
    b = oracle.forward(x, Wg, None, k, True, 0.0, lambda e: ex[e], E, shared=None)
    np.testing.assert_allclose(a["out"] - b["out"], torch_dense_swiglu(x, *sh).numpy(),
                               rtol=1e-12, atol=1e-12)


def test_token_sample_matches_full_layer():
    T, d, E, k, f = 21, 16, 6, 2, 24
    x, Wg, ex, sh = _layer(T, d, E, k, f, shared=True, seed=8)
    full = oracle.forward(x, Wg, None, k, True, 1.0, lambda e: ex[e], E, shared=sh)
    toks = [20, 3, 0, 11]
    part = oracle.forward(x, Wg, None, k, True, 1.0, lambda e: ex[e], E, shared=sh, tokens=toks)
    np.testing.assert_allclose(part["out"], full["out"][toks], rtol=1e-13, atol=1e-15)
    for key in ("topk_idx", "sorted_assign", "inv_perm", "offsets"):
        np.testing.assert_array_equal(part[key], full[key])


def _fsum_layer(x, Wg, ex, k, renorm, cap, shared):
    """Pure-Python brute force with exactly rounded sums (math.fsum)."""
    T, d = x.shape
    E = Wg.shape[1]
    f = ex[0][0].shape[1]

    def ffn(v, wg, wu, wd):
        g = [math.fsum(v[i] * wg[i, c] for i in range(d)) for c in range(f)]
        u = [math.fsum(v[i] * wu[i, c] for i in range(d)) for c in range(f)]
        h = [g[c] / (1.0 + math.exp(-g[c])) * u[c] for c in range(f)]
        return [math.fsum(h[c] * wd[c, o] for c in range(f)) for o in range(d)]

    seen = [0] * E
    out = []
    for t in range(T):
        lg = [float(np.float32(math.fsum(x[t, i] * Wg[i, e] for i in range(d)))) for e in range(E)]
        m = max(lg)
        ex_ = [math.exp(v - m) for v in lg]
        z = math.fsum(ex_)
        pr = [v / z for v in ex_]
        chosen = sorted(range(E), key=lambda e: (-pr[e], e))[:k]
        den = math.fsum(pr[e] for e in chosen) if renorm else 1.0
        acc = [0.0] * d
        for e in chosen:
            keep = cap is None or seen[e] < cap
            seen[e] += 1
            if keep:
                y = ffn(x[t], *ex[e])
                acc = [acc[o] + pr[e] / den * y[o] for o in range(d)]
        if shared is not None:
            y = ffn(x[t], *shared)
            acc = [acc[o] + y[o] for o in range(d)]
        out.append(acc)
    return np.array(out)


@pytest.mark.parametrize("renorm,cf,shared", [(True, 0.0, False), (False, 0.0, True), (True, 1.0, False)])
def test_brute_force_tiny_layer(renorm, cf, shared):
    T, d, E, k, f = 6, 8, 4, 2, 16
    x, Wg, ex, sh = _layer(T, d, E, k, f, shared=shared, seed=21)
    cap = oracle.capacity(T, k, E, cf)
    r = oracle.forward(x, Wg, None, k, renorm, cf, lambda e: ex[e], E, shared=sh)
    if cf > 0:
        assert cap == 3
    ref = _fsum_layer(x, Wg, ex, k, renorm, cap, sh)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-13)


def test_tiny_config_subset_brute_force():
    """The tiny fp32 workload's own inputs, first tokens, checked by brute force."""
    cfg = synth.CONFIGS["tiny_f32"].with_(T=3, d=32, f=16)
    inp = synth.make_inputs(cfg)
    x = inp["x"].double().numpy()
    Wg = inp["W_g"].double().numpy()
    ex = [(inp["W_gate"][e].double().numpy(), inp["W_up"][e].double().numpy(),
           inp["W_down"][e].double().numpy()) for e in range(cfg.E)]
    r = oracle.forward(x, Wg, None, cfg.k, True, 0.0, lambda e: ex[e], cfg.E)
    ref = _fsum_layer(x, Wg, ex, cfg.k, True, None, None)
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-15)


def test_certificate_flags_near_ties():
    x = np.array([[1.0, 1.0]])
    W = np.array([[0.5, 0.5, 0.1], [0.25, 0.25, 0.0]])    # experts 0 and 1 tie exactly
    c = oracle.routing_certificate(x, W, None, 2)
    assert not c["ok"][0]
    W2 = np.array([[0.5, 0.25, 0.1], [0.25, 0.25, 0.0]])
    assert oracle.routing_certificate(x, W2, None, 2)["ok"][0]


def _fp64_sum_in_order(terms, order):
    acc = 0.0
    for i in order:
        acc = acc + float(terms[i])              # one IEEE fp64 addition per term
    return acc


def test_logit_error_bound_holds_for_every_summation_order():
    """The certificate's bound against the exact sum (Fractions) of every
    ordering of the additions.  Adding tiny terms one by one to 1 loses each
    of them (ties to even), so some order misses the exact sum by (d - 1)
    units of roundoff: more than half of the bound, which a halved bound
    would no longer cover."""
    u = 2.0 ** -53
    d = 7
    x = np.ones((1, d))
    W = np.array([[1.0], *[[u]] * (d - 1)])
    terms = (x[0] * W[:, 0]).tolist()
    exact = sum(Fraction(t) for t in terms)
    worst = max(abs(Fraction(_fp64_sum_in_order(terms, o)) - exact) for o in itertools.permutations(range(d)))
    bound = float(oracle.logit_error_bound(x, W)[0, 0])
    assert worst == Fraction(d - 1) * Fraction(u)
    assert Fraction(bound) >= worst
    assert worst > Fraction(bound) / 2
    # with a bias term (d + 1 additions) and random mixed-sign terms
    rng = np.random.default_rng(5)
    for _ in range(20):
        x = rng.normal(size=(1, 6)) * np.exp2(rng.integers(-30, 30, size=(1, 6)))
        W = rng.normal(size=(6, 1))
        b = rng.normal(size=1)
        terms = (x[0] * W[:, 0]).tolist() + [float(b[0])]
        if any(Fraction(t) != Fraction(x[0, i]) * Fraction(W[i, 0]) for i, t in enumerate(terms[:6])):
            continue                              # keep only exact products
        exact = sum(Fraction(t) for t in terms)
        bound = Fraction(float(oracle.logit_error_bound(x, W, b)[0, 0]))
        for o in itertools.permutations(range(7)):
            assert abs(Fraction(_fp64_sum_in_order(terms, o)) - exact) <= bound


def test_certificate_rejects_a_token_whose_selection_depends_on_the_order():
    """Expert 1's sum lies a quarter fp64 ulp above the midpoint between the
    fp32 values 1 and 1 + 2^-23.  Depending on the order of its additions it
    rounds to either, so its fp32 logit either beats expert 0's (exactly 1)
    or ties with it, and the tie goes to expert 0: the top-1 is not fixed.
    The fp64 error bounds are ~1e-15 against a gap of 6e-8, so only the
    certificate's fp32 ulp term can reject this token."""
    m = 1.0 + 2.0 ** -24
    e1, e2 = 0.75 * 2.0 ** -52, -0.5 * 2.0 ** -52
    x = np.ones((1, 3))
    W = np.array([[1.0, m], [0.0, e1], [0.0, e2]])
    picks = set()
    for o in itertools.permutations(range(3)):
        l32 = np.array([[np.float32(_fp64_sum_in_order(W[:, e], o)) for e in range(2)]], dtype=np.float32)
        picks.add(int(oracle.topk_select(l32, 1)[0, 0]))
    assert picks == {0, 1}
    c = oracle.routing_certificate(x, W, None, 1)
    assert not c["ok"][0]
    assert float(c["bound"].max()) < 1e-14
    # well apart (expert 1 a few fp32 ulps above expert 0): certified, and every order agrees
    W2 = W.copy()
    W2[0, 1] = 1.0 + 2.0 ** -20
    assert oracle.routing_certificate(x, W2, None, 1)["ok"][0]
    assert {int(oracle.topk_select(np.array([[np.float32(_fp64_sum_in_order(W2[:, e], o)) for e in range(2)]],
                                            dtype=np.float32), 1)[0, 0])
            for o in itertools.permutations(range(3))} == {1}


@pytest.mark.parametrize("seed", range(6))
def test_certificate_is_sound_against_every_summation_order(seed):
    """Tiny routers with planted near-ties: wherever the certificate accepts a
    token, every ordering of every expert's additions (bias included) gives the
    same fp32 top-k and slot order."""
    rng = np.random.default_rng(seed)
    T, d, E, k = 6, 4, 4, 2
    x = np.float32(rng.normal(size=(T, d))).astype(np.float64)
    W = np.float32(rng.normal(size=(d, E))).astype(np.float64)
    W[:, 1] = W[:, 0] + np.float32(rng.normal(size=d) * 1e-7)   # experts 0 and 1 nearly tie
    b = np.float32(rng.normal(size=E) * 0.1).astype(np.float64)
    cert = oracle.routing_certificate(x, W, b, k)
    orders = list(itertools.permutations(range(d + 1)))
    for t in range(T):
        seen = set()
        for o in orders[::7]:
            l32 = np.array([[np.float32(_fp64_sum_in_order(list(x[t] * W[:, e]) + [b[e]], o)) for e in range(E)]],
                           dtype=np.float32)
            seen.add(tuple(oracle.topk_select(l32, k)[0].tolist()))
        if cert["ok"][t]:
            assert len(seen) == 1, (t, seen)


def test_selection_uses_fp32_logits_where_fp64_probabilities_merge():
    """Logits more than ~745 below the maximum have fp64 probabilities that
    underflow to 0, so ranking probabilities would tie experts 2 and 3 and
    take the lower index.  The selection is made on the fp32 logits, which
    stay distinct: expert 3 (-1000) comes before expert 2 (-1001).  The token
    is certified: its logit gaps are exact and large."""
    l = np.array([[0.0, 0.5, -1001.0, -1000.0]], dtype=np.float32)
    p = oracle.softmax_rows(l)
    assert p[0, 2] == p[0, 3] == 0.0
    assert oracle.topk_select(l, 3)[0].tolist() == [1, 0, 3]
    x = np.ones((1, 1))
    assert oracle.routing_certificate(x, l.astype(np.float64), None, 3)["ok"][0]
    w = oracle.routing_weights(p, oracle.topk_select(l, 3), True)
    assert w[0, 2] == 0.0 and w[0].sum() == pytest.approx(1.0, rel=1e-15)
    # an exact fp32 tie among the chosen experts is rejected (the tie order is a convention)
    assert not oracle.routing_certificate(x, np.array([[0.0, 0.5, -1.0, -1.0]]), None, 3)["ok"][0]


def test_workload_shapes_match_pages(golden_dir):
    rows = read_golden(golden_dir, "mixtral_shapes.txt")
    for name in ("mixtral_decode", "mixtral_decode_b8", "mixtral_prefill"):
        c = synth.CONFIGS[name]
        assert (c.d, c.f, c.E, c.k) == (rows["hidden_size"][0], rows["intermediate_size"][0],
                                        rows["num_local_experts"][0], rows["num_experts_per_tok"][0])


# ----------------------------------------------------------------------------
# Router telemetry ([SWT] "Load Balancing Loss")
# ----------------------------------------------------------------------------
def test_router_telemetry_closed_forms():
    T, E, k = 12, 6, 2
    # equal logits: every probability is 1/E and ties pick experts 0..k-1 for
    # every token, so routed = [T, T, 0, ...] and the loss is E * k * (1/E) = k
    l = np.zeros((T, E), dtype=np.float32)
    idx = oracle.topk_select(l, k)
    r = oracle.router_telemetry(l, idx, E)
    assert r["routed"].tolist() == [T, T, 0, 0, 0, 0]
    np.testing.assert_allclose(r["prob_mean"], 1.0 / E, rtol=1e-15)
    assert r["lb_loss"] == pytest.approx(k, rel=1e-14)
    # balanced routing with uniform probabilities: loss = E * sum (1/E)(k/E) = k
    bal = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)], dtype=np.int32)
    rb = oracle.router_telemetry(l, bal, E)
    assert rb["routed"].tolist() == [T * k // E] * E
    assert rb["lb_loss"] == pytest.approx(k, rel=1e-14)
    # all probability on expert 0 and top-1 routing there: loss -> E
    lc = np.full((T, E), -60.0, dtype=np.float32)
    lc[:, 0] = 0.0
    rc = oracle.router_telemetry(lc, np.zeros((T, 1), dtype=np.int32), E)
    assert rc["routed"].tolist() == [T] + [0] * (E - 1)
    assert rc["lb_loss"] == pytest.approx(E, rel=1e-20 + 1e-12)


def test_router_telemetry_worked_example():
    # two experts, logits 0 and ln 3: softmax [1/4, 3/4]
    ln3 = np.float32(math.log(3.0))
    # tokens with mirrored logits, top-1: P = [1/2, 1/2], one token each -> loss 2 (1/4 + 1/4) = 1
    l = np.array([[0.0, ln3], [ln3, 0.0]], dtype=np.float32)
    r = oracle.router_telemetry(l, np.array([[1], [0]], dtype=np.int32), 2)
    np.testing.assert_allclose(r["prob_mean"], [0.5, 0.5], rtol=1e-7)
    assert r["lb_loss"] == pytest.approx(1.0, rel=1e-7)
    # both tokens [0, ln 3], both routed to expert 1: P = [1/4, 3/4], f = [0, 1] -> loss 2 * 3/4 = 1.5
    # (the renormalised top-1 weight would give P = [0, 1] and loss 2)
    l2 = np.array([[0.0, ln3], [0.0, ln3]], dtype=np.float32)
    r2 = oracle.router_telemetry(l2, np.array([[1], [1]], dtype=np.int32), 2)
    np.testing.assert_allclose(r2["prob_mean"], [0.25, 0.75], rtol=1e-7)
    assert r2["routed"].tolist() == [0, 2]
    assert r2["lb_loss"] == pytest.approx(1.5, rel=1e-7)


def test_router_telemetry_invariants():
    rng = np.random.default_rng(21)
    T, E, k = 37, 9, 3
    l = rng.normal(size=(T, E)).astype(np.float32)
    idx = oracle.topk_select(l, k)
    r = oracle.router_telemetry(l, idx, E)
    assert math.fsum(r["prob_mean"]) == pytest.approx(1.0, rel=1e-14)
    assert r["routed"].sum() == T * k
    np.testing.assert_array_equal(r["routed"], np.bincount(idx.ravel(), minlength=E))
    # relabelling the experts permutes the per-expert outputs and keeps the loss
    pi = rng.permutation(E)
    inv = np.argsort(pi)
    rp = oracle.router_telemetry(l[:, pi], inv[idx].astype(np.int32), E)
    np.testing.assert_array_equal(rp["routed"], r["routed"][pi])
    np.testing.assert_allclose(rp["prob_mean"], r["prob_mean"][pi], rtol=1e-14)
    assert rp["lb_loss"] == pytest.approx(r["lb_loss"], rel=1e-14)
    # empty batch
    r0 = oracle.router_telemetry(np.zeros((0, E), dtype=np.float32), np.zeros((0, k), dtype=np.int32), E)
    assert r0["routed"].sum() == 0 and r0["lb_loss"] == 0.0


# ----------------------------------------------------------------------------
# Expert-choice routing (Design Patterns, Pattern 3)
# ----------------------------------------------------------------------------
def test_expert_choice_capacity_closed_forms():
    assert oracle.expert_choice_capacity(10, 2, 4, 0.0) == 5          # T k / E
    assert oracle.expert_choice_capacity(10, 2, 4, 1.25) == 7         # ceil(6.25)
    assert oracle.expert_choice_capacity(10, 2, 4, 0.01) == 1         # at least one token
    assert oracle.expert_choice_capacity(10, 2, 4, 100.0) == 10       # at most T


@pytest.mark.parametrize("seed,T,E,k,cf,renorm", [(1, 9, 4, 2, 0.0, True), (2, 13, 5, 1, 1.5, False),
                                                  (3, 6, 3, 3, 0.0, True), (4, 17, 6, 2, 0.7, False)])
def test_expert_choice_selection_property(seed, T, E, k, cf, renorm):
    rng = np.random.default_rng(seed)
    l = rng.normal(size=(T, E)).astype(np.float32)
    l[2] = l[5 % T]                                    # a duplicated token row: equal scores
    r = oracle.expert_choice_routing(l, k, cf, renorm)
    C, s = r["capacity"], r["scores"]
    assert C == oracle.expert_choice_capacity(T, k, E, cf)
    assert r["offsets"].tolist() == [e * C for e in range(E + 1)]
    for e in range(E):
        chosen = [t for t in range(T) if r["pos"][t, e] >= 0]
        assert len(chosen) == C
        rows = r["sorted_tokens"][r["offsets"][e]:r["offsets"][e + 1]].tolist()
        assert rows == sorted(chosen)                  # rows in ascending token order
        assert all(r["pos"][t, e] == r["offsets"][e] + rows.index(t) for t in chosen)
        for t in chosen:                               # every chosen token beats every other one
            for u in range(T):
                if r["pos"][u, e] < 0:
                    assert s[t, e] > s[u, e] or (s[t, e] == s[u, e] and t < u)
    times = (r["pos"] >= 0).sum(axis=1)
    assert times.sum() == E * C
    for t in range(T):
        w = r["weight"][t]
        if renorm and times[t] > 0:
            assert math.fsum(w) == pytest.approx(1.0, rel=1e-15)
        if not renorm:
            np.testing.assert_array_equal(w[r["pos"][t] >= 0], s[t][r["pos"][t] >= 0].astype(np.float64))
        assert np.all(w[r["pos"][t] < 0] == 0.0)


def test_expert_choice_ties_go_to_lower_token():
    l = np.zeros((7, 3), dtype=np.float32)             # every score 1/3
    r = oracle.expert_choice_routing(l, 1, 0.0, False)
    assert r["capacity"] == 3
    assert r["sorted_tokens"].tolist() == [0, 1, 2] * 3


def test_expert_choice_all_tokens_equals_token_choice_over_all_experts():
    # C = T: every expert takes every token with weight = its full-softmax score,
    # which is the token-choice layer with k = E and no renormalisation
    T, d, E, f = 8, 16, 4, 24
    x, Wg, ex, sh = _layer(T, d, E, E, f, shared=True, seed=3)
    ec = oracle.expert_choice_forward(x, Wg, None, E, False, 0.0, lambda e: ex[e], E, shared=sh)
    assert ec["capacity"] == T
    tc = oracle.forward(x, Wg, None, E, False, 0.0, lambda e: ex[e], E, shared=sh)
    np.testing.assert_allclose(ec["out"], tc["out"], rtol=2e-7, atol=1e-9)  # fp32-rounded scores


def test_expert_choice_single_expert_is_dense_swiglu():
    T, d, f = 11, 24, 40
    x, Wg, ex, _ = _layer(T, d, 1, 1, f)
    r = oracle.expert_choice_forward(x, Wg, None, 1, True, float(T), lambda e: ex[e], 1)
    assert r["capacity"] == T and np.all(r["weight"] == 1.0)
    np.testing.assert_allclose(r["out"], torch_dense_swiglu(x, *ex[0]).numpy(), rtol=1e-12, atol=1e-12)


def test_expert_choice_relabelling_invariance():
    T, d, E, k, f = 10, 16, 5, 2, 20
    x, Wg, ex, _ = _layer(T, d, E, k, f, seed=8)
    r0 = oracle.expert_choice_forward(x, Wg, None, k, True, 0.0, lambda e: ex[e], E)
    pi = np.random.default_rng(4).permutation(E)       # experts relabelled
    r1 = oracle.expert_choice_forward(x, Wg[:, pi], None, k, True, 0.0, lambda e: ex[pi[e]], E)
    np.testing.assert_array_equal(r1["pos"] >= 0, (r0["pos"] >= 0)[:, pi])
    np.testing.assert_allclose(r1["out"], r0["out"], rtol=1e-13, atol=1e-13)
    tp = np.random.default_rng(5).permutation(T)       # tokens relabelled (scores are distinct)
    r2 = oracle.expert_choice_forward(x[tp], Wg, None, k, True, 0.0, lambda e: ex[e], E)
    np.testing.assert_allclose(r2["out"], r0["out"][tp], rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# MXFP8 block scaling (E4M3 elements, one power-of-two scale per 32 values)
# --------------------------------------------------------------------------
_POS = [(c, float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)))
        for c in range(0x7F)]                      # the 127 non-negative finite codes, from torch's decoder


def _brute_e4m3(v):
    """Nearest non-negative E4M3 value by exhaustive search in exact rationals,
    ties to the even code; magnitude clamped to 448 first, sign carried."""
    a = min(abs(Fraction(v)), Fraction(448))
    best = min(_POS, key=lambda cv: (abs(a - Fraction(cv[1])), cv[0] & 1))
    return best[0] | (0x80 if math.copysign(1.0, v) < 0 else 0)


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_encode(vals)
    assert np.array_equal(got, codes)              # includes -0 -> 0x80


def test_e4m3_encode_ties_saturation_and_subnormals():
    cases = [(1.0625, 0x38), (1.1875, 0x3A),       # midpoints: 1|1.125 -> 1 (even), 1.125|1.25 -> 1.25
             (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),   # subnormal midpoints
             (-(2.0 ** -10), 0x80), (5 * 2.0 ** -10, 0x02), (7 * 2.0 ** -10, 0x04),
             (448.0, 0x7E), (464.0, 0x7E), (1e30, 0x7E), (-1e30, 0xFE), (0.0, 0x00), (-0.0, 0x80),
             (240.0, 0x77), (248.0, 0x78), (232.0, 0x76)]   # 224 (0x76) | 240 (0x77) | 256 (0x78)
    for v, c in cases:
        assert oracle.e4m3_encode(np.array([v]))[0] == c, v
        assert _brute_e4m3(v) == c, v


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.normal(0, 1, 300) * np.exp2(rng.integers(-12, 10, 300)),
                        (rng.integers(-1200, 1200, 200) / 4.0) * 2.0 ** -9])   # many exact ties
    got = oracle.e4m3_encode(v)
    ref = np.array([_brute_e4m3(float(t)) for t in v], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e4m3_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(8)
    v = np.clip(rng.normal(0, 1, 50000) * np.exp2(rng.integers(-12, 9, 50000)), -448, 448).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v.astype(np.float64)), ref)


def test_mx_scale_rule_zero_block_and_powers_of_two():
    codes, sc = oracle.mx_quantize(np.zeros((2, 64)))
    assert np.all(codes == 0) and np.all(sc == 0)
    for p in (-130, -100, -3, 0, 5, 100):
        b = np.zeros(32)
        b[7] = -(2.0 ** p)
        codes, sc = oracle.mx_quantize(b[None, :])
        e = max(p - 8, -127)
        assert sc[0, 0] == e + 127
        if p - 8 >= -127:
            assert codes[0, 7] == 0xF8                 # -256 = -(2^8): exponent field 15, mantissa 0
    # the scaled block maximum lies in [256, 512) whenever the exponent is not clamped
    rng = np.random.default_rng(9)
    v = rng.normal(0, 1, (40, 32)) * np.exp2(rng.integers(-60, 60, (40, 1)))
    _, sc = oracle.mx_quantize(v)
    r = np.abs(v).max(axis=1) / np.exp2(sc[:, 0].astype(np.float64) - 127)
    assert np.all((r >= 256) & (r < 512))


def test_mx_quantize_blocks_are_independent_and_along_last_axis():
    rng = np.random.default_rng(10)
    v = rng.normal(0, 1, (3, 96)) * np.array([1e-3, 1.0, 1e3])[None, :].repeat(32, axis=1)
    codes, sc = oracle.mx_quantize(v)
    assert codes.shape == (3, 96) and sc.shape == (3, 3)
    for j in range(3):
        cj, sj = oracle.mx_quantize(v[:, 32 * j:32 * j + 32])
        assert np.array_equal(cj, codes[:, 32 * j:32 * j + 32]) and np.array_equal(sj[:, 0], sc[:, j])


def test_mx_roundtrip_exact_for_representable_blocks_and_error_bound():
    rng = np.random.default_rng(11)
    # blocks built from E4M3 values with the maximum in [256, 448], times 2^s: exact round trip
    pos = np.array([v for _, v in _POS])
    el = rng.choice(pos, (16, 32)) * rng.choice([-1.0, 1.0], (16, 32))
    el[:, 0] = rng.choice(pos[(pos >= 256)], 16)
    s = rng.integers(-20, 20, (16, 1)).astype(np.float64)
    v = el * np.exp2(s)
    np.testing.assert_array_equal(oracle.mx_roundtrip(v), v)
    # general blocks: half an E4M3 step relative (2^-4) or half the smallest
    # subnormal step times the scale; clamped values lose less than 64 * scale
    v = rng.normal(0, 1, (200, 32)) * np.exp2(rng.integers(-30, 30, (200, 1)))
    q = oracle.mx_roundtrip(v)
    _, sc = oracle.mx_quantize(v)
    scale = np.exp2(sc.astype(np.float64) - 127).repeat(32, axis=1)
    err = np.abs(q - v)
    clamped = np.abs(v) > 448 * scale
    assert np.all(err[~clamped] <= np.maximum(2.0 ** -4 * np.abs(v), 2.0 ** -10 * scale)[~clamped])
    assert np.all(err[clamped] < 64 * scale[clamped])
    assert np.all(np.abs(q[clamped]) == 448 * scale[clamped])


def test_mx_dequantize_values():
    codes = np.array([[0x38] + [0xB8] + [0x01] + [0] * 29])   # 1, -1, 2^-9
    for s in (0, 120, 127, 130, 254):
        got = oracle.mx_dequantize(codes, np.array([[s]], dtype=np.uint8))
        f = 2.0 ** (s - 127)
        assert got[0, 0] == f and got[0, 1] == -f and got[0, 2] == 2.0 ** -9 * f and np.all(got[0, 3:] == 0)


# --------------------------------------------------------------------------
# MXFP4 block scaling (E2M1 elements, the same power-of-two scale per 32 values)
# --------------------------------------------------------------------------
# The OCP E2M1 element values written out (sign-magnitude, codes 0..7 and 8..15)
_E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _brute_e2m1(v):
    """Nearest E2M1 magnitude by exhaustive search in exact rationals, ties to
    the even code; magnitude clamped to 6 first, sign carried as bit 3."""
    a = min(abs(Fraction(v)), Fraction(6))
    best = min(range(8), key=lambda c: (abs(a - Fraction(_E2M1_TABLE[c])), c & 1))
    return best | (8 if math.copysign(1.0, v) < 0 else 0)


def test_e2m1_decode_table():
    got = oracle.e2m1_decode(np.arange(16, dtype=np.uint8))
    want = np.array(_E2M1_TABLE + [-t for t in _E2M1_TABLE])
    assert np.array_equal(got, want) and np.signbit(got[8])        # code 8 is -0
    assert np.array_equal(oracle.e2m1_decode(np.array([0x17, 0xF2], dtype=np.uint8)), [6.0, 1.0])   # low nibble


def test_e2m1_encode_roundtrip_ties_and_saturation():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(oracle.e2m1_encode(oracle.e2m1_decode(codes)), codes)
    # every midpoint goes to the even code: 0|0.5 -> 0, 0.5|1 -> 1, 1|1.5 -> 1, 1.5|2 -> 2, 2|3 -> 2, 3|4 -> 4, 4|6 -> 4
    for v, c in [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
                 (6.0, 7), (7.99, 7), (1e30, 7), (-1e30, 15), (-0.1, 8), (-0.0, 8), (0.0, 0), (0.2500001, 1)]:
        assert oracle.e2m1_encode(np.array([v]))[0] == c, v
        assert _brute_e2m1(v) == c, v


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(17)
    v = np.concatenate([rng.normal(0, 2, 400), rng.integers(-28, 28, 200) / 4.0])   # many exact ties
    got = oracle.e2m1_encode(v)
    ref = np.array([_brute_e2m1(float(t)) for t in v], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_mx4_scale_rule_zero_block_and_block_maximum():
    codes, sc = oracle.mx4_quantize(np.zeros((2, 64)))
    assert np.all(codes == 0) and np.all(sc == 0)
    for p in (-130, -100, -3, 0, 5, 100):
        b = np.zeros(32)
        b[3] = -(2.0 ** p)
        codes, sc = oracle.mx4_quantize(b[None, :])
        assert sc[0, 0] == max(p - 2, -127) + 127
        if p - 2 >= -127:
            assert codes[0, 3] == 8 | 6                 # -4 = -(2^2): the scaled maximum of a power of two
    rng = np.random.default_rng(18)
    v = rng.normal(0, 1, (40, 32)) * np.exp2(rng.integers(-60, 60, (40, 1)))
    _, sc = oracle.mx4_quantize(v)
    r = np.abs(v).max(axis=1) / np.exp2(sc[:, 0].astype(np.float64) - 127)
    assert np.all((r >= 4) & (r < 8))                   # 2^emax <= scaled max < 2^(emax+1)


def test_mx4_roundtrip_exact_for_representable_blocks_and_error_bound():
    rng = np.random.default_rng(19)
    pos = np.array(_E2M1_TABLE)
    el = rng.choice(pos, (16, 32)) * rng.choice([-1.0, 1.0], (16, 32))
    el[:, 0] = rng.choice([4.0, 6.0], 16)               # block maximum in [4, 8): scale 2^s exactly
    s = rng.integers(-20, 20, (16, 1)).astype(np.float64)
    v = el * np.exp2(s)
    np.testing.assert_array_equal(oracle.mx4_dequantize(*oracle.mx4_quantize(v)), v)
    # general blocks: half an element step, at most a quarter of the magnitude or
    # of the scale; clamped values (|v| in (6, 8) x scale) lose less than 2 x scale
    v = rng.normal(0, 1, (300, 32)) * np.exp2(rng.integers(-30, 30, (300, 1)))
    c, sc = oracle.mx4_quantize(v)
    q = oracle.mx4_dequantize(c, sc)
    scale = np.exp2(sc.astype(np.float64) - 127).repeat(32, axis=1)
    err = np.abs(q - v)
    clamped = np.abs(v) > 6 * scale
    assert np.all(err[~clamped] <= np.maximum(0.25 * np.abs(v), 0.25 * scale)[~clamped])
    assert np.all(err[clamped] < 2 * scale[clamped]) and np.all(np.abs(q[clamped]) == 6 * scale[clamped])
    # blocks are independent and run along the last axis
    w = rng.normal(0, 1, (20, 64)) * np.array([1e-3, 1e3]).repeat(32)[None, :]
    cj, sj = oracle.mx4_quantize(w[:, 32:64])
    c2, s2 = oracle.mx4_quantize(w)
    assert np.array_equal(cj, c2[:, 32:64]) and np.array_equal(sj[:, 0], s2[:, 1])


def test_quant_hooks_are_on_expert_inputs_and_activations():
    T, d, E, k, f = 11, 16, 4, 2, 24
    x, Wg, ex, sh = _layer(T, d, E, k, f, shared=True, seed=3)
    base = oracle.forward(x, Wg, None, k, True, 0.0, lambda e: ex[e], E, sh)
    ident = oracle.forward(x, Wg, None, k, True, 0.0, lambda e: ex[e], E, sh,
                           quant_x=lambda X: X, quant_h=lambda H: H)
    np.testing.assert_array_equal(ident["out"], base["out"])
    # quant_x: experts see |x| while routing still uses x
    r = oracle.forward(x, Wg, None, k, True, 0.0, lambda e: ex[e], E, sh, quant_x=np.abs)
    assert np.array_equal(r["topk_idx"], base["topk_idx"])
    ref = torch_dense_swiglu(np.abs(x), *sh).numpy()
    for t in range(T):
        for j in range(k):
            ref[t] += base["topk_w"][t, j] * torch_dense_swiglu(np.abs(x[t:t + 1]), *ex[base["topk_idx"][t, j]]).numpy()[0]
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
    # quant_h acts on silu(x Wg) * (x Wu), before the down projection
    relu = lambda H: np.maximum(H, 0.0)
    r = oracle.forward(x, Wg, None, k, True, 0.0, lambda e: ex[e], E, sh, quant_h=relu)

    def dense_relu(xx, wg, wu, wd):
        X = torch.from_numpy(xx)
        H = torch.nn.functional.silu(X @ torch.from_numpy(wg)) * (X @ torch.from_numpy(wu))
        return torch.relu(H) @ torch.from_numpy(wd)
    ref = dense_relu(x, *sh).numpy()
    for t in range(T):
        for j in range(k):
            ref[t] += base["topk_w"][t, j] * dense_relu(x[t:t + 1], *ex[base["topk_idx"][t, j]]).numpy()[0]
    np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Backward (gradients of L = sum(dout * out))
# --------------------------------------------------------------------------
def _fd(fun, v, h):
    """Central differences of the scalar fun at every element of v."""
    g = np.zeros_like(v)
    it = np.nditer(v, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = v[i]
        v[i] = old + h
        fp = fun()
        v[i] = old - h
        fm = fun()
        v[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def test_dsilu_against_torch_autograd_and_differences():
    z = np.linspace(-30, 30, 601)
    zt = torch.from_numpy(z.copy()).requires_grad_(True)
    torch.nn.functional.silu(zt).sum().backward()
    np.testing.assert_allclose(oracle.dsilu(z), zt.grad.numpy(), rtol=1e-13, atol=1e-15)
    h = 1e-6
    np.testing.assert_allclose(oracle.dsilu(z), (oracle.silu(z + h) - oracle.silu(z - h)) / (2 * h),
                               rtol=1e-6, atol=1e-8)


def test_expert_ffn_backward_against_torch_autograd():
    rng = np.random.default_rng(21)
    n, d, f = 7, 12, 20                                # d != f: a transposed operand fails
    X, Wg, Wu, Wd = (rng.normal(0, s, sh) for s, sh in ((1, (n, d)), (0.3, (d, f)), (0.3, (d, f)), (0.3, (f, d))))
    dY = rng.normal(0, 1, (n, d))
    b = oracle.expert_ffn_backward(X, Wg, Wu, Wd, dY)
    ts = [torch.from_numpy(a.copy()).requires_grad_(True) for a in (X, Wg, Wu, Wd)]
    Y = (torch.nn.functional.silu(ts[0] @ ts[1]) * (ts[0] @ ts[2])) @ ts[3]
    (Y * torch.from_numpy(dY)).sum().backward()
    for key, t in zip(("dX", "dW_gate", "dW_up", "dW_down"), ts):
        np.testing.assert_allclose(b[key], t.grad.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("renorm", [True, False])
def test_routing_weights_backward_against_differences(renorm):
    rng = np.random.default_rng(22)
    T, E, k = 5, 7, 3
    l = rng.normal(0, 1.5, (T, E))
    idx = oracle.topk_select(l, k)
    g = rng.normal(0, 1, (T, k))
    dl = oracle.routing_weights_backward(oracle.softmax_rows(l), idx, g, renorm)
    fun = lambda: float((oracle.routing_weights(oracle.softmax_rows(l), idx, renorm) * g).sum())
    np.testing.assert_allclose(dl, _fd(fun, l, 1e-6), rtol=1e-6, atol=1e-9)
    if renorm:                                          # a softmax over the chosen logits: rows sum to 0
        np.testing.assert_allclose(dl.sum(axis=1), 0.0, atol=1e-14)


def _bwd_layer(T, d, E, k, f, shared, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (T, d))
    Wg = rng.normal(0, 0.6, (d, E))
    bias = rng.normal(0, 0.3, E)
    ex = [tuple(rng.normal(0, 0.3, sh) for sh in ((d, f), (d, f), (f, d))) for _ in range(E)]
    sh = tuple(rng.normal(0, 0.3, s) for s in ((d, f), (d, f), (f, d))) if shared else None
    dout = rng.normal(0, 1, (T, d))
    return x, Wg, bias, ex, sh, dout


@pytest.mark.parametrize("renorm,cf,shared", [(True, 0.0, False), (False, 0.0, True), (True, 0.7, True)])
def test_layer_backward_against_central_differences(renorm, cf, shared):
    """Every gradient of the whole layer (router included, with unrounded
    logits) against central differences of L = sum(dout * out)."""
    T, d, E, k, f = 6, 5, 4, 2, 3
    x, Wg, bias, ex, sh, dout = _bwd_layer(T, d, E, k, f, shared, seed=23 + int(renorm) + int(10 * cf))
    run = lambda: oracle.forward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh, round_logits=False)
    L = lambda: float((run()["out"] * dout).sum())
    r0 = run()
    b = oracle.backward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh, dout, round_logits=False)
    h, tol = 1e-5, dict(rtol=2e-5, atol=2e-7)
    np.testing.assert_allclose(b["dx"], _fd(L, x, h), **tol)
    np.testing.assert_allclose(b["dW_g"], _fd(L, Wg, h), **tol)
    np.testing.assert_allclose(b["d_bias"], _fd(L, bias, h), **tol)
    for e in range(E):
        for key, m in (("dW_gate", 0), ("dW_up", 1), ("dW_down", 2)):
            np.testing.assert_allclose(b[key][e], _fd(L, ex[e][m], h), **tol)
    if shared:
        for key, m in (("dWs_gate", 0), ("dWs_up", 1), ("dWs_down", 2)):
            np.testing.assert_allclose(b[key], _fd(L, sh[m], h), **tol)
    # the selection did not move under the perturbations, and capacity dropped something when asked to
    assert np.array_equal(run()["topk_idx"], r0["topk_idx"])
    if cf:
        assert r0["n_dropped"] > 0
        assert np.all(b["g"][r0["inv_perm"].reshape(T, k) < 0] == 0.0)


def test_layer_backward_against_torch_autograd_gather_all_form():
    """The chosen-experts backward equals torch autograd of the run-every-expert
    form (zero weight for unchosen or dropped assignments), with rounded logits."""
    T, d, E, k, f = 9, 6, 5, 2, 4
    x, Wg, bias, ex, sh, dout = _bwd_layer(T, d, E, k, f, True, seed=31)
    cf = 0.9
    r = oracle.forward(x, Wg, bias, k, True, cf, lambda e: ex[e], E, sh)
    b = oracle.backward(x, Wg, bias, k, True, cf, lambda e: ex[e], E, sh, dout)
    keep = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            if r["inv_perm"][t * k + j] >= 0:
                keep[t, r["topk_idx"][t, j]] = 1.0
    chosen = np.zeros((T, E))
    for t in range(T):
        chosen[t, r["topk_idx"][t]] = 1.0
    tt = lambda a: torch.from_numpy(np.array(a, dtype=np.float64)).requires_grad_(True)
    xt, Wgt, bt = tt(x), tt(Wg), tt(bias)
    ext = [[tt(m) for m in trip] for trip in ex]
    sht = [tt(m) for m in sh]
    lg = xt @ Wgt + bt
    p = torch.softmax(lg, dim=1) * torch.from_numpy(chosen)
    w = p / p.sum(dim=1, keepdim=True)
    ffn = lambda X, a, b_, c: (torch.nn.functional.silu(X @ a) * (X @ b_)) @ c
    out = sum(w[:, e:e + 1] * torch.from_numpy(keep[:, e:e + 1]) * ffn(xt, *ext[e]) for e in range(E))
    out = out + ffn(xt, *sht)
    (out * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(out.detach().numpy(), r["out"], rtol=1e-6, atol=1e-6)   # fp32 logits vs fp64
    tol = dict(rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(b["dx"], xt.grad.numpy(), **tol)
    np.testing.assert_allclose(b["dW_g"], Wgt.grad.numpy(), **tol)
    np.testing.assert_allclose(b["d_bias"], bt.grad.numpy(), **tol)
    for e in range(E):
        np.testing.assert_allclose(b["dW_gate"][e], ext[e][0].grad.numpy(), **tol)
        np.testing.assert_allclose(b["dW_up"][e], ext[e][1].grad.numpy(), **tol)
        np.testing.assert_allclose(b["dW_down"][e], ext[e][2].grad.numpy(), **tol)
    for key, m in (("dWs_gate", 0), ("dWs_up", 1), ("dWs_down", 2)):
        np.testing.assert_allclose(b[key], sht[m].grad.numpy(), **tol)


def test_layer_backward_single_expert_is_dense_backward():
    T, d, f = 8, 6, 10
    x, Wg, bias, ex, _, dout = _bwd_layer(T, d, 1, 1, f, False, seed=33)
    b = oracle.backward(x, Wg, bias, 1, True, 0.0, lambda e: ex[e], 1, None, dout)
    dense = oracle.expert_ffn_backward(x, *ex[0], dout)
    np.testing.assert_allclose(b["dx"], dense["dX"], rtol=1e-13, atol=1e-13)   # w = 1: no router gradient
    assert np.all(b["d_logits"] == 0.0) and np.all(b["dW_g"] == 0.0)
    np.testing.assert_allclose(b["dW_down"][0], dense["dW_down"], rtol=1e-13, atol=1e-13)


def test_layer_backward_relabelling_permutes_expert_gradients():
    T, d, E, k, f = 10, 6, 5, 2, 4
    x, Wg, bias, ex, _, dout = _bwd_layer(T, d, E, k, f, False, seed=35)
    perm = np.array([3, 0, 4, 1, 2])
    b = oracle.backward(x, Wg, bias, k, True, 0.0, lambda e: ex[e], E, None, dout)
    b2 = oracle.backward(x, Wg[:, perm], bias[perm], k, True, 0.0, lambda e: ex[perm[e]], E, None, dout)
    np.testing.assert_allclose(b2["dx"], b["dx"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b2["dW_g"], b["dW_g"][:, perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(b2["dW_down"], b["dW_down"][perm], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# Backward of the expert-choice layer
# --------------------------------------------------------------------------
@pytest.mark.parametrize("renorm,cf,shared", [(True, 1.0, False), (False, 1.0, True), (True, 1.5, True)])
def test_ec_layer_backward_against_central_differences(renorm, cf, shared):
    """Every gradient of the expert-choice layer (unrounded logits and scores)
    against central differences of L = sum(dout * out); the layer has tokens
    that no expert took and tokens that several experts took."""
    T, d, E, k, f = 8, 5, 4, 1, 3
    x, Wg, bias, ex, sh, dout = _bwd_layer(T, d, E, k, f, shared, seed=61 + int(renorm) + int(10 * cf))
    run = lambda: oracle.expert_choice_forward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh,
                                               round_logits=False)
    L = lambda: float((run()["out"] * dout).sum())
    r0 = run()
    taken = (r0["pos"] >= 0).sum(axis=1)
    assert (taken == 0).any() and (taken >= 2).any()
    b = oracle.expert_choice_backward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh, dout, round_logits=False)
    h, tol = 1e-5, dict(rtol=2e-5, atol=2e-7)
    np.testing.assert_allclose(b["dx"], _fd(L, x, h), **tol)
    np.testing.assert_allclose(b["dW_g"], _fd(L, Wg, h), **tol)
    np.testing.assert_allclose(b["d_bias"], _fd(L, bias, h), **tol)
    for e in range(E):
        for key, m in (("dW_gate", 0), ("dW_up", 1), ("dW_down", 2)):
            np.testing.assert_allclose(b[key][e], _fd(L, ex[e][m], h), **tol)
    if shared:
        for key, m in (("dWs_gate", 0), ("dWs_up", 1), ("dWs_down", 2)):
            np.testing.assert_allclose(b[key], _fd(L, sh[m], h), **tol)
    assert np.array_equal(run()["pos"], r0["pos"])      # the selection did not move
    assert np.all(b["g"][r0["pos"] < 0] == 0.0)
    assert np.all(b["d_logits"][taken == 0] == 0.0)       # untaken tokens: no router gradient


@pytest.mark.parametrize("renorm", [True, False])
def test_ec_backward_against_torch_autograd_gather_all_form(renorm):
    """The expert-choice backward equals torch autograd of the run-every-expert
    form (weight zero where the expert did not take the token), rounded logits."""
    T, d, E, k, f = 11, 6, 5, 2, 4
    x, Wg, bias, ex, sh, dout = _bwd_layer(T, d, E, k, f, True, seed=71 + int(renorm))
    cf = 0.8
    r = oracle.expert_choice_forward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh)
    b = oracle.expert_choice_backward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh, dout)
    mask = torch.from_numpy((r["pos"] >= 0).astype(np.float64))
    tt = lambda a: torch.from_numpy(np.array(a, dtype=np.float64)).requires_grad_(True)
    xt, Wgt, bt = tt(x), tt(Wg), tt(bias)
    ext = [[tt(m) for m in trip] for trip in ex]
    sht = [tt(m) for m in sh]
    p = torch.softmax(xt @ Wgt + bt, dim=1) * mask
    w = p / p.sum(dim=1, keepdim=True).clamp_min(1e-300) if renorm else p
    ffn = lambda X, a, b_, c: (torch.nn.functional.silu(X @ a) * (X @ b_)) @ c
    out = sum(w[:, e:e + 1] * ffn(xt, *ext[e]) for e in range(E)) + ffn(xt, *sht)
    (out * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(out.detach().numpy(), r["out"], rtol=1e-6, atol=1e-6)   # fp32 scores vs fp64
    tol = dict(rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(b["dx"], xt.grad.numpy(), **tol)
    np.testing.assert_allclose(b["dW_g"], Wgt.grad.numpy(), **tol)
    np.testing.assert_allclose(b["d_bias"], bt.grad.numpy(), **tol)
    for e in range(E):
        for key, m in (("dW_gate", 0), ("dW_up", 1), ("dW_down", 2)):
            np.testing.assert_allclose(b[key][e], ext[e][m].grad.numpy(), **tol)
    for key, m in (("dWs_gate", 0), ("dWs_up", 1), ("dWs_down", 2)):
        np.testing.assert_allclose(b[key], sht[m].grad.numpy(), **tol)


@pytest.mark.parametrize("renorm", [True, False])
def test_ec_backward_with_every_token_taken_is_the_token_choice_backward_with_k_equal_E(renorm):
    """C = T: every expert takes every token, so the layer is the token-choice
    layer with k = E (every expert chosen, no capacity) and both backwards agree."""
    T, d, E, f = 6, 5, 3, 4
    x, Wg, bias, ex, sh, dout = _bwd_layer(T, d, E, E, f, True, seed=81 + int(renorm))
    ec = oracle.expert_choice_backward(x, Wg, bias, E, renorm, 1.0, lambda e: ex[e], E, sh, dout, round_logits=False)
    assert ec["capacity"] == T and (ec["pos"] >= 0).all()
    tc = oracle.backward(x, Wg, bias, E, renorm, 0.0, lambda e: ex[e], E, sh, dout, round_logits=False)
    for key in ("dx", "dW_g", "d_bias", "dW_gate", "dW_up", "dW_down", "dWs_gate", "dWs_up", "dWs_down", "d_logits"):
        np.testing.assert_allclose(ec[key], tc[key], rtol=1e-12, atol=1e-13, err_msg=key)


# --------------------------------------------------------------------------
# Backward of block-scaled layers: the forward's quantisation of the expert
# inputs and of the activated rows, differentiated as the identity
# --------------------------------------------------------------------------
def _qh(H):
    return oracle.mx_roundtrip(H, as_fp32=True)


@pytest.mark.parametrize("ec", [False, True])
def test_backward_with_identity_hooks_is_the_plain_backward(ec):
    T, d, E, k, f = 9, 64, 4, 2, 64
    x, Wg, bias, ex, sh, dout = _bwd_layer(T, d, E, k, f, True, seed=91 + int(ec))
    fn = oracle.expert_choice_backward if ec else oracle.backward
    a = fn(x, Wg, bias, k, True, 0.9, lambda e: ex[e], E, sh, dout)
    b = fn(x, Wg, bias, k, True, 0.9, lambda e: ex[e], E, sh, dout, quant_x=lambda v: v, quant_h=lambda v: v)
    for key in ("dx", "dW_g", "d_bias", "dW_gate", "dW_up", "dW_down", "dWs_gate", "dWs_up", "dWs_down"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("ec,renorm", [(False, True), (False, False), (True, True)])
def test_block_scaled_backward_against_torch_autograd_straight_through(ec, renorm):
    """torch autograd of the run-every-expert form in which each quantiser is
    q(v) = v + (Q(v) - v).detach() (Q: the oracle's MX round trip, applied to
    the expert inputs and to the activated rows)."""
    T, d, E, k, f = 10, 64, 4, 2, 64
    x, Wg, bias, ex, sh, dout = _bwd_layer(T, d, E, k, f, True, seed=95 + int(ec) + 2 * int(renorm))
    cf = 0.9
    hooks = dict(quant_x=oracle.mx_roundtrip, quant_h=_qh)
    if ec:
        r = oracle.expert_choice_forward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh, **hooks)
        b = oracle.expert_choice_backward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh, dout, **hooks)
        mask = (r["pos"] >= 0).astype(np.float64)
    else:
        r = oracle.forward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh, **hooks)
        b = oracle.backward(x, Wg, bias, k, renorm, cf, lambda e: ex[e], E, sh, dout, **hooks)
        mask = np.zeros((T, E))
        for t in range(T):
            for j in range(k):
                if r["inv_perm"][t * k + j] >= 0:
                    mask[t, r["topk_idx"][t, j]] = 1.0
        chosen = np.zeros((T, E))
        for t in range(T):
            chosen[t, r["topk_idx"][t]] = 1.0
    tt = lambda a: torch.from_numpy(np.array(a, dtype=np.float64)).requires_grad_(True)
    ste = lambda v, Q: v + (torch.from_numpy(Q(v.detach().numpy())) - v).detach()
    xt, Wgt, bt = tt(x), tt(Wg), tt(bias)
    ext = [[tt(m) for m in trip] for trip in ex]
    sht = [tt(m) for m in sh]
    p = torch.softmax(xt @ Wgt + bt, dim=1)
    if ec:
        w = p * torch.from_numpy(mask)
        if renorm:
            w = w / w.sum(dim=1, keepdim=True).clamp_min(1e-300)
    else:
        pc = p * torch.from_numpy(chosen)
        w = (pc / pc.sum(dim=1, keepdim=True) if renorm else pc) * torch.from_numpy(mask)
    xq = ste(xt, oracle.mx_roundtrip)

    def ffn(a, b_, c):
        H = torch.nn.functional.silu(xq @ a) * (xq @ b_)
        return ste(H, _qh) @ c
    out = sum(w[:, e:e + 1] * ffn(*ext[e]) for e in range(E)) + ffn(*sht)
    (out * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(out.detach().numpy(), r["out"], rtol=1e-6, atol=1e-6)   # fp32 logits vs fp64
    tol = dict(rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(b["dx"], xt.grad.numpy(), **tol)
    np.testing.assert_allclose(b["dW_g"], Wgt.grad.numpy(), **tol)
    np.testing.assert_allclose(b["d_bias"], bt.grad.numpy(), **tol)
    for e in range(E):
        for key, m in (("dW_gate", 0), ("dW_up", 1), ("dW_down", 2)):
            np.testing.assert_allclose(b[key][e], ext[e][m].grad.numpy(), **tol)
    for key, m in (("dWs_gate", 0), ("dWs_up", 1), ("dWs_down", 2)):
        np.testing.assert_allclose(b[key], sht[m].grad.numpy(), **tol)
    # the quantisation is not the identity on these inputs
    assert np.abs(oracle.mx_roundtrip(x) - x).max() > 1e-3
