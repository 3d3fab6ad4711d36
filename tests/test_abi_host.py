"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol the header declares, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def ops():
    from sparse_mixture_experts_12_amd import _lib
    return _lib


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_header_symbol(ops):
    names = header_functions()
    assert set(names) == set(ops.EXPORTS)
    for n in names:
        assert hasattr(ops.LIB, n), n


def test_probe_library_exports_its_header_symbols():
    """libmoe_probe.so (the roofline probes bench.py --probe times) exports
    what include/moe_probe.h declares and rejects bad arguments before any
    launch."""
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "moe_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(probe_[a-z0-9_]+)\s*\(", src)))
    assert names == ["probe_hbm_read", "probe_mfma_bf16"]
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_mixture_experts_12_amd", "libmoe_probe.so"))
    for n in names:
        assert hasattr(lib, n), n
    lib.probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    invalid = 1   # hipErrorInvalidValue
    assert lib.probe_hbm_read(None, 1 << 20, None, 8, None) == invalid
    assert lib.probe_hbm_read(16, 100, 16, 8, None) == invalid          # not a multiple of 32 KB
    assert lib.probe_hbm_read(16, 1 << 20, 16, 0, None) == invalid
    assert lib.probe_mfma_bf16(16, 8, 3, 16, None) == invalid           # odd iteration count
    assert lib.probe_mfma_bf16(None, 8, 4, 16, None) == invalid


def test_capacity_matches_oracle(ops):
    for (T, k, E, cf) in [(512, 8, 128, 1.25), (1, 8, 128, 1.25), (64, 2, 8, 0.0), (10, 1, 4, 1.0),
                          (7, 3, 5, 0.01), (4096, 2, 8, 1.1)]:
        d = ops.make_desc(T, 64, E, k, 64, capacity_factor=cf)
        want = oracle.capacity(T, k, E, cf)
        assert ops.capacity(d) == (-1 if want is None else want), (T, k, E, cf)


@pytest.mark.parametrize("field,value,status", [
    ("d", 63, 1), ("f", 96, 1), ("E", 0, 1), ("E", 1024, 1), ("top_k", 0, 1), ("top_k", 9, 1),
    ("T", -1, 1), ("renormalize", 2, 1), ("capacity_factor", -1.0, 1), ("path", 3, 1),
    ("act_dtype", 2, 1), ("w_dtype", 7, 1)])
def test_desc_validation(ops, field, value, status):
    d = ops.make_desc(4, 64, 8, 2, 64)
    setattr(d, field, value)
    assert ops.workspace_size(d) == 0
    ws = ctypes.c_void_p(0)
    r = ops.LIB.moe_forward(ctypes.byref(d), None, None, None, None, ws, 0, None)
    assert r == status, ops.last_error()


def test_unsupported_pairs_and_paths(ops):
    d = ops.make_desc(4, 64, 8, 2, 64, act="f32", wdt="bf16")
    assert ops.LIB.moe_forward(ctypes.byref(d), None, None, None, None, None, 0, None) == ops.MOE_ERR_UNSUPPORTED
    d = ops.make_desc(9, 64, 8, 2, 64, path=ops.PATH_FUSED_DECODE)
    assert ops.LIB.moe_forward(ctypes.byref(d), None, None, None, None, None, 0, None) == ops.MOE_ERR_UNSUPPORTED
    assert "T <= 8" in ops.last_error()
    d = ops.make_desc(2, 64, 8, 2, 64, act="f32", wdt="f32", path=ops.PATH_FUSED_DECODE)
    assert ops.LIB.moe_forward(ctypes.byref(d), None, None, None, None, None, 0, None) == ops.MOE_ERR_UNSUPPORTED


def test_null_and_alignment_checks(ops):
    d = ops.make_desc(4, 64, 8, 2, 64)
    w = ops.Weights()
    # x NULL
    assert ops.LIB.moe_forward(ctypes.byref(d), None, ctypes.byref(w), 16, None, None, 0, None) == 1
    # misaligned x
    assert ops.LIB.moe_forward(ctypes.byref(d), 18, ctypes.byref(w), 16, None, None, 0, None) == 1
    assert "aligned" in ops.last_error()
    # W_g missing
    assert ops.LIB.moe_forward(ctypes.byref(d), 16, ctypes.byref(w), 16, None, None, 0, None) == 1
    assert "W_g" in ops.last_error()
    # fp8 without scales
    d8 = ops.make_desc(4, 64, 8, 2, 64, wdt="fp8")
    w8 = ops.Weights(W_g=16, W_gate=16, W_up=16, W_down=16)
    assert ops.LIB.moe_forward(ctypes.byref(d8), 16, ctypes.byref(w8), 16, None, None, 0, None) == 1
    assert "s_gate" in ops.last_error()
    # shared expert requested but missing
    ds = ops.make_desc(4, 64, 8, 2, 64, has_shared=True)
    ws_ = ops.Weights(W_g=16, W_gate=16, W_up=16, W_down=16)
    assert ops.LIB.moe_forward(ctypes.byref(ds), 16, ctypes.byref(ws_), 16, None, None, 0, None) == 1
    assert "Ws_gate" in ops.last_error()


def test_workspace_checks(ops):
    d = ops.make_desc(4, 64, 8, 2, 64)
    w = ops.Weights(W_g=16, W_gate=16, W_up=16, W_down=16)
    need = ops.workspace_size(d)
    assert need > 0
    assert ops.LIB.moe_forward(ctypes.byref(d), 16, ctypes.byref(w), 16, None, 256, need - 1, None) == 3
    assert ops.LIB.moe_forward(ctypes.byref(d), 16, ctypes.byref(w), 16, None, None, need, None) == 3
    assert ops.LIB.moe_forward(ctypes.byref(d), 16, ctypes.byref(w), 16, None, 16, need, None) == 1


def test_zero_tokens_is_a_noop(ops):
    d = ops.make_desc(0, 64, 8, 2, 64)
    st = ops.Stats()
    assert ops.LIB.moe_forward(ctypes.byref(d), None, None, None, ctypes.byref(st), None, 0, None) == 0
    for fn, args in (("moe_route", 8), ("moe_permute", 9), ("moe_grouped_ffn", 8)):
        f = getattr(ops.LIB, fn)
        a = [None] * args
        a[-2] = 0                     # workspace bytes
        assert f(ctypes.byref(d), *a) == 0
    assert ops.LIB.moe_combine(ctypes.byref(d), None, None, None, None, None) == 0


def test_workspace_grows_with_tokens(ops):
    sizes = [ops.workspace_size(ops.desc_from_cfg(synth.CONFIGS["fine_grained"], T=t)) for t in (1, 64, 2048)]
    assert sizes[0] < sizes[1] < sizes[2]


def test_oracle_and_library_are_independent():
    """The oracle imports nothing of the product, the product nothing of the oracle."""
    for dirpath, _, files in os.walk(os.path.join(ROOT, "oracle")):
        for fn in files:
            if fn.endswith(".py"):
                src = open(os.path.join(dirpath, fn)).read()
                assert "sparse_mixture_experts_12_amd" not in src and "synth" not in src, fn
    pkg = os.path.join(ROOT, "sparse_mixture_experts_12_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in src and "from oracle" not in src, fn


def test_expert_choice_validation(ops):
    EC = ops.ROUTING_EXPERT_CHOICE
    d = ops.make_desc(4, 64, 8, 2, 64)
    d.routing = 2
    assert ops.LIB.moe_forward(ctypes.byref(d), None, None, None, None, None, 0, None) == ops.MOE_ERR_INVALID_ARG
    d = ops.make_desc(8193, 64, 8, 2, 64)
    d.routing = EC
    assert ops.LIB.moe_forward(ctypes.byref(d), None, None, None, None, None, 0, None) == ops.MOE_ERR_UNSUPPORTED
    d = ops.make_desc(4, 64, 8, 2, 64, path=ops.PATH_FUSED_DECODE)
    d.routing = EC
    assert ops.LIB.moe_forward(ctypes.byref(d), None, None, None, None, None, 0, None) == ops.MOE_ERR_UNSUPPORTED
    d = ops.make_desc(40, 64, 8, 2, 64)
    d.routing = EC
    for call in (lambda: ops.LIB.moe_route(ctypes.byref(d), None, None, None, None, None, None, 0, None),
                 lambda: ops.LIB.moe_permute(ctypes.byref(d), None, None, None, None, None, None, None, 0, None),
                 lambda: ops.LIB.moe_combine(ctypes.byref(d), None, None, None, None, None)):
        assert call() == ops.MOE_ERR_UNSUPPORTED
        assert "moe_forward" in ops.last_error()


def test_expert_choice_capacity_and_workspace(ops):
    import oracle
    for T, k, E, cf in [(40, 2, 8, 0.0), (40, 2, 8, 1.25), (7, 1, 4, 0.01), (10, 2, 4, 100.0)]:
        d = ops.make_desc(T, 64, E, k, 64, capacity_factor=cf)
        d.routing = ops.ROUTING_EXPERT_CHOICE
        assert ops.LIB.moe_capacity(ctypes.byref(d)) == oracle.expert_choice_capacity(T, k, E, cf)
    tc = ops.make_desc(40, 64, 8, 2, 64, capacity_factor=4.0)
    ec = ops.make_desc(40, 64, 8, 2, 64, capacity_factor=4.0)
    ec.routing = ops.ROUTING_EXPERT_CHOICE                 # C = 40: every expert takes every token
    assert ops.LIB.moe_workspace_size(ctypes.byref(ec)) > ops.LIB.moe_workspace_size(ctypes.byref(tc))


@pytest.mark.parametrize("wdt", ["mxfp8", "mxfp4"])
def test_mx_validation(ops, wdt):
    def fwd(d):
        return ops.LIB.moe_forward(ctypes.byref(d), None, None, None, None, None, 0, None)
    d = ops.make_desc(40, 192, 8, 2, 256, wdt=wdt)           # d % 128 != 0
    assert fwd(d) == ops.MOE_ERR_UNSUPPORTED and "multiples of 128" in ops.last_error()
    d = ops.make_desc(4, 256, 8, 2, 256, wdt=wdt, path=ops.PATH_FUSED_DECODE)
    assert fwd(d) == ops.MOE_ERR_UNSUPPORTED and "grouped" in ops.last_error()
    d = ops.make_desc(4, 256, 8, 2, 256, act="f32", wdt=wdt)
    assert fwd(d) == ops.MOE_ERR_UNSUPPORTED
    d = ops.make_desc(1 << 20, 4096, 8, 2, 14336, wdt=wdt)   # 32-bit row offsets would overflow
    assert fwd(d) == ops.MOE_ERR_UNSUPPORTED and "2^31" in ops.last_error()
    # a valid MX descriptor sizes a workspace holding x and H codes + scales
    d = ops.make_desc(100, 256, 8, 2, 384, wdt=wdt)
    b = ops.make_desc(100, 256, 8, 2, 384, wdt="bf16")
    assert ops.workspace_size(d) > 0 and ops.workspace_size(b) > 0
    # weights without their block scales are rejected before any HIP call
    w = ops.Weights(W_g=16, W_gate=16, W_up=16, W_down=16)
    r = ops.LIB.moe_forward(ctypes.byref(d), ctypes.c_void_p(16), ctypes.byref(w), ctypes.c_void_p(16), None,
                            ctypes.c_void_p(256), 1 << 40, None)
    assert r == ops.MOE_ERR_INVALID_ARG and "mx_gate" in ops.last_error()


def test_mx_quantize_argument_checks(ops):
    q = ctypes.c_void_p(16)
    assert ops.LIB.moe_quantize_mxfp8(q, ops.MOE_BF16, 4, 48, q, q, None) == ops.MOE_ERR_INVALID_ARG
    assert ops.LIB.moe_quantize_mxfp8(q, ops.MOE_FP8_E4M3, 4, 64, q, q, None) == ops.MOE_ERR_INVALID_ARG
    assert ops.LIB.moe_quantize_mxfp8(q, ops.MOE_BF16, -1, 64, q, q, None) == ops.MOE_ERR_INVALID_ARG
    assert ops.LIB.moe_quantize_mxfp8(None, ops.MOE_BF16, 0, 64, None, None, None) == ops.MOE_OK
    assert ops.LIB.moe_quantize_mxfp8(None, ops.MOE_BF16, 3, 64, q, q, None) == ops.MOE_ERR_INVALID_ARG


def test_synth_mx_weights_follow_the_oracle_quantiser():
    """The input recipe's weight quantiser (torch) and the oracle's (numpy)
    are separate implementations of the same OCP rule; they must agree."""
    import numpy as np
    import torch
    rng = np.random.default_rng(5)
    w = (rng.normal(0, 0.02, (64, 256)) * np.exp2(rng.integers(-8, 8, (64, 1)))).astype(np.float32)
    w[3, :32] = 0.0
    q, s = synth.quantize_mxfp8_rows(torch.from_numpy(w))
    rq, rs = oracle.mx_quantize(w.astype(np.float64))
    np.testing.assert_array_equal(s.numpy(), rs)
    np.testing.assert_array_equal(q.view(torch.uint8).numpy(), rq)


def test_synth_mxfp4_weights_follow_the_oracle_quantiser():
    """MXFP4: the recipe's torch quantiser (packed two codes per byte, the
    even element in the low nibble) against the oracle's numpy one."""
    import numpy as np
    import torch
    rng = np.random.default_rng(6)
    w = (rng.normal(0, 0.02, (64, 256)) * np.exp2(rng.integers(-8, 8, (64, 1)))).astype(np.float32)
    w[3, :32] = 0.0
    w[5, :64] = (rng.integers(-28, 28, 64) / 4.0).astype(np.float32)   # exact midpoints
    w[6, :32] = -1e-30                                                 # rounds to -0
    q, s = synth.quantize_mxfp4_rows(torch.from_numpy(w))
    rq, rs = oracle.mx4_quantize(w.astype(np.float64))
    qn = q.numpy()
    assert qn.shape == (64, 128) and s.shape == (64, 8)
    np.testing.assert_array_equal(s.numpy(), rs)
    np.testing.assert_array_equal(np.stack([qn & 15, qn >> 4], axis=-1).reshape(64, 256), rq)


def test_backward_validation(ops):
    def bwd(d, g=None):
        gs = g if g is not None else ops.Grads()
        return ops.LIB.moe_backward(ctypes.byref(d), None, None, None, ctypes.byref(gs), None, 0, None)
    d = ops.make_desc(40, 256, 8, 2, 256, act="bf16", wdt="f32")       # not a layer dtype pair
    assert bwd(d) != ops.MOE_OK and ops.backward_workspace_size(d) == 0
    # block-scaled weights: taken; the workspace adds the bf16 weight values and the quantised x and H
    for wdt in ("mxfp8", "mxfp4"):
        dm = ops.make_desc(40, 256, 8, 2, 256, wdt=wdt)
        assert bwd(dm) == ops.MOE_ERR_INVALID_ARG and "dW_g" in ops.last_error(), wdt
        assert ops.backward_workspace_size(dm) > ops.backward_workspace_size(ops.make_desc(40, 256, 8, 2, 256))
    # fp32 layers: taken; gathered rows and SwiGLU-backward outputs are fp32
    d32 = ops.make_desc(40, 256, 8, 2, 256, act="f32", wdt="f32")
    assert bwd(d32) == ops.MOE_ERR_INVALID_ARG and "dW_g" in ops.last_error()
    assert ops.backward_workspace_size(d32) > ops.backward_workspace_size(ops.make_desc(40, 256, 8, 2, 256))
    # fp8 weights: taken; the workspace adds the bf16 weight values (3 E d f + 3 d f with the shared expert)
    d8 = ops.make_desc(40, 256, 8, 2, 256, wdt="fp8", has_shared=True)
    db = ops.make_desc(40, 256, 8, 2, 256, has_shared=True)
    assert bwd(d8) == ops.MOE_ERR_INVALID_ARG and "dW_g" in ops.last_error()
    assert ops.backward_workspace_size(d8) >= ops.backward_workspace_size(db) + 2 * (3 * 8 + 3) * 256 * 256
    # expert choice: bf16 layers are taken; the padded row space holds E C rows
    d = ops.make_desc(40, 256, 8, 2, 256)
    d.routing = ops.ROUTING_EXPERT_CHOICE
    assert bwd(d) == ops.MOE_ERR_INVALID_ARG and "dW_g" in ops.last_error()
    tc = ops.make_desc(40, 256, 8, 2, 256, capacity_factor=4.0)
    ec = ops.make_desc(40, 256, 8, 2, 256, capacity_factor=4.0)       # C = T = 40: 320 rows, T k = 80
    ec.routing = ops.ROUTING_EXPERT_CHOICE
    assert ops.backward_workspace_size(ec) > ops.backward_workspace_size(tc) > 0
    ecm = ops.make_desc(40, 256, 8, 2, 256, wdt="mxfp8")
    ecm.routing = ops.ROUTING_EXPERT_CHOICE
    assert ops.backward_workspace_size(ecm) > 0
    d = ops.make_desc(40, 256, 8, 2, 256)
    assert ops.backward_workspace_size(d) > ops.workspace_size(d)
    assert bwd(d) == ops.MOE_ERR_INVALID_ARG and "dW_g" in ops.last_error()
    r = ops.LIB.moe_backward(ctypes.byref(d), None, None, None, None, None, 0, None)
    assert r == ops.MOE_ERR_INVALID_ARG and "grads" in ops.last_error()
    g = ops.Grads(dW_g=16, dW_gate=16, dW_up=16, dW_down=16)
    d = ops.make_desc(40, 256, 8, 2, 256, has_shared=True)
    w = ops.Weights(W_g=16, W_gate=16, W_up=16, W_down=16)
    r = ops.LIB.moe_backward(ctypes.byref(d), None, ctypes.byref(w), None, ctypes.byref(g), None, 0, None)
    assert r == ops.MOE_ERR_INVALID_ARG and "dWs_gate" in ops.last_error()


def test_noalloc_declines_before_any_hip_call(ops):
    """The allocation-free forward validates the descriptor and its scratch
    need on the host first: a layer larger than the library's array is
    declined with no device work (this runs without a GPU)."""
    import ctypes
    big = ops.make_desc(4096, 4096, 8, 2, 14336)
    assert ops.workspace_size(big) > ops.NOALLOC_SCRATCH_BYTES
    st = ops.LIB.moe_forward_noalloc(ctypes.byref(big), None, None, None, None, None)
    assert st == ops.MOE_ERR_UNSUPPORTED
    assert "scratch" in ops.last_error()
    bad = ops.make_desc(4, 100, 8, 2, 64)                 # d not a multiple of 64
    assert ops.LIB.moe_forward_noalloc(ctypes.byref(bad), None, None, None, None, None) == ops.MOE_ERR_INVALID_ARG
