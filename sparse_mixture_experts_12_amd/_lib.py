"""ctypes binding of libmoe.so (the gfx950 MoE layer library).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the layer runs in the library's kernels.  If the
library is missing, importing this module raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_LIB", os.path.join(_PKG, "libmoe.so"))

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_MXFP8, MOE_MXFP4 = range(5)
PATH_AUTO, PATH_GROUPED, PATH_FUSED_DECODE = range(3)
ROUTING_TOKEN_CHOICE, ROUTING_EXPERT_CHOICE = range(2)
_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "mxfp8": MOE_MXFP8, "mxfp4": MOE_MXFP4}

# Every symbol the header declares.
EXPORTS = ("moe_workspace_size", "moe_capacity", "moe_route", "moe_permute", "moe_grouped_ffn",
           "moe_combine", "moe_forward", "moe_forward_noalloc", "moe_quantize_mxfp8", "moe_backward_workspace_size", "moe_backward",
           "moe_status_string", "moe_last_error")


class Desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("f", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("capacity_factor", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("w_dtype", ctypes.c_int32), ("has_shared", ctypes.c_int32), ("path", ctypes.c_int32),
                ("routing", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "W_g", "router_bias", "W_gate", "W_up", "W_down", "s_gate", "s_up", "s_down",
        "Ws_gate", "Ws_up", "Ws_down", "ss_gate", "ss_up", "ss_down",
        "mx_gate", "mx_up", "mx_down", "mxs_gate", "mxs_up", "mxs_down")]


class Stats(ctypes.Structure):
    _fields_ = [("path_taken", ctypes.c_int32), ("d_n_dropped", ctypes.c_void_p),
                ("d_counts", ctypes.c_void_p), ("ev_begin", ctypes.c_void_p), ("ev_end", ctypes.c_void_p),
                ("d_routed", ctypes.c_void_p), ("d_prob_mean", ctypes.c_void_p), ("d_lb_loss", ctypes.c_void_p)]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "dx", "dW_g", "d_bias", "dW_gate", "dW_up", "dW_down", "dWs_gate", "dWs_up", "dWs_down",
        "ev_begin", "ev_end")]


class MoEError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {status_string(status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "or python sparse_mixture_experts_12_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    DP, WP, SP = ctypes.POINTER(Desc), ctypes.POINTER(Weights), ctypes.POINTER(Stats)
    sig = {
        "moe_workspace_size": (S, [DP]),
        "moe_capacity": (ctypes.c_int32, [DP]),
        "moe_route": (ctypes.c_int, [DP, P, WP, P, P, P, P, S, P]),
        "moe_permute": (ctypes.c_int, [DP, P, P, P, P, P, P, P, S, P]),
        "moe_grouped_ffn": (ctypes.c_int, [DP, P, WP, P, P, P, P, S, P]),
        "moe_combine": (ctypes.c_int, [DP, P, P, P, P, P]),
        "moe_forward": (ctypes.c_int, [DP, P, WP, P, SP, P, S, P]),
        "moe_forward_noalloc": (ctypes.c_int, [DP, P, WP, P, SP, P]),
        "moe_quantize_mxfp8": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, P, P, P]),
        "moe_backward_workspace_size": (S, [DP]),
        "moe_backward": (ctypes.c_int, [DP, P, WP, P, ctypes.POINTER(Grads), P, S, P]),
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    return lib


LIB = _load()


def status_string(s: int) -> str:
    return LIB.moe_status_string(s).decode()


def last_error() -> str:
    return LIB.moe_last_error().decode()


def _check(status: int, fn: str):
    if status != MOE_OK:
        raise MoEError(status, fn, last_error())


def make_desc(T, d, E, top_k, f, act="bf16", wdt="bf16", renormalize=True, capacity_factor=0.0,
              has_shared=False, path=PATH_AUTO) -> Desc:
    return Desc(T, d, E, top_k, f, int(bool(renormalize)), float(capacity_factor), _DT[act], _DT[wdt],
                int(bool(has_shared)), int(path))


def desc_from_cfg(cfg, path=PATH_AUTO, T=None, routing=ROUTING_TOKEN_CHOICE) -> Desc:
    d = make_desc(cfg.T if T is None else T, cfg.d, cfg.E, cfg.k, cfg.f, cfg.act, cfg.wdt,
                  cfg.renormalize, cfg.capacity_factor, cfg.shared, path)
    d.routing = routing
    return d


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def weights_struct(inp: dict) -> Weights:
    """inp: a dict with the keys of synth.make_inputs (device tensors)."""
    return Weights(*[_ptr(inp.get(n)) for n in (
        "W_g", "bias", "W_gate", "W_up", "W_down", "s_gate", "s_up", "s_down",
        "Ws_gate", "Ws_up", "Ws_down", "ss_gate", "ss_up", "ss_down",
        "mx_gate", "mx_up", "mx_down", "mxs_gate", "mxs_up", "mxs_down")])


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def workspace_size(desc: Desc) -> int:
    return int(LIB.moe_workspace_size(ctypes.byref(desc)))


def capacity(desc: Desc) -> int:
    return int(LIB.moe_capacity(ctypes.byref(desc)))


def alloc_workspace(desc: Desc, device="cuda") -> torch.Tensor:
    n = workspace_size(desc)
    if n == 0:
        raise MoEError(MOE_ERR_INVALID_ARG, "moe_workspace_size", last_error())
    return torch.empty(n, dtype=torch.uint8, device=device)


def route(desc, x, weights: Weights, topk_idx, topk_w, logits=None, ws=None, stream=None):
    _check(LIB.moe_route(ctypes.byref(desc), _ptr(x), ctypes.byref(weights), _ptr(topk_idx), _ptr(topk_w),
                         _ptr(logits), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)), "moe_route")


def permute(desc, topk_idx, counts, offsets, sorted_assign, inv_perm, n_dropped, ws, stream=None):
    _check(LIB.moe_permute(ctypes.byref(desc), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(sorted_assign),
                           _ptr(inv_perm), _ptr(n_dropped), _ptr(ws), ws.numel(), _stream(stream)), "moe_permute")


def grouped_ffn(desc, x, weights: Weights, sorted_assign, offsets, y_sorted, ws, stream=None):
    _check(LIB.moe_grouped_ffn(ctypes.byref(desc), _ptr(x), ctypes.byref(weights), _ptr(sorted_assign),
                               _ptr(offsets), _ptr(y_sorted), _ptr(ws), ws.numel(), _stream(stream)),
           "moe_grouped_ffn")


def combine(desc, y_sorted, inv_perm, topk_w, out, stream=None):
    _check(LIB.moe_combine(ctypes.byref(desc), _ptr(y_sorted), _ptr(inv_perm), _ptr(topk_w), _ptr(out),
                           _stream(stream)), "moe_combine")


@dataclass
class ForwardStats:
    path_taken: int


def forward(desc, x, weights: Weights, out, ws, stats: Stats | None = None, stream=None) -> int:
    st = stats if stats is not None else Stats()
    _check(LIB.moe_forward(ctypes.byref(desc), _ptr(x), ctypes.byref(weights), _ptr(out), ctypes.byref(st),
                           _ptr(ws), ws.numel(), _stream(stream)), "moe_forward")
    return st.path_taken


NOALLOC_SCRATCH_BYTES = 128 << 20      # MOE_NOALLOC_SCRATCH_BYTES


def forward_noalloc(desc, x, weights: Weights, out, stats: Stats | None = None, stream=None) -> int:
    """moe_forward_noalloc: the whole layer with the library's own per-GPU scratch."""
    st = stats if stats is not None else Stats()
    _check(LIB.moe_forward_noalloc(ctypes.byref(desc), _ptr(x), ctypes.byref(weights), _ptr(out),
                                   ctypes.byref(st), _stream(stream)), "moe_forward_noalloc")
    return st.path_taken


def quantize_mxfp8(x, codes, scales, stream=None):
    """x: [rows, cols] f32 or bf16 device tensor -> codes [rows, cols] and
    scales [rows, cols / 32] (uint8 device tensors)."""
    dt = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16}[x.dtype]
    rows = x.numel() // x.shape[-1] if x.dim() else 0
    _check(LIB.moe_quantize_mxfp8(_ptr(x), dt, rows, x.shape[-1], _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_mxfp8")


def backward_workspace_size(desc: Desc) -> int:
    return int(LIB.moe_backward_workspace_size(ctypes.byref(desc)))


def alloc_backward_workspace(desc: Desc, device="cuda") -> torch.Tensor:
    n = backward_workspace_size(desc)
    if n == 0:
        raise MoEError(MOE_ERR_UNSUPPORTED, "moe_backward_workspace_size", last_error())
    return torch.empty(n, dtype=torch.uint8, device=device)


def grads_struct(g: dict, ev_begin=None, ev_end=None) -> Grads:
    """g: dict with the keys of Grads (device fp32 tensors or None)."""
    return Grads(*[_ptr(g.get(n)) for n in ("dx", "dW_g", "d_bias", "dW_gate", "dW_up", "dW_down",
                                             "dWs_gate", "dWs_up", "dWs_down")], ev_begin, ev_end)


def backward(desc, x, weights: Weights, dout, grads: Grads, ws, stream=None):
    _check(LIB.moe_backward(ctypes.byref(desc), _ptr(x), ctypes.byref(weights), _ptr(dout), ctypes.byref(grads),
                            _ptr(ws), ws.numel(), _stream(stream)), "moe_backward")
