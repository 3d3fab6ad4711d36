"""Shared helpers of the GPU parity tests: seeded inputs on the device, the
same tensors widened exactly for the CPU oracle, and tolerance checks."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

# max|gpu - oracle| / max|oracle| bounds per weight type (fp32, bf16, fp8)
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "mxfp8": 6e-2, "mxfp4": 6e-2}


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def codes(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def unpack_e2m1(t: torch.Tensor) -> np.ndarray:
    """Two E2M1 codes per byte (element 2j in the low nibble) -> one per byte."""
    b = codes(t)
    return np.stack([b & 0x0F, b >> 4], axis=-1).reshape(*b.shape[:-1], 2 * b.shape[-1])


class OracleInputs:
    """The device inputs of one layer call, seen by the oracle (exact fp64)."""

    def __init__(self, inp: dict):
        self.inp = inp
        self.cfg = inp["cfg"]
        self.x = to64(inp["x"])
        self.W_g = to64(inp["W_g"])
        self.bias = None if inp["bias"] is None else to64(inp["bias"])

    def _triple(self, g, u, dn, sg, su, sd):
        if self.cfg.wdt == "mxfp8":         # output-major codes + block scales -> [in, out] values
            return tuple(oracle.mx_dequantize(codes(w), sc.cpu().numpy()).T for w, sc in ((g, sg), (u, su), (dn, sd)))
        if self.cfg.wdt == "mxfp4":
            return tuple(oracle.mx4_dequantize(unpack_e2m1(w), sc.cpu().numpy()).T
                         for w, sc in ((g, sg), (u, su), (dn, sd)))
        if self.cfg.wdt == "fp8":
            return (oracle.dequantize(codes(g), sg.cpu().numpy(), 1),
                    oracle.dequantize(codes(u), su.cpu().numpy(), 1),
                    oracle.dequantize(codes(dn), sd.cpu().numpy(), 1))
        return to64(g), to64(u), to64(dn)

    def expert(self, e: int):
        i = self.inp
        if self.cfg.wdt in ("mxfp8", "mxfp4"):
            return self._triple(i["W_gate"][e], i["W_up"][e], i["W_down"][e],
                                i["mx_gate"][e], i["mx_up"][e], i["mx_down"][e])
        if self.cfg.wdt == "fp8":
            return self._triple(i["W_gate"][e], i["W_up"][e], i["W_down"][e],
                                i["s_gate"][e], i["s_up"][e], i["s_down"][e])
        return self._triple(i["W_gate"][e], i["W_up"][e], i["W_down"][e], None, None, None)

    def shared(self):
        i = self.inp
        if not self.cfg.shared:
            return None
        if self.cfg.wdt in ("mxfp8", "mxfp4"):
            return self._triple(i["Ws_gate"], i["Ws_up"], i["Ws_down"], i["mxs_gate"], i["mxs_up"], i["mxs_down"])
        return self._triple(i["Ws_gate"], i["Ws_up"], i["Ws_down"], i["ss_gate"], i["ss_up"], i["ss_down"])

    def quant_hooks(self) -> dict:
        """Block-scaled layers (MXFP8 or MXFP4 weights): expert inputs and the
        fp32 SwiGLU activations are MXFP8-quantised before their products."""
        if self.cfg.wdt not in ("mxfp8", "mxfp4"):
            return {}
        return {"quant_x": oracle.mx_roundtrip, "quant_h": lambda H: oracle.mx_roundtrip(H, as_fp32=True)}

    def ffn(self, X, e=None):
        """One expert's (or, e None, the shared expert's) FFN of rows X."""
        h = self.quant_hooks()
        qx = h.get("quant_x")
        return oracle.expert_ffn(X if qx is None else qx(X), *(self.shared() if e is None else self.expert(e)),
                                 quant_h=h.get("quant_h"))

    def forward(self, tokens=None):
        c = self.cfg
        return oracle.forward(self.x, self.W_g, self.bias, c.k, c.renormalize, np.float32(c.capacity_factor),
                              self.expert, c.E, shared=self.shared(), tokens=tokens, **self.quant_hooks())

    def certificate(self):
        return oracle.routing_certificate(self.x, self.W_g, self.bias, self.cfg.k)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.abs(ref).max())
    return float(np.abs(got - ref).max()) / (den if den > 0 else 1.0)


def assert_close(got, ref, tol, what=""):
    e = rel_err(np.asarray(got, np.float64), np.asarray(ref, np.float64))
    assert e <= tol, f"{what}: max|gpu-oracle|/max|oracle| = {e:.3e} > {tol:.1e}"
    return e


def device_inputs(cfg: synth.MoEConfig, router_only=False) -> dict:
    print(f"[inputs] {cfg}", flush=True)
    return synth.make_inputs(cfg, "cuda", router_only=router_only)


def ec_boundary_is_clear(ref):
    """The C-th and (C+1)-th scores of every expert are distinct fp32 values whose
    fp64 sources are far (relatively 1e-12) from an fp32 rounding midpoint, so a
    different fp64 summation order cannot change any selection."""
    probs = oracle.softmax_rows(ref["logits"])
    s32 = ref["scores"]
    T, E = s32.shape
    Cap = ref["capacity"]
    if Cap >= T:
        return True
    for e in range(E):
        order = sorted(range(T), key=lambda t: (-float(s32[t, e]), t))
        for t in order[Cap - 1:Cap + 1]:
            p = probs[t, e]
            lo = np.float32(p)
            nb = np.nextafter(lo, np.float32(np.inf if p > lo else -np.inf))
            mid = (float(lo) + float(nb)) / 2.0
            if abs(p - mid) <= 1e-12 * abs(p):
                return False
    return True
