"""Seeded synthetic inputs for the routed MoE SwiGLU feed-forward layer.

This module only draws random tensors and stores them in the types the layer
consumes (fp32, bf16, or OCP fp8 e4m3fn codes with per-output-channel fp32
scale factors).  It holds none of the layer's arithmetic: the CPU oracle (fed
by the tests) and the HIP library both receive exactly the tensors returned
here, so the two sides never share code beyond this input recipe.

Recipe (every tensor has its own seed derived from the config seed, the tensor
name and the expert id, so one expert can be regenerated on its own):
  x        ~ N(0, 1)     drawn in fp32, then stored in the activation dtype
  W_g      ~ N(0, 0.02)  router weight [d, E], activation dtype
  experts  ~ N(0, 0.02)  W_gate/W_up [E, d, f], W_down [E, f, d]
  bias     optional per-expert router bias, b[e] = -s * ln(e + 1) (Zipf rank
           weights in log space), fp32
  fp8      per output channel c: s[c] = max|w[:, c]| / 448, q = RNE(w / s)
           as float8_e4m3fn (the largest finite e4m3fn value is 448).
  mxfp8    OCP Microscaling weights, stored output-major (W_gate, W_up
           [E, f, d], W_down [E, d, f]) with one E8M0 scale byte per 32
           consecutive input-dimension values (mx_gate, mx_up [E, f, d/32],
           mx_down [E, d, f/32]): s = floor(log2 max|block|) - 8 clamped to
           [-127, 127], q = RNE(w / 2^s) clamped to +-448 as float8_e4m3fn,
           byte = s + 127.  The layer receives these codes as given.
  mxfp4    the same layout and scale bytes with E2M1 elements, two per byte
           (element 2j in the low nibble): s = floor(log2 max|block|) - 2,
           q = RNE(w / 2^s) to {0, 0.5, 1, 1.5, 2, 3, 4, 6} with sign, |q| <= 6.
"""
from __future__ import annotations

import dataclasses
import hashlib
from dataclasses import dataclass
from typing import Optional

import torch

FP8_MAX = 448.0


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    act: str = "bf16"          # activation / router dtype: "f32" | "bf16"
    wdt: str = "bf16"          # expert weight dtype: "f32" | "bf16" | "fp8" | "mxfp8" | "mxfp4"
    renormalize: bool = True
    capacity_factor: float = 0.0   # 0 => uncapped
    shared: bool = False       # one always-on shared expert (same f)
    bias: str = "none"         # "none" | "zipf"
    zipf_s: float = 1.1
    seed: int = 0
    x_std: float = 1.0
    w_std: float = 0.02

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    @property
    def n_assign(self) -> int:
        return self.T * self.k


# The five workloads (sizes from the pages' model shapes: Mixtral 8x7B
# hidden 4096 / intermediate 14336 / 8 experts / top-2; a fine-grained
# DeepSeek-style layer with shared expert; an fp8 layer with capacity).
CONFIGS = {
    "tiny_f32": MoEConfig("tiny_f32", T=64, d=256, E=8, k=2, f=512, act="f32", wdt="f32"),
    "mixtral_decode": MoEConfig("mixtral_decode", T=1, d=4096, E=8, k=2, f=14336),
    "mixtral_decode_b8": MoEConfig("mixtral_decode_b8", T=8, d=4096, E=8, k=2, f=14336),
    "mixtral_prefill": MoEConfig("mixtral_prefill", T=4096, d=4096, E=8, k=2, f=14336),
    "fine_grained": MoEConfig("fine_grained", T=2048, d=7168, E=256, k=8, f=2048,
                              shared=True, bias="zipf"),
    "fp8_capacity": MoEConfig("fp8_capacity", T=512, d=2048, E=128, k=8, f=768,
                              wdt="fp8", capacity_factor=1.25),
    "fp8_capacity_decode": MoEConfig("fp8_capacity_decode", T=1, d=2048, E=128, k=8, f=768,
                                     wdt="fp8", capacity_factor=1.25),
    # block-scaled (MXFP8) variants of the two prefill-shaped layers
    "mixtral_prefill_mxfp8": MoEConfig("mixtral_prefill_mxfp8", T=4096, d=4096, E=8, k=2, f=14336,
                                       wdt="mxfp8"),
    "fine_grained_mxfp8": MoEConfig("fine_grained_mxfp8", T=2048, d=7168, E=256, k=8, f=2048,
                                    wdt="mxfp8", shared=True, bias="zipf"),
    # MXFP4 weights (E2M1 codes, two per byte) with MXFP8 activations
    "mixtral_prefill_mxfp4": MoEConfig("mixtral_prefill_mxfp4", T=4096, d=4096, E=8, k=2, f=14336,
                                       wdt="mxfp4"),
    "fine_grained_mxfp4": MoEConfig("fine_grained_mxfp4", T=2048, d=7168, E=256, k=8, f=2048,
                                    wdt="mxfp4", shared=True, bias="zipf"),
}


def tensor_seed(seed: int, name: str, expert: int = -1) -> int:
    h = hashlib.sha256(f"{seed}/{name}/{expert}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _normal(shape, std, seed, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def _store(t32: torch.Tensor, dt: str) -> torch.Tensor:
    if dt == "f32":
        return t32
    if dt == "bf16":
        return t32.to(torch.bfloat16)
    raise ValueError(dt)


def quantize_fp8_per_channel(w32: torch.Tensor, channel_dim: int):
    """w32 fp32 -> (q float8_e4m3fn, s fp32 per channel along channel_dim)."""
    red = [i for i in range(w32.dim()) if i != channel_dim]
    amax = w32.abs().amax(dim=red)
    s = torch.clamp(amax, min=1e-30) / FP8_MAX
    shape = [1] * w32.dim()
    shape[channel_dim] = -1
    q = torch.clamp(w32 / s.view(shape), -FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q, s.to(torch.float32)


def quantize_mxfp8_rows(w32: torch.Tensor):
    """w32 fp32 [..., K], K % 32 == 0 -> (codes float8_e4m3fn [..., K],
    scales uint8 [..., K / 32]), blocks of 32 along the last axis."""
    K = w32.shape[-1]
    b = w32.reshape(*w32.shape[:-1], K // 32, 32)
    amax = b.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                       # amax = m 2^ex, m in [0.5, 1)
    s = torch.where(amax > 0, ex - 9, torch.full_like(ex, -127)).clamp(-127, 127)
    q = torch.clamp(torch.ldexp(b, (-s).unsqueeze(-1).to(b.dtype)), -FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return q.reshape(w32.shape), (s + 127).to(torch.uint8)


_E2M1_MIDS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]   # midpoints of 0, .5, 1, 1.5, 2, 3, 4, 6


def quantize_mxfp4_rows(w32: torch.Tensor):
    """w32 fp32 [..., K], K % 32 == 0 -> (codes uint8 [..., K / 2], two E2M1
    codes per byte, element 2 j in the low nibble and 2 j + 1 in the high
    one; scales uint8 [..., K / 32]), blocks of 32 along the last axis:
    s = floor(log2 max|block|) - 2, elements rounded to the nearest E2M1
    value (ties to the even code, magnitudes above 6 saturated)."""
    K = w32.shape[-1]
    b = w32.reshape(*w32.shape[:-1], K // 32, 32)
    amax = b.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)                       # amax = m 2^ex, m in [0.5, 1)
    s = torch.where(amax > 0, ex - 3, torch.full_like(ex, -127)).clamp(-127, 127)
    y = torch.ldexp(b, (-s).unsqueeze(-1).to(b.dtype))
    a = y.abs().clamp(max=6.0)
    mids = torch.tensor(_E2M1_MIDS, dtype=a.dtype, device=a.device)
    code = torch.bucketize(a, mids)                 # mids[i - 1] < a <= mids[i] -> i
    at_mid = (code < 7) & (a == mids[code.clamp(max=6)])
    code = torch.where(at_mid & (code % 2 == 1), code + 1, code)   # a tie goes to the even code
    code = code | torch.where(torch.signbit(y), 8, 0)
    code = code.to(torch.uint8).reshape(*w32.shape[:-1], K)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), (s + 127).to(torch.uint8)


def _expert_mats(cfg: MoEConfig, tag: str, e: int, device):
    wg = _normal((cfg.d, cfg.f), cfg.w_std, tensor_seed(cfg.seed, tag + "gate", e), device)
    wu = _normal((cfg.d, cfg.f), cfg.w_std, tensor_seed(cfg.seed, tag + "up", e), device)
    wd = _normal((cfg.f, cfg.d), cfg.w_std, tensor_seed(cfg.seed, tag + "down", e), device)
    return wg, wu, wd


def router_bias(cfg: MoEConfig, device="cpu") -> Optional[torch.Tensor]:
    if cfg.bias == "none":
        return None
    if cfg.bias == "zipf":
        r = torch.arange(cfg.E, dtype=torch.float64)
        return (-cfg.zipf_s * torch.log1p(r)).to(torch.float32).to(device)
    raise ValueError(cfg.bias)


def make_inputs(cfg: MoEConfig, device="cpu", router_only: bool = False) -> dict:
    """All tensors of one layer call, on `device` (contiguous, row-major).

    keys: x [T,d]; W_g [d,E]; bias [E] | None; W_gate, W_up [E,d,f];
    W_down [E,f,d]; s_gate, s_up [E,f], s_down [E,d] (fp8 only, else None);
    Ws_gate, Ws_up [d,f], Ws_down [f,d] (+ ss_gate, ss_up, ss_down for fp8)
    when cfg.shared, else None.
    """
    dev = torch.device(device)
    out = {"cfg": cfg}
    out["x"] = _store(_normal((cfg.T, cfg.d), cfg.x_std, tensor_seed(cfg.seed, "x"), dev), cfg.act)
    out["W_g"] = _store(_normal((cfg.d, cfg.E), cfg.w_std, tensor_seed(cfg.seed, "router"), dev), cfg.act)
    out["bias"] = router_bias(cfg, dev)
    if router_only:
        return out

    def alloc(shape):
        dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn,
              "mxfp8": torch.float8_e4m3fn}[cfg.wdt]
        return torch.empty(shape, dtype=dt, device=dev)

    E, d, f = cfg.E, cfg.d, cfg.f
    if cfg.wdt in ("mxfp8", "mxfp4"):
        return _make_mx_weights(cfg, dev, out)
    Wg, Wu, Wd = alloc((E, d, f)), alloc((E, d, f)), alloc((E, f, d))
    fp8 = cfg.wdt == "fp8"
    if fp8:
        sg = torch.empty((E, f), dtype=torch.float32, device=dev)
        su = torch.empty((E, f), dtype=torch.float32, device=dev)
        sd = torch.empty((E, d), dtype=torch.float32, device=dev)
    for e in range(E):
        wg, wu, wd = _expert_mats(cfg, "", e, dev)
        if fp8:
            Wg[e], sg[e] = quantize_fp8_per_channel(wg, 1)
            Wu[e], su[e] = quantize_fp8_per_channel(wu, 1)
            Wd[e], sd[e] = quantize_fp8_per_channel(wd, 1)
        else:
            Wg[e], Wu[e], Wd[e] = _store(wg, cfg.wdt), _store(wu, cfg.wdt), _store(wd, cfg.wdt)
        del wg, wu, wd
    out.update(W_gate=Wg, W_up=Wu, W_down=Wd)
    out.update(s_gate=sg if fp8 else None, s_up=su if fp8 else None, s_down=sd if fp8 else None)

    out.update(Ws_gate=None, Ws_up=None, Ws_down=None, ss_gate=None, ss_up=None, ss_down=None)
    if cfg.shared:
        wg, wu, wd = _expert_mats(cfg, "shared_", 0, dev)
        if fp8:
            out["Ws_gate"], out["ss_gate"] = quantize_fp8_per_channel(wg, 1)
            out["Ws_up"], out["ss_up"] = quantize_fp8_per_channel(wu, 1)
            out["Ws_down"], out["ss_down"] = quantize_fp8_per_channel(wd, 1)
        else:
            out["Ws_gate"], out["Ws_up"], out["Ws_down"] = (
                _store(wg, cfg.wdt), _store(wu, cfg.wdt), _store(wd, cfg.wdt))
    return out


def _make_mx_weights(cfg: MoEConfig, dev, out: dict) -> dict:
    """MXFP8 codes [E, N, K] (float8_e4m3fn) or MXFP4 codes [E, N, K / 2]
    (uint8, two per byte), output-major, with scales [E, N, K / 32]."""
    E, d, f = cfg.E, cfg.d, cfg.f
    fp4 = cfg.wdt == "mxfp4"
    quant = quantize_mxfp4_rows if fp4 else quantize_mxfp8_rows
    if fp4:
        q8 = lambda *shape: torch.empty(shape[:-1] + (shape[-1] // 2,), dtype=torch.uint8, device=dev)
    else:
        q8 = lambda *shape: torch.empty(shape, dtype=torch.float8_e4m3fn, device=dev)
    u8 = lambda *shape: torch.empty(shape, dtype=torch.uint8, device=dev)
    Wg, Wu, Wd = q8(E, f, d), q8(E, f, d), q8(E, d, f)
    sg, su, sd = u8(E, f, d // 32), u8(E, f, d // 32), u8(E, d, f // 32)
    for e in range(E):
        wg, wu, wd = _expert_mats(cfg, "", e, dev)
        Wg[e], sg[e] = quant(wg.t().contiguous())
        Wu[e], su[e] = quant(wu.t().contiguous())
        Wd[e], sd[e] = quant(wd.t().contiguous())
        del wg, wu, wd
    out.update(W_gate=Wg, W_up=Wu, W_down=Wd, mx_gate=sg, mx_up=su, mx_down=sd,
               s_gate=None, s_up=None, s_down=None)
    out.update(Ws_gate=None, Ws_up=None, Ws_down=None, ss_gate=None, ss_up=None, ss_down=None,
               mxs_gate=None, mxs_up=None, mxs_down=None)
    if cfg.shared:
        wg, wu, wd = _expert_mats(cfg, "shared_", 0, dev)
        out["Ws_gate"], out["mxs_gate"] = quant(wg.t().contiguous())
        out["Ws_up"], out["mxs_up"] = quant(wu.t().contiguous())
        out["Ws_down"], out["mxs_down"] = quant(wd.t().contiguous())
    return out


def weight_bytes_per_expert(cfg: MoEConfig) -> int:
    if cfg.wdt == "mxfp4":
        return 3 * cfg.d * cfg.f // 2 + 3 * cfg.d * cfg.f // 32
    es = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp8": 1}[cfg.wdt]
    b = 3 * cfg.d * cfg.f * es
    if cfg.wdt == "fp8":
        b += (2 * cfg.f + cfg.d) * 4
    if cfg.wdt == "mxfp8":
        b += 3 * cfg.d * cfg.f // 32
    return b
