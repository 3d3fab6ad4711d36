#!/usr/bin/env python3
"""Throughput of the routed MoE SwiGLU layer forward on one MI355X.

One step = one whole layer call (router -> top-k -> dispatch -> expert SwiGLU
FFN -> weighted combine) on seeded synthetic inputs already resident in HBM.
The default workload is the Mixtral-shaped single-token decode (T=1, d=4096,
E=8, top-2, f=14336, bf16).  Expert weights rotate over several copies so that
every step streams them from HBM, not from the 256 MB last-level cache.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (timed
live with HIP events on the layer's stream around every launch of it), and
the CPU oracle timed on a bounded sample on this host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0        # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
FP8_PEAK_TFLOPS = 5000.0         # dense fp8 MFMA (also the MXFP8 scaled MFMA)
LLC_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", default="mixtral_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="skip the second timed region (per-launch events on the dominant kernel)")
    ap.add_argument("--routing", choices=["token", "expert"], default="token",
                    help="token choice (the pages' default) or expert choice (every expert takes its C best tokens)")
    ap.add_argument("--backward", action="store_true",
                    help="time moe_backward (dL/dx and every weight gradient for a random dout) instead "
                         "of the forward; every layer dtype, either routing")
    ap.add_argument("--telemetry", action="store_true",
                    help="also request the router telemetry outputs (routed load, mean probability, "
                         "load-balancing loss) inside the timed region")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the region that replays the layer from a captured HIP graph")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --workload (a default run also times the other seeded workloads and reports "
                         "them under the \"workloads\" key)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain device copy of known size (for HBM counter scaling)")
    ap.add_argument("--probe", action="store_true",
                    help="instead of the layer, time the roofline probes (libmoe_probe.so): a pure HBM read stream "
                         "and back-to-back bf16 MFMAs on register operands (random and zero data), the ceilings "
                         "this part sustains")
    ap.add_argument("--library-gemm", action="store_true",
                    help="instead of the layer, time torch.mm (hipBLASLt) on the workload's per-expert gate/up "
                         "and down GEMM shapes with balanced routing: the vendor library's rate on this part, "
                         "for the MFMA roofline's context")
    return ap.parse_args()


class HipEvents:
    """Raw hipEvent_t handles (the library records them on its own stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value


def algorithmic_work(cfg, counts, touched):
    """Bytes and flops the layer must move/do for this routing (per call)."""
    import synth
    es = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp8": 1, "mxfp4": 0.5}[cfg.wdt]
    ae = 4 if cfg.act == "f32" else 2
    wexp = synth.weight_bytes_per_expert(cfg)
    n_exp = touched + (1 if cfg.shared else 0)
    bytes_total = cfg.T * cfg.d * ae + cfg.d * cfg.E * ae + n_exp * wexp + cfg.T * cfg.d * ae
    rows = int(sum(counts)) + (cfg.T if cfg.shared else 0)
    flops = 2 * cfg.T * cfg.d * cfg.E + 6 * rows * cfg.d * cfg.f
    return bytes_total, flops, n_exp * wexp, es


def split_decode(cfg) -> bool:
    """Whether the decode path runs row-split (gate/up and down in two kernels):
    the fused kernel would get fewer than 200 work-groups of 64 columns."""
    units = min(cfg.T * cfg.k, cfg.E) + (1 if cfg.shared else 0)
    return units * (cfg.f // 64) < 200


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the
    kernel's sources are unchanged since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}__{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for src in kv["source_files"].split(","):
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != kv["source_sha256"]:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def cpu_baseline(cfg, inp, budget_s=12.0, max_calls=2000):
    """The CPU oracle, as it stands, on single-token (decode) or small-batch calls."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    import torch
    to64 = lambda t: t.detach().to(torch.float64).cpu().numpy()
    x = to64(inp["x"])
    W_g = to64(inp["W_g"])
    bias = None if inp["bias"] is None else to64(inp["bias"])
    cache = {}

    cd = lambda t: t.contiguous().view(torch.uint8).cpu().numpy()
    mx = cfg.wdt in ("mxfp8", "mxfp4")

    def mx_codes(w):                          # MXFP4: two E2M1 codes per byte, element 2j low
        b = cd(w)
        if cfg.wdt != "mxfp4":
            return b
        return np.stack([b & 0x0F, b >> 4], axis=-1).reshape(*b.shape[:-1], 2 * b.shape[-1])

    def mx_triple(g, u, dn, sg, su, sd):     # output-major codes + block scales -> [in, out] values
        deq = oracle.mx4_dequantize if cfg.wdt == "mxfp4" else oracle.mx_dequantize
        return tuple(deq(mx_codes(w), sc.cpu().numpy()).T for w, sc in ((g, sg), (u, su), (dn, sd)))

    def expert(e):
        if e not in cache:
            if mx:
                cache[e] = mx_triple(inp["W_gate"][e], inp["W_up"][e], inp["W_down"][e],
                                     inp["mx_gate"][e], inp["mx_up"][e], inp["mx_down"][e])
            elif cfg.wdt == "fp8":
                cd = lambda t: t.contiguous().view(torch.uint8).cpu().numpy()
                cache[e] = (oracle.dequantize(cd(inp["W_gate"][e]), inp["s_gate"][e].cpu().numpy(), 1),
                            oracle.dequantize(cd(inp["W_up"][e]), inp["s_up"][e].cpu().numpy(), 1),
                            oracle.dequantize(cd(inp["W_down"][e]), inp["s_down"][e].cpu().numpy(), 1))
            else:
                cache[e] = (to64(inp["W_gate"][e]), to64(inp["W_up"][e]), to64(inp["W_down"][e]))
        return cache[e]

    shared = None
    if cfg.shared and mx:
        shared = mx_triple(inp["Ws_gate"], inp["Ws_up"], inp["Ws_down"],
                           inp["mxs_gate"], inp["mxs_up"], inp["mxs_down"])
    elif cfg.shared and cfg.wdt == "fp8":
        shared = (oracle.dequantize(cd(inp["Ws_gate"]), inp["ss_gate"].cpu().numpy(), 1),
                  oracle.dequantize(cd(inp["Ws_up"]), inp["ss_up"].cpu().numpy(), 1),
                  oracle.dequantize(cd(inp["Ws_down"]), inp["ss_down"].cpu().numpy(), 1))
    elif cfg.shared:
        shared = (to64(inp["Ws_gate"]), to64(inp["Ws_up"]), to64(inp["Ws_down"]))
    hooks = {}
    if mx:
        hooks = {"quant_x": oracle.mx_roundtrip, "quant_h": lambda H: oracle.mx_roundtrip(H, as_fp32=True)}
    tb = min(cfg.T, 8)             # tokens per oracle call
    call = lambda t0: oracle.forward(x[t0:t0 + tb], W_g, bias, cfg.k, cfg.renormalize,
                                     np.float32(cfg.capacity_factor), expert, cfg.E, shared=shared, **hooks)
    call(0)                        # untimed: widen the touched experts' weights once
    n = 0
    t_start = time.perf_counter()
    while n < max_calls and (time.perf_counter() - t_start) < budget_s:
        call((n * tb) % max(1, cfg.T - tb + 1))
        n += 1
    dt = time.perf_counter() - t_start
    return {"value": n * tb / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} oracle layer calls of {tb} token(s) each of the {cfg.name} workload "
                      f"(routing over all E experts, fp64 SwiGLU of the chosen experts), {dt:.1f} s"}


def bench_backward(args, cfg):
    """moe_backward on the workload: whole-call throughput (tokens/s), the dX
    GEMM (the largest row-tile GEMM, 4 rows d f flops) against the roofline its
    arithmetic intensity reaches first (bf16 MFMA, or HBM for small experts),
    and the oracle's backward on a small token sample."""
    import numpy as np
    import torch
    import synth
    from sparse_mixture_experts_12_amd import _lib as ops
    steps = args.steps if args.steps is not None else 10
    warmup = args.warmup if args.warmup is not None else 3
    print(f"[bench] backward workload={cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f} "
          f"routing={args.routing} steps={steps} warmup={warmup}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(cfg, "cuda")
    ec = args.routing == "expert"
    desc = ops.desc_from_cfg(cfg, routing=ops.ROUTING_EXPERT_CHOICE if ec else ops.ROUTING_TOKEN_CHOICE)
    w = ops.weights_struct(inp)
    gen = torch.Generator(device="cpu").manual_seed(7)
    adt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    dout = torch.randn((cfg.T, cfg.d), generator=gen).to(adt).cuda()
    ws = ops.alloc_backward_workspace(desc)
    z = lambda *sh: torch.empty(sh, dtype=torch.float32, device="cuda")
    g = {"dx": z(cfg.T, cfg.d), "dW_g": z(cfg.d, cfg.E), "d_bias": z(cfg.E) if inp["bias"] is not None else None,
         "dW_gate": z(cfg.E, cfg.d, cfg.f), "dW_up": z(cfg.E, cfg.d, cfg.f), "dW_down": z(cfg.E, cfg.f, cfg.d)}
    if cfg.shared:
        g.update(dWs_gate=z(cfg.d, cfg.f), dWs_up=z(cfg.d, cfg.f), dWs_down=z(cfg.f, cfg.d))
    gs = ops.grads_struct(g)
    # routing facts (kept rows) from one forward with stats
    counts = torch.zeros(cfg.E, dtype=torch.int32, device="cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=adt, device="cuda")
    fws = ops.alloc_workspace(desc)
    ops.forward(desc, inp["x"], w, out, fws, stats=ops.Stats(d_counts=counts.data_ptr()))
    torch.cuda.synchronize()
    cnt = counts.cpu().numpy()
    rows = int(cnt.sum()) + (cfg.T if cfg.shared else 0)
    n_exp = int((cnt > 0).sum()) + (1 if cfg.shared else 0)
    del fws
    for _ in range(warmup):
        ops.backward(desc, inp["x"], w, dout, gs, ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        ops.backward(desc, inp["x"], w, dout, gs, ws)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms = total_ms / steps
    kern_ms = float("nan")
    if not args.no_kernel_events:
        hev = HipEvents()
        eb = [hev.create() for _ in range(steps)]
        ee = [hev.create() for _ in range(steps)]
        for i in range(steps):
            ops.backward(desc, inp["x"], w, dout, ops.grads_struct(g, eb[i].value, ee[i].value), ws)
        torch.cuda.synchronize()
        kern_ms = sum(hev.elapsed_ms(eb[i], ee[i]) for i in range(steps)) / steps
    have_k = kern_ms == kern_ms
    kflops = 4 * rows * cfg.d * cfg.f                   # dX = [dG | dU] [W_gate | W_up]^T
    # its bytes: the touched experts' W_gate and W_up (bf16), dG and dU (bf16),
    # dX rows written in fp32; the bound is whichever roofline the arithmetic
    # intensity reaches first, as for the forward's gate/up GEMM
    # (fp32 layers: fp32 weights and rows, and the fp32 vector peak for the SIMT GEMM)
    f32 = cfg.act == "f32"
    es = 4 if f32 else 2
    kbytes = n_exp * 2 * cfg.d * cfg.f * es + rows * 2 * cfg.f * es + rows * cfg.d * 4
    flops = 16 * rows * cfg.d * cfg.f + 4 * cfg.T * cfg.d * cfg.E
    t = kern_ms / 1e3 if have_k else None
    cpeak = FP32_PEAK_TFLOPS if f32 else BF16_PEAK_TFLOPS
    if kflops / kbytes >= cpeak * 1e12 / (HBM_PEAK_GBS * 1e9):
        bound, peak, unit = ("alu" if f32 else "mfma"), cpeak, "TFLOP/s"
        achieved = kflops / t / 1e12 if have_k else None
    else:
        bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
        achieved = kbytes / t / 1e9 if have_k else None
    roof = {"bound": bound, "achieved": round(achieved, 2) if have_k else None, "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4) if have_k else None,
            # the stored counters cover token-choice routing only
            "traffic": None if ec else measured_traffic("bwd_dx_gemm", cfg.name),
            "kernel": "bwd_rows_f32_kernel (dX)" if f32 else "bwd_rows_kernel<NTS> (dX)",
            "kernel_ms": round(kern_ms, 5) if have_k else None, "alg_flops": int(kflops), "alg_bytes": int(kbytes),
            "mfma_frac": round(kflops / t / 1e12 / BF16_PEAK_TFLOPS, 4) if have_k and not f32 else None,
            "hbm_frac": round(kbytes / t / 1e9 / HBM_PEAK_GBS, 4) if have_k else None}
    if args.copy_calibration:     # the plain copy kernel whose counters scale the GEMM's (see main)
        a = torch.ones(1 << 27, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle's backward", file=sys.stderr, flush=True)
        cpu = cpu_baseline_backward(cfg, inp, dout, ec)
    line = {
        "metric": "MoE-layer backward tokens/s (dL/dx and all weight gradients)",
        "value": round(cfg.T * steps / (total_ms / 1e3), 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32" if f32 else "bf16", "data": "synthetic (seeded N(0,1) activations and dout, "
        "N(0,0.02) weights)",
        "config": {"workload": cfg.name, "pass": "backward", "T": cfg.T, "d": cfg.d, "E": cfg.E, "top_k": cfg.k,
                   "f": cfg.f, "shared_expert": cfg.shared, "capacity_factor": cfg.capacity_factor,
                   "routing": args.routing, "weights": cfg.wdt},
        "layer": {"alg_flops": int(flops), "tflops": round(flops / (ms / 1e3) / 1e12, 2)},
        "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


def bench_library_gemm(args, cfg):
    """torch.mm (hipBLASLt) on the layer's GEMM shapes: per expert M = T k / E
    rows (balanced routing), gate/up as one [M, d] x [d, 2 f] product, down as
    [M, f] x [f, d]; E products per step, bf16 in, bf16 out.  Context for the
    grouped GEMMs' MFMA fraction, not a layer measurement."""
    import torch
    if cfg.wdt != "bf16" or cfg.act != "bf16":
        print("--library-gemm takes bf16 layers", file=sys.stderr)
        sys.exit(2)
    steps = args.steps if args.steps is not None else 10
    warmup = args.warmup if args.warmup is not None else 3
    M = cfg.T * cfg.k // cfg.E
    gen = torch.Generator(device="cuda").manual_seed(11)
    shapes = {"gate_up": (M, cfg.d, 2 * cfg.f), "down": (M, cfg.f, cfg.d)}
    out = {}
    for name, (m, kk, n) in shapes.items():
        A = [torch.randn((m, kk), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(cfg.E)]
        B = [(torch.randn((kk, n), generator=gen, device="cuda") * 0.02).to(torch.bfloat16) for _ in range(cfg.E)]
        C = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _ in range(cfg.E)]

        def step():
            for e in range(cfg.E):
                torch.mm(A[e], B[e], out=C[e])
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        flops = 2.0 * cfg.E * m * kk * n
        tf = flops / (ms / 1e3) / 1e12
        out[name] = {"M": m, "K": kk, "N": n, "products": cfg.E, "ms": round(ms, 5), "tflops": round(tf, 1),
                     "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        print(f"[bench] library GEMM {name}: {cfg.E} x [{m}x{kk}] x [{kk}x{n}] {ms:.4f} ms, {tf:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        del A, B, C
        torch.cuda.empty_cache()
    line = {"metric": "library bf16 GEMM TFLOP/s (torch.mm on hipBLASLt) at the layer's per-expert GEMM shapes",
            "value": out["gate_up"]["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
            "higher_is_better": True, "dtype": "bf16", "data": "synthetic (seeded N(0,1) rows, N(0,0.02) weights)",
            "config": {"workload": cfg.name, "rows_per_expert": M, "experts": cfg.E}, "gemms": out,
            "peak": BF16_PEAK_TFLOPS}
    print(json.dumps(line), flush=True)


def cpu_baseline_backward(cfg, inp, dout, ec=False, budget_s=12.0, max_calls=200):
    """The oracle's backward, as it stands, on calls of a few tokens of the
    workload (expert choice: the selection among those tokens)."""
    import numpy as np
    import oracle
    import torch
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    to64 = lambda t: t.detach().to(torch.float64).cpu().numpy()
    x, W_g, d64 = to64(inp["x"]), to64(inp["W_g"]), to64(dout)
    bias = None if inp["bias"] is None else to64(inp["bias"])
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = (to64(inp["W_gate"][e]), to64(inp["W_up"][e]), to64(inp["W_down"][e]))
        return cache[e]
    shared = (to64(inp["Ws_gate"]), to64(inp["Ws_up"]), to64(inp["Ws_down"])) if cfg.shared else None
    tb = min(cfg.T, 4)
    fn = oracle.expert_choice_backward if ec else oracle.backward
    call = lambda t0: fn(x[t0:t0 + tb], W_g, bias, cfg.k, cfg.renormalize, np.float32(cfg.capacity_factor), expert,
                         cfg.E, shared, d64[t0:t0 + tb])
    call(0)
    n = 0
    t_start = time.perf_counter()
    while n < max_calls and (time.perf_counter() - t_start) < budget_s:
        call((n * tb) % max(1, cfg.T - tb + 1))
        n += 1
    dt = time.perf_counter() - t_start
    return {"value": n * tb / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} oracle {'expert-choice ' if ec else ''}backward calls of {tb} tokens each of the "
                      f"{cfg.name} workload (routing, fp64 expert and router gradients), {dt:.1f} s"}


def measure(args, cfg, steps=None, warmup=None, cpu=True, graph=True, copy_calibration=False):
    """One workload: the timed regions below, returned as the JSON line's dict."""
    import torch
    import synth
    from sparse_mixture_experts_12_amd import _lib as ops

    decode = cfg.T <= 8 and cfg.act == "bf16" and args.routing == "token"
    steps = steps if steps is not None else (200 if decode else 20)
    # a few ms of warm-up lets the clocks settle before the timed region
    warmup = warmup if warmup is not None else 10
    print(f"[bench] workload={cfg.name} T={cfg.T} d={cfg.d} E={cfg.E} k={cfg.k} f={cfg.f} "
          f"act={cfg.act} w={cfg.wdt} steps={steps} warmup={warmup}", file=sys.stderr, flush=True)

    inp = synth.make_inputs(cfg, "cuda")
    wbytes = synth.weight_bytes_per_expert(cfg) * (cfg.E + (1 if cfg.shared else 0))
    n_copies = max(1, min(8, math.ceil(2 * LLC_BYTES / max(1, wbytes)) + 1)) if wbytes < 4 * LLC_BYTES else 1
    if decode:
        n_copies = max(n_copies, 2)
    copies = [inp]
    for _ in range(n_copies - 1):
        c = dict(inp)
        for key in ("W_gate", "W_up", "W_down", "Ws_gate", "Ws_up", "Ws_down"):
            if inp.get(key) is not None:
                c[key] = inp[key].clone()
        copies.append(c)
    wstructs = [ops.weights_struct(c) for c in copies]
    routing = ops.ROUTING_EXPERT_CHOICE if args.routing == "expert" else ops.ROUTING_TOKEN_CHOICE
    desc = ops.desc_from_cfg(cfg, routing=routing)
    ws = ops.alloc_workspace(desc)
    dt = torch.float32 if cfg.act == "f32" else torch.bfloat16
    out = torch.empty((cfg.T, cfg.d), dtype=dt, device="cuda")
    counts = torch.zeros(cfg.E, dtype=torch.int32, device="cuda")
    nd = torch.zeros(1, dtype=torch.int32, device="cuda")

    # routing facts for the algorithmic work (one untimed call with stats)
    st0 = ops.Stats(d_n_dropped=nd.data_ptr(), d_counts=counts.data_ptr())
    path = ops.forward(desc, inp["x"], wstructs[0], out, ws, stats=st0)
    torch.cuda.synchronize()
    cnt = counts.cpu().numpy()
    touched = int((cnt > 0).sum())
    n_dropped = int(nd.cpu()[0])

    # Region 1 (headline): `steps` whole layer calls, nothing else on the stream.
    # Region 2: the same calls again, with HIP events stamped by the dispatch of
    # the dominant kernel itself, for its average duration (the events add a
    # few microseconds per step, so they are kept out of region 1).
    hev = HipEvents()
    ev_b = [hev.create() for _ in range(steps)]
    ev_e = [hev.create() for _ in range(steps)]
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        ops.forward(desc, inp["x"], wstructs[i % n_copies], out, ws)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    plain = ops.Stats()
    if args.telemetry:
        tel_routed = torch.zeros(cfg.E, dtype=torch.int32, device="cuda")
        tel_pm = torch.zeros(cfg.E, dtype=torch.float32, device="cuda")
        tel_loss = torch.zeros(1, dtype=torch.float32, device="cuda")
        plain = ops.Stats(d_routed=tel_routed.data_ptr(), d_prob_mean=tel_pm.data_ptr(),
                          d_lb_loss=tel_loss.data_ptr())
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        ops.forward(desc, inp["x"], wstructs[i % n_copies], out, ws, stats=plain)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / steps
    tokens_per_s = cfg.T * steps / (total_ms / 1e3)
    if args.telemetry:
        print(f"[bench] telemetry: load-balancing loss {float(tel_loss.cpu()[0]):.6f}, "
              f"max routed load {int(tel_routed.max())}, idle experts {int((tel_routed == 0).sum())}",
              file=sys.stderr, flush=True)
    kern_ms = float("nan")
    step_pct = None
    if not args.no_kernel_events:
        stats = [ops.Stats(ev_begin=ev_b[i].value, ev_end=ev_e[i].value) for i in range(steps)]
        for i in range(steps):
            ops.forward(desc, inp["x"], wstructs[i % n_copies], out, ws, stats=stats[i])
        torch.cuda.synchronize()
        kern_ms = sum(hev.elapsed_ms(ev_b[i], ev_e[i]) for i in range(steps)) / steps
        # Region 3: the same calls with an event between consecutive steps, for
        # the per-step spread (each event adds a little to its step)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        marks[0].record(stream)
        for i in range(steps):
            ops.forward(desc, inp["x"], wstructs[i % n_copies], out, ws, stats=plain)
            marks[i + 1].record(stream)
        torch.cuda.synchronize()
        per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
        q = lambda f: per_step[min(steps - 1, int(f * (steps - 1) + 0.5))]
        step_pct = {"p10": round(q(0.1), 5), "p50": round(q(0.5), 5), "p90": round(q(0.9), 5)}

    # Region 4: the same layer calls captured once into a HIP graph (one call per
    # weight copy) and replayed, as a serving loop would run them: the per-step
    # cost without host-side launch work between the kernels.
    graph_ms = None
    if graph:
        gstream = torch.cuda.Stream()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gstream):
            for c in range(n_copies):
                ops.forward(desc, inp["x"], wstructs[c], out, ws)
        reps = max(1, steps // n_copies)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (reps * n_copies)
        del graph

    bytes_total, flops, wbytes_used, _ = algorithmic_work(cfg, cnt, touched)
    layer_peak = (FP32_PEAK_TFLOPS if cfg.act == "f32" else
                  FP8_PEAK_TFLOPS if cfg.wdt in ("mxfp8", "mxfp4") else BF16_PEAK_TFLOPS)
    t_star = max(bytes_total / (HBM_PEAK_GBS * 1e9), flops / (layer_peak * 1e12))
    have_k = kern_ms == kern_ms            # False when the second region was skipped
    if decode:
        # dominant kernel = fused decode FFN: streams the chosen experts' weights (+ x)
        ae = 2
        kbytes = wbytes_used + cfg.T * cfg.d * ae
        achieved = kbytes / (kern_ms / 1e3) / 1e9 if have_k else None
        roof = {"bound": "hbm", "achieved": round(achieved, 1) if have_k else None, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4) if have_k else None,
                "traffic": measured_traffic("decode_ffn_kernel", cfg.name),
                "kernel": "decode_ffn_kernel" + (" + decode_down_kernel" if split_decode(cfg) else ""), "kernel_ms": round(kern_ms, 5) if have_k else None,
                "alg_bytes": int(kbytes)}
    else:
        # dominant kernel = grouped gate/up GEMM + SwiGLU: 2/3 of the expert flops.
        # Its bound is whichever roofline its arithmetic intensity hits first:
        # MFMA for Mixtral-sized experts, HBM for fine-grained and fp8 layers.
        f32 = cfg.act == "f32"
        rows = int(cnt.sum()) + (cfg.T if cfg.shared else 0)
        kflops = 4 * rows * cfg.d * cfg.f
        n_exp = touched + (1 if cfg.shared else 0)
        mx = cfg.wdt in ("mxfp8", "mxfp4")
        es = {"f32": 4, "bf16": 2, "fp8": 1, "mxfp8": 1, "mxfp4": 0.5}[cfg.wdt]
        scales = 2 * cfg.f * 4 if cfg.wdt == "fp8" else (2 * cfg.f * cfg.d // 32 if mx else 0)
        if mx:      # x and H travel as codes plus one scale byte per 32 values
            kbytes = (n_exp * (int(2 * cfg.d * cfg.f * es) + scales)
                      + (cfg.T * cfg.d + rows * cfg.f) * 33 // 32)
        else:
            ae = 4 if f32 else 2
            kbytes = n_exp * (2 * cfg.d * cfg.f * es + scales) + cfg.T * cfg.d * ae + rows * cfg.f * ae
        peak_f = FP32_PEAK_TFLOPS if f32 else (FP8_PEAK_TFLOPS if mx else BF16_PEAK_TFLOPS)
        ridge = peak_f * 1e12 / (HBM_PEAK_GBS * 1e9)
        kname = ("gemm_f32_*kernel" if f32 else "gemm_mx_kernel" if mx else
                 "gemm_dl_kernel")
        t = kern_ms / 1e3 if have_k else None
        if kflops / kbytes >= ridge:
            bound, peak, unit = "mfma", peak_f, "TFLOP/s"
            achieved = kflops / t / 1e12 if have_k else None
        else:
            bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
            achieved = kbytes / t / 1e9 if have_k else None
        roof = {"bound": bound, "achieved": round(achieved, 2) if have_k else None, "peak": peak,
                "unit": unit, "frac": round(achieved / peak, 4) if have_k else None,
                # the stored counters cover token-choice routing only
                "traffic": measured_traffic("gemm_gateup", cfg.name) if args.routing == "token" else None,
                "kernel": f"{kname}<gate/up>", "kernel_ms": round(kern_ms, 5) if have_k else None,
                "alg_flops": int(kflops), "alg_bytes": int(kbytes),
                "mfma_frac": round(kflops / t / 1e12 / peak_f, 4) if have_k else None,
                "hbm_frac": round(kbytes / t / 1e9 / HBM_PEAK_GBS, 4) if have_k else None}

    if copy_calibration:
        # a plain elementwise kernel of known traffic (256 MiB read, 256 MiB
        # written) whose HBM counters scale the layer kernels' counters
        a = torch.ones(1 << 27, dtype=torch.bfloat16, device="cuda")
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()

    cpu_line = None
    if cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu_line = cpu_baseline(cfg, inp)

    line = {
        "metric": "MoE-layer tokens/s; decode HBM GB/s, prefill MFMA TFLOP/s vs peak",
        "value": round(tokens_per_s, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "bf16 x fp8", "mxfp8": "mxfp8",
                                                                    "mxfp4": "mxfp8 x mxfp4"}[cfg.wdt] if cfg.act == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "top_k": cfg.k, "f": cfg.f,
                   "act": cfg.act, "weights": cfg.wdt, "shared_expert": cfg.shared,
                   "capacity_factor": cfg.capacity_factor, "path": "fused_decode" if path == 2 else "grouped",
                   "experts_touched": touched, "dropped_share": n_dropped / max(1, cfg.T * cfg.k),
                   "weight_copies": n_copies, "telemetry": bool(args.telemetry), "routing": args.routing},
        "layer": {"alg_bytes": int(bytes_total), "alg_flops": int(flops),
                  "hbm_GBps": round(bytes_total / (ms_per_step / 1e3) / 1e9, 1),
                  "tflops": round(flops / (ms_per_step / 1e3) / 1e12, 3),
                  # roofline time of the whole layer, max(bytes / HBM peak, flops / MFMA peak), against ms_per_step
                  "t_star_ms": round(t_star * 1e3, 5), "t_star_frac": round(t_star * 1e3 / ms_per_step, 4),
                  # per-step spread, from a third region with an event between steps
                  "step_ms": step_pct,
                  # the same steps replayed from a captured HIP graph
                  "graph_ms_per_step": round(graph_ms, 5) if graph_ms else None,
                  "graph_tokens_per_s": round(cfg.T / (graph_ms / 1e3), 2) if graph_ms else None,
                  "experts_empty": int(cfg.E - touched)},
        "roofline": roof,
        "cpu_baseline": cpu_line,
    }
    return line


# Workloads timed after the headline in a default run, each with its own
# warm-up and timed regions (no graph region, no CPU oracle): the prefill half
# of the metric and the other seeded workloads.
EXTRA_WORKLOADS = ("mixtral_prefill", "fine_grained", "fp8_capacity", "fp8_capacity_decode", "mixtral_decode_b8",
                   "tiny_f32")


def workload_row(line):
    """The compact per-workload record carried under the headline line's "workloads" key."""
    r, lay, c = line["roofline"], line["layer"], line["config"]
    return {"T": c["T"], "ms_per_step": line["ms_per_step"], "tokens_per_s": line["value"],
            "t_star_frac": lay["t_star_frac"], "path": c["path"], "experts_touched": c["experts_touched"],
            "dropped_share": c["dropped_share"], "kernel": r["kernel"], "kernel_ms": r["kernel_ms"],
            "bound": r["bound"], "achieved": r["achieved"], "unit": r["unit"], "frac": r["frac"],
            "mfma_frac": r.get("mfma_frac"), "hbm_frac": r.get("hbm_frac"), "traffic": r["traffic"]}


def bench_probe(args):
    """Roofline probes: HBM read rate of a 4 GiB stream, and the bf16 MFMA rate on
    register operands (no memory traffic) with random and with zero data."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_mixture_experts_12_amd", "libmoe_probe.so"))
    lib.probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    steps = args.steps or 10
    warmup = args.warmup if args.warmup is not None else 3

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    out = {"probe": "roofline", "steps": steps, "warmup": warmup}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.view(torch.int32).random_()
    rd = {}
    for grid in (64, 128, 256, 512, 1024, 2048, 8192, 32768, 131072):
        sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
        ms = timed(lambda: lib.probe_hbm_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, sp))
        rd[grid] = nbytes / (ms * 1e-3) / 1e9
    best = max(rd, key=rd.get)
    # grids of at most 256 work-groups put one on each of that many CUs: the per-CU streaming rate
    out["hbm_read_per_cu_GBps"] = {str(g): round(v / g, 2) for g, v in rd.items() if g <= 256}
    out["hbm_read"] = {"bytes": nbytes, "GBps_by_grid": {str(g): round(v, 1) for g, v in rd.items()},
                       "best_GBps": round(rd[best], 1), "frac_of_8TBps": round(rd[best] / HBM_PEAK_GBS, 4)}
    del buf
    grid, iters = 2048, 4096
    flops = grid * 4 * iters * 8 * 32768
    res = {}
    for kind in ("random", "zero"):
        src = torch.randn(grid * 256 * 64, device="cuda").to(torch.bfloat16)
        if kind == "zero":
            src.zero_()
        o = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
        ms = timed(lambda: lib.probe_mfma_bf16(src.data_ptr(), grid, iters, o.data_ptr(), sp))
        tf = flops / (ms * 1e-3) / 1e12
        res[kind] = {"ms": round(ms, 4), "TFLOPs": round(tf, 1), "frac_of_2500": round(tf / BF16_PEAK_TFLOPS, 4)}
    out["mfma_bf16_register_only"] = {"grid": grid, "iters": iters, "flops": flops, **res}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer would shard by tokens or by experts across GPUs)", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth

    if args.probe:
        return bench_probe(args)
    cfg = synth.CONFIGS[args.workload]
    if args.library_gemm:
        return bench_library_gemm(args, cfg)
    if args.backward:
        return bench_backward(args, cfg)
    line = measure(args, cfg, args.steps, args.warmup, cpu=not args.no_cpu_baseline, graph=not args.no_graph,
                   copy_calibration=args.copy_calibration)
    if not args.no_extra and args.routing == "token":
        rows = {}
        for name in EXTRA_WORKLOADS:
            if name == args.workload:
                continue
            torch.cuda.empty_cache()
            rows[name] = workload_row(measure(args, synth.CONFIGS[name], cpu=False, graph=False))
            print(f"[bench] {name}: {rows[name]['ms_per_step']} ms/step, {rows[name]['kernel']} "
                  f"{rows[name]['frac']} of its {rows[name]['bound']} roofline", file=sys.stderr, flush=True)
        line["workloads"] = rows
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
