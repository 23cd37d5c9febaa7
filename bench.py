#!/usr/bin/env python3
"""Throughput of one Beam MoE layer forward on one MI355X.

A step is one pass of the whole layer (route -> permute -> experts ->
combine_norm) over one batch of seeded synthetic tokens, with the inputs
and all 256 experts' weights resident in HBM.  Default workload: the Beam
decode shape, T = 8 tokens, bf16 experts.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--all]

The roofline object describes the dominant kernel (GEMM1: gate/up
projection + SwiGLU), timed with HIP events recorded on the stream it runs
on, inside the timed region.  The cpu_baseline object times the CPU oracle
on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_MFMA_TFLOPS = 2500.0        # dense
FP8_MFMA_TFLOPS = 5000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
EXPERTS_SRC = os.path.join(ROOT, "expert_routed_ffn_amd", "csrc", "experts.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_t8")
    ap.add_argument("--all", action="store_true", help="also time the other Beam workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (counter calibration) and exit")
    return ap.parse_args()


class HipEvents:
    """Raw hipEvent_t handles (ctypes), so the library can record them on its
    own launch stream."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev.value

    def record(self, ev, stream):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)


def kernel_hash():
    return hashlib.sha256(open(EXPERTS_SRC, "rb").read()).hexdigest()[:16]


def lcfg(wl):
    import expert_routed_ffn_amd as beam
    return beam.LayerCfg(wl.hidden, wl.n_experts, wl.n_groups, wl.topk_groups, wl.topk,
                         wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)


def packed_stacks(wl, dev):
    """All experts' weights in the packed layout the expert GEMM reads
    (built once, before any timing)."""
    import torch
    import expert_routed_ffn_amd as beam
    import synth
    st = beam.packed_expert_stacks(lcfg(wl), lambda e: synth.make_expert(wl, e, dev), wl.n_experts, dev)
    torch.cuda.synchronize()
    return st


def layer_setup(wl, stacks, dev):
    import torch
    import expert_routed_ffn_amd as beam
    import synth
    cfg = beam.LayerCfg(wl.hidden, wl.n_experts, wl.n_groups, wl.topk_groups, wl.topk,
                        wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)
    w_r, bias = synth.make_router(wl, dev)
    x, h, gp, gq = synth.make_activations(wl, dev)
    fp8 = wl.w_dtype == "fp8"
    w_dt = beam.BEAM_FP8_E4M3 if fp8 else beam.BEAM_BF16
    bufs = beam.alloc_buffers(cfg, wl.T, x.dtype, w_dt, y_dtype=torch.bfloat16 if fp8 else torch.float32,
                              device=dev)
    wgu, wd, sgu, sd = stacks
    state = dict(cfg=cfg, w_r=w_r, bias=bias, x=x, h=h.clone(), h0=h, gp=gp, gq=gq, bufs=bufs,
                 wgu=wgu, wd=wd, sgu=sgu, sd=sd)
    return state


def run_step(wl, s, events=None):
    import expert_routed_ffn_amd as beam
    beam.moe_layer(s["cfg"], s["x"], s["w_r"], s["bias"], s["wgu"], s["wd"], s["h"], s["gp"], s["gq"],
                   wl.n, s["bufs"], s_gate_up=s["sgu"], s_down=s["sd"], events=events)


def time_workload(wl, stacks, steps, warmup, hipev, dev):
    """Returns dict with ms/step, GEMM1/GEMM2 average ms, touched experts."""
    import torch
    s = layer_setup(wl, stacks, dev)
    stream = torch.cuda.current_stream().cuda_stream
    evs = [[hipev.create() for _ in range(4)] for _ in range(steps)]
    t0, t1 = hipev.create(), hipev.create()
    for _ in range(warmup):
        run_step(wl, s)
    torch.cuda.synchronize()
    hipev.record(t0, stream)
    for i in range(steps):
        run_step(wl, s, events=evs[i])
    hipev.record(t1, stream)
    torch.cuda.synchronize()
    total_ms = hipev.elapsed_ms(t0, t1)
    g1 = sum(hipev.elapsed_ms(e[0], e[1]) for e in evs) / steps
    g2 = sum(hipev.elapsed_ms(e[2], e[3]) for e in evs) / steps
    offs = s["bufs"].expert_offsets.cpu()
    D = int(((offs[1:] - offs[:-1]) > 0).sum())
    return dict(ms_per_step=total_ms / steps, gemm1_ms=g1, gemm2_ms=g2, touched=D, state=s)


def algorithmic(wl, D):
    """Algorithmic bytes and flops of GEMM1, GEMM2 and the whole layer.

    Per touched expert: gate/up 2*F*H weights, down H*F weights (2 bytes bf16,
    1 byte fp8 plus per-row fp32 scales).  Flops per (token, expert) pair:
    2*H*2F (GEMM1) + 2*F*H (GEMM2)."""
    H, F, T, K, E = wl.hidden, wl.d_ff, wl.T, wl.topk, wl.n_experts
    es = 1 if wl.w_dtype == "fp8" else 2
    TK = T * K
    g1_w = D * (2 * F * H * es + (2 * F * 4 if es == 1 else 0))
    g1_bytes = g1_w + T * H * es + TK * F * (4 if es == 1 else 2)
    g2_w = D * (H * F * es + (H * 4 if es == 1 else 0))
    g2_bytes = g2_w + TK * F * (1 if es == 1 else 2) + TK * H * (2 if es == 1 else 4)
    layer_bytes = g1_w + g2_w + E * H * 4 + 4 * T * H * 2   # weights + W_r + x, h, h', x_next
    g1_flops = 2 * TK * H * 2 * F
    g2_flops = 2 * TK * F * H
    return dict(g1_bytes=g1_bytes, g2_bytes=g2_bytes, layer_bytes=layer_bytes, g1_flops=g1_flops,
                g2_flops=g2_flops, router_flops=2 * T * H * E)


def traffic_for(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if it is missing or was taken on a different kernel source."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = t.get(workload, {}).get(kernel)
    if not rec or rec.get("kernel_src_hash") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, state, n_tokens, min_seconds=10.0, max_reps=8):
    """Times the CPU oracle on the first n_tokens tokens of the workload (all
    of them for the decode shape), repeating the pass until at least
    min_seconds of CPU work have been timed.  The experts' plain bf16 weights
    are staged on the host before the clock starts; the oracle widens them
    to fp64 itself as part of its work."""
    import numpy as np
    import torch
    import oracle
    import synth
    s = state
    tokens = list(range(min(n_tokens, wl.T)))
    xn = synth.to_f64(s["x"])[tokens]
    w_r = synth.to_f64(s["w_r"])
    bias = synth.to_f64(s["bias"])
    ocfg = dict(n_experts=wl.n_experts, n_groups=wl.n_groups, topk_groups=wl.topk_groups,
                topk=wl.topk, group_topn=wl.group_topn, routed_scale=wl.routed_scale,
                hidden=wl.hidden, d_ff=wl.d_ff, rms_eps=wl.rms_eps)
    routes = oracle.route(oracle.router_logits(xn, w_r), bias, ocfg)
    need = sorted({int(e) for r in routes for e in r.ids})
    # plain row-major weights of the needed experts, staged on the host before the clock
    host = {}
    for e in need:
        a, b, c, d = synth.make_expert(wl, e, s["x"].device)
        host[e] = (a.cpu(), b.cpu(), None if c is None else synth.to_f64(c), None if d is None else synth.to_f64(d))
    fp8 = wl.w_dtype == "fp8"
    if fp8:
        ew = lambda e: {"q_gu": host[e][0].numpy(), "s_gu": host[e][2], "q_d": host[e][1].numpy(), "s_d": host[e][3]}
    else:
        ew = lambda e: {"w_gu": host[e][0].to(torch.float64).numpy(), "w_d": host[e][1].to(torch.float64).numpy()}
    h = synth.to_f64(s["h0"])[tokens]
    gp, gq = synth.to_f64(s["gp"]), synth.to_f64(s["gq"])
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        oracle.layer_tokens(ocfg, xn, w_r, bias, ew, h, gp, gq, wl.n, w_dtype=wl.w_dtype,
                            rnd=oracle.round_bf16)
        dt += time.perf_counter() - t0
        reps += 1
    cores = len(os.sched_getaffinity(0))
    return {"value": len(tokens) * reps / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(tokens)} of the {wl.T} tokens of {wl.name} through the whole layer (router, "
                      f"selection, the {len(need)} experts they use as fp64 SwiGLU MLPs, combine, norm "
                      f"boundary), {reps} passes, {dt:.1f} s on {cores} host threads"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs the MoE layer on one GPU; multi-GPU runs "
                                   "(--gpus > 1) are not supported", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}))
        return
    import expert_routed_ffn_amd as beam
    import synth
    if not os.path.exists(beam.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    hipev = HipEvents()

    wl = synth.WORKLOADS[args.workload]
    stacks = packed_stacks(wl, dev)
    torch.cuda.synchronize()
    r = time_workload(wl, stacks, args.steps, args.warmup, hipev, dev)
    D = r["touched"]
    alg = algorithmic(wl, D)
    fp8 = wl.w_dtype == "fp8"
    g1_s = r["gemm1_ms"] / 1e3
    achieved = alg["g1_bytes"] / g1_s / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_for(wl.name, "gemm1"),
                "kernel": "beam_expert_gemm (GEMM1 gate/up + SwiGLU)",
                "kernel_avg_us": round(r["gemm1_ms"] * 1e3, 2),
                "algorithmic_bytes": alg["g1_bytes"]}
    if wl.T * wl.topk / max(D, 1) >= 315 * (2 if fp8 else 1):
        peak = FP8_MFMA_TFLOPS if fp8 else BF16_MFMA_TFLOPS
        ach = alg["g1_flops"] / g1_s / 1e12
        roofline.update({"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(ach / peak, 4)})
    step_s = r["ms_per_step"] / 1e3
    layer_hbm = alg["layer_bytes"] / step_s / 1e9
    out = {
        "metric": "MoE-layer tokens/s (one Beam MoE layer forward incl. routing and norm boundary)",
        "value": round(wl.T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "us_per_layer": round(r["ms_per_step"] * 1e3, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if fp8 else "bf16",
        "data": "synthetic (seeded; all 256 experts resident in HBM)",
        "config": {"workload": wl.name, "T": wl.T, "hidden": wl.hidden, "n_experts": wl.n_experts,
                   "groups": f"{wl.topk_groups}/{wl.n_groups}", "topk": wl.topk, "d_ff": wl.d_ff,
                   "expert_weights": wl.w_dtype, "router": "fp32", "experts_touched": D,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "layer_hbm": {"achieved": round(layer_hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(layer_hbm / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg["layer_bytes"]},
        "kernels_us": {"gemm1": round(r["gemm1_ms"] * 1e3, 2), "gemm2": round(r["gemm2_ms"] * 1e3, 2)},
    }
    if args.all:
        extra = {}
        names = [n for n in synth.WORKLOAD_ORDER if n not in ("tiny_fp32", wl.name)]
        by_dtype = {wl.w_dtype: stacks}
        for name in names:
            w2 = synth.WORKLOADS[name]
            if w2.w_dtype not in by_dtype:
                by_dtype[w2.w_dtype] = packed_stacks(w2, dev)
            r2 = time_workload(w2, by_dtype[w2.w_dtype], max(3, args.steps // 5), 2, hipev, dev)
            a2 = algorithmic(w2, r2["touched"])
            fl = a2["g1_flops"] + a2["g2_flops"]
            peak = FP8_MFMA_TFLOPS if w2.w_dtype == "fp8" else BF16_MFMA_TFLOPS
            sec = r2["ms_per_step"] / 1e3
            extra[name] = {"us_per_layer": round(r2["ms_per_step"] * 1e3, 1),
                           "tokens_per_s": round(w2.T / sec, 1),
                           "experts_touched": r2["touched"],
                           "hbm_frac": round(a2["layer_bytes"] / sec / 1e9 / HBM_PEAK_GBS, 4),
                           "mfma_frac": round(fl / sec / 1e12 / peak, 4),
                           "gemm1_us": round(r2["gemm1_ms"] * 1e3, 1), "gemm2_us": round(r2["gemm2_ms"] * 1e3, 1)}
            del r2
        out["other_workloads"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, r["state"], args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
