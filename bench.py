#!/usr/bin/env python3
"""Throughput of one Beam MoE layer forward on one MI355X.

A step is one pass of the whole layer (route -> permute -> experts ->
combine_norm) over one batch of seeded synthetic tokens, with the inputs
and all 256 experts' weights resident in HBM.  The headline line is the
Beam decode shape (T = 8 tokens, bf16 experts); the same JSON line carries
the other shapes the metric is quoted on (T = 64 with skewed routes,
T = 2048 prefill, T = 16384 with fp8 experts, and T = 16384 with bf16
experts), the shapes with 4-bit MXFP4 experts (T = 8, 64 and 16384), the
dense layers (d_ff 20480, T = 8 and 2048) and one GPU's share of the layer
under 8-way expert parallelism (T = 8 and 2048) under "configs".  Prints
one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--configs a,b|none]
    (--workload dense_t8 / dense_t2048 / ep8_shard_t8 / ep8_shard_t2048 prints
    that row's entry alone, for profiling runs)

Timing: one pair of HIP events on the launch stream around the whole timed
region (`ms_per_step` is the region over K) and one pair around the experts
call of every timed step; the per-stage times (route, permute, experts,
combine_norm) come from a second pass of K steps with an event after every
C-ABI call, so that those markers do not sit inside the timed region.  The
`roofline` object describes the dominant call, beam_moe_experts (its
work-item, GEMM1 + SwiGLU and GEMM2 kernels), against HBM or MFMA peak
depending on the rows per touched expert.  A hipGraph replay of the same
step is timed as well.  `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_MFMA_TFLOPS = 2500.0        # dense
FP8_MFMA_TFLOPS = 5000.0
FP4_MFMA_TFLOPS = 10100.0
MFMA_PEAK = {"bf16": BF16_MFMA_TFLOPS, "f32": BF16_MFMA_TFLOPS, "fp8": FP8_MFMA_TFLOPS, "mxfp4": FP4_MFMA_TFLOPS}
WEIGHT_BYTES = {"bf16": 2.0, "f32": 4.0, "fp8": 1.0, "mxfp4": 0.5 + 1.0 / 32}   # per weight, with block scales


def ridge_rows(w_dtype):
    """Rows per expert at which the expert GEMMs' flops per weight byte
    reach the MFMA peak over the HBM peak (312.5 for bf16 and fp8, about
    335 for MXFP4)."""
    return MFMA_PEAK[w_dtype] * 1e12 / (HBM_PEAK_GBS * 1e9) / (2.0 / WEIGHT_BYTES[w_dtype])
SIDE_STREAM_MIN_T = 1024          # tokens from which the input quantisation gets its own stream
RIDGE_ROWS = 312.5               # rows per expert where weight streaming stops bounding (bf16 and fp8)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the sources of every kernel inside the experts and dense MLP calls (the
# GEMMs, work items, SwiGLU slices, e4m3 and MXFP4 re-quantisation of a)
EXPERTS_SRCS = [os.path.join(ROOT, "expert_routed_ffn_amd", "csrc", f)
                for f in ("experts.hip", "common.h", "mx.hip")]
DEFAULT_CONFIGS = ("skew_t64,prefill_t2048,prefill_fp8_t16384,prefill_bf16_t16384,"
                   "decode_t8_mxfp4,skew_t64_mxfp4,prefill_mxfp4_t16384,dense_t8,dense_t2048,ep8_shard_t8,"
                   "ep8_shard_t2048")
METRIC = "MoE-layer tokens/s (one Beam MoE layer forward incl. routing and norm boundary)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_t8")
    ap.add_argument("--configs", default=DEFAULT_CONFIGS,
                    help="comma-separated extra workloads timed into the same line, or 'none'")
    ap.add_argument("--no-graph", action="store_true", help="skip the hipGraph replay timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (counter calibration) and exit")
    ap.add_argument("--gemm-reference", action="store_true",
                    help="only time the vendor library (hipBLASLt through torch) on dense bf16 / fp8 GEMMs "
                         "of the expert GEMM sizes, as a reference for the expert kernels, and exit")
    return ap.parse_args()


def gemm_reference():
    """Dense GEMMs in the vendor library at the expert GEMM sizes, one JSON
    line each: all T*K = 131072 rows of the T = 16384 layer against one
    weight matrix (GEMM1 5120 x 5120, GEMM2 5120 x 2560), and one expert's
    share (512 rows).  A reference for the grouped kernels, not a path of
    the layer."""
    import torch
    dev = "cuda:0"
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(n):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n * 1e3

    for M, N, K in [(131072, 5120, 5120), (131072, 5120, 2560), (512, 5120, 5120), (512, 5120, 2560)]:
        a = torch.randn(M, K, device=dev, dtype=torch.bfloat16)
        b = torch.randn(N, K, device=dev, dtype=torch.bfloat16)
        flop = 2.0 * M * N * K
        us = timed(lambda: a @ b.t())
        a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
        one = torch.ones((), device=dev)
        us8 = timed(lambda: torch._scaled_mm(a8, b8.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16))
        print(json.dumps({"gemm": [M, N, K], "bf16_us": round(us, 1), "bf16_tflops": round(flop / us / 1e6, 1),
                          "fp8_us": round(us8, 1), "fp8_tflops": round(flop / us8 / 1e6, 1)}), flush=True)
        del a, b, a8, b8


class HipEvents:
    """Raw hipEvent_t handles (ctypes) recorded on the launch stream."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
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
    h = hashlib.sha256()
    for f in EXPERTS_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


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
    w_r, bias = synth.make_router(wl, dev)
    x, h, gp, gq = synth.make_activations(wl, dev)
    fp8 = wl.w_dtype == "fp8"
    mx = wl.w_dtype == "mxfp4"
    w_dt = beam.BEAM_FP8_E4M3 if fp8 else (beam.BEAM_MXFP4 if mx else beam.BEAM_BF16)
    bufs = beam.alloc_buffers(lcfg(wl), wl.T, x.dtype, w_dt, y_dtype=torch.bfloat16 if fp8 else torch.float32,
                              device=dev)
    wgu, wd, sgu, sd = stacks
    # 8-bit / 4-bit experts at large T: the input quantisation runs on a
    # second stream (default priority) alongside the router and the
    # permutation.  At decode sizes the fork and join of a second stream
    # cost more than the few-µs quantisation they would hide, so it runs in
    # line there.
    side = torch.cuda.Stream() if (fp8 or mx) and wl.T >= SIDE_STREAM_MIN_T else None
    return dict(cfg=lcfg(wl), w_r=w_r, bias=bias, x=x, h=h.clone(), h0=h, gp=gp, gq=gq, bufs=bufs,
                wgu=wgu, wd=wd, sgu=sgu, sd=sd, fp8=fp8, mx=mx, side=side)


def run_step(wl, s, hipev=None, evs=None, stream=None, marks=(0, 1, 2, 3, 4)):
    """One layer step through the C-ABI calls; with evs (5 events) an event
    is recorded on the launch stream before the first call and after the
    route, permute, experts and combine_norm calls (only those of them that
    `marks` lists, so the timed steps carry no more markers than the
    roofline needs).  With 8-bit or 4-bit
    experts the input quantisation runs either on a second stream alongside
    the route and permute calls (the experts call waits for it) or in line,
    in the route stage (MXFP4) or inside the permute call (e4m3)."""
    import torch
    import expert_routed_ffn_amd as beam
    cfg, b = s["cfg"], s["bufs"]
    mark = (lambda i: hipev.record(evs[i], stream) if i in marks else None) if evs is not None \
        else (lambda i: None)
    side = s["side"]
    mark(0)
    if side is not None:
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        if s["fp8"]:
            beam.beam_moe_quantize_fp8(cfg, s["x"], b.x_q, b.x_scale, stream=side)
        else:
            beam.beam_moe_quantize_mx(cfg, s["x"], b.x_q, b.x_scale, stream=side)
    beam.beam_moe_route(cfg, s["x"], s["w_r"], s["bias"], b.topk_ids, b.topk_w, b.logits, b.ws)
    if s["mx"] and side is None:   # in line: timed in the route stage
        beam.beam_moe_quantize_mx(cfg, s["x"], b.x_q, b.x_scale)
    mark(1)
    inline8 = s["fp8"] and side is None   # in line: inside the permute call
    beam.beam_moe_permute(cfg, b.topk_ids, b.expert_offsets, b.row_token, b.pair_row,
                          x=s["x"] if inline8 else None, x_q=b.x_q if inline8 else None,
                          x_scale=b.x_scale if inline8 else None, ws=b.ws)
    if side is not None:
        main.wait_stream(side)
    mark(2)
    beam.beam_moe_experts(cfg, wl.T, b.x_q if (s["fp8"] or s["mx"]) else s["x"], b.expert_offsets, b.row_token,
                          s["wgu"], s["wd"], b.y, x_scale=b.x_scale, s_gate_up=s["sgu"], s_down=s["sd"],
                          ws=b.ws)
    mark(3)
    beam.beam_moe_combine_norm(cfg, b.y, b.pair_row, b.topk_w, s["h"], b.x_next, s["gp"], s["gq"], wl.n,
                               b.moe_out)
    mark(4)


def stats(v):
    return {"median": round(statistics.median(v), 2), "min": round(min(v), 2),
            "mean": round(sum(v) / len(v), 2)}


def time_workload(wl, stacks, steps, warmup, hipev, dev, graph=True):
    """The timed region per step, the experts call's time in each timed step
    (events around that call only), touched experts, per-step stage times
    (µs) from a second, fully marked pass of the same number of steps after
    the timed region, and (optionally) the hipGraph replay time per step."""
    import torch
    s = layer_setup(wl, stacks, dev)
    stream = torch.cuda.current_stream().cuda_stream
    evs = [[hipev.create() for _ in range(5)] for _ in range(steps)]
    evs2 = [[hipev.create() for _ in range(5)] for _ in range(steps)]
    t0, t1 = hipev.create(), hipev.create()
    for _ in range(warmup):
        run_step(wl, s)
    torch.cuda.synchronize()
    hipev.record(t0, stream)
    for i in range(steps):
        run_step(wl, s, hipev, evs[i], stream, marks=(2, 3))
    hipev.record(t1, stream)
    torch.cuda.synchronize()
    region_ms = hipev.elapsed_ms(t0, t1)
    for i in range(steps):
        run_step(wl, s, hipev, evs2[i], stream)
    torch.cuda.synchronize()
    per = {k: [] for k in ("layer", "route", "permute", "experts", "combine_norm")}
    for e, f in zip(evs, evs2):
        per["experts"].append(hipev.elapsed_ms(e[2], e[3]) * 1e3)
        per["layer"].append(hipev.elapsed_ms(f[0], f[4]) * 1e3)
        per["route"].append(hipev.elapsed_ms(f[0], f[1]) * 1e3)
        per["permute"].append(hipev.elapsed_ms(f[1], f[2]) * 1e3)
        per["combine_norm"].append(hipev.elapsed_ms(f[3], f[4]) * 1e3)
    offs = s["bufs"].expert_offsets.cpu()
    D = int(((offs[1:] - offs[:-1]) > 0).sum())
    out = dict(ms_per_step=region_ms / steps, per=per, touched=D, state=s)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_step(wl, s)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        cs = torch.cuda.current_stream().cuda_stream
        hipev.record(t0, cs)
        for _ in range(steps):
            g.replay()
        hipev.record(t1, cs)
        torch.cuda.synchronize()
        out["graph_us_per_layer"] = hipev.elapsed_ms(t0, t1) * 1e3 / steps
        del g
    return out


def algorithmic(wl, D):
    """Algorithmic bytes and flops (what the method itself must move and
    compute): the touched experts' weights (+ fp8 per-row scales), W_r,
    and x, h in, h' and x_next out.  Permuted copies, the SwiGLU
    intermediate and the expert outputs y are not credited.
    Flops per (token, expert) pair: 2*H*2F (GEMM1) + 2*F*H (GEMM2)."""
    H, F, T, K, E = wl.hidden, wl.d_ff, wl.T, wl.topk, wl.n_experts
    fp8 = wl.w_dtype == "fp8"
    mx = wl.w_dtype == "mxfp4"
    if mx:    # E2M1 half-bytes plus one E8M0 byte per 32 weights / activations
        w_expert = 3 * H * F // 2 + 3 * H * F // 32
        x_read = T * H // 2 + T * H // 32
    else:
        es = 1 if fp8 else 2
        w_expert = 3 * H * F * es + ((2 * F + H) * 4 if fp8 else 0)
        x_read = T * H * (1 if fp8 else 2) + (T * 4 if fp8 else 0)     # the GEMM input: e4m3 codes + scales, or bf16
    experts_bytes = D * w_expert + x_read
    layer_bytes = D * w_expert + E * H * 4 + 4 * T * H * 2
    experts_flops = 6 * H * F * T * K
    return dict(w_expert=w_expert, experts_bytes=experts_bytes, layer_bytes=layer_bytes,
                experts_flops=experts_flops, layer_flops=experts_flops + 2 * T * H * E)


def traffic_for(workload, call="experts"):
    """Measured HBM bytes per beam_moe_experts (or beam_moe_dense_mlp) call
    from the committed rocprofv3 counter summary, or None if it is missing
    or was taken on different sources of the call's kernels."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    rec = t.get(workload, {}).get(call)
    if not rec or rec.get("kernel_src_hash") != kernel_hash():
        return None
    return rec.get("bytes_per_call")


def roofline_entry(wl, r):
    """Roofline of the dominant call (beam_moe_experts) and of the layer."""
    D = r["touched"]
    alg = algorithmic(wl, D)
    fp8 = wl.w_dtype == "fp8"
    mx = wl.w_dtype == "mxfp4"
    ex_us = sum(r["per"]["experts"]) / len(r["per"]["experts"])
    ex_s = ex_us / 1e6
    rows_per_expert = wl.T * wl.topk / max(D, 1)
    if rows_per_expert >= ridge_rows(wl.w_dtype):
        peak = MFMA_PEAK[wl.w_dtype]
        ach = alg["experts_flops"] / ex_s / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "algorithmic_flops": alg["experts_flops"]}
    else:
        ach = alg["experts_bytes"] / ex_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "algorithmic_bytes": alg["experts_bytes"]}
    roof.update({"traffic": traffic_for(wl.name),
                 "kernel": "beam_moe_experts call (work items, GEMM1 + SwiGLU, GEMM2"
                           + (", e4m3 re-quantisation of a" if fp8 else "")
                           + (", MXFP4 quantisation of a" if mx else "") + ")",
                 "kernel_avg_us": round(ex_us, 2)})
    step_s = r["ms_per_step"] / 1e3
    peak_f = MFMA_PEAK[wl.w_dtype]
    layer = {"hbm_frac": round(alg["layer_bytes"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
             "mfma_frac": round(alg["layer_flops"] / step_s / 1e12 / peak_f, 4),
             "algorithmic_bytes": alg["layer_bytes"], "algorithmic_flops": alg["layer_flops"]}
    return roof, layer


def cpu_baseline(wl, state, n_tokens, min_seconds=10.0, max_reps=8):
    """Times the CPU oracle on the first n_tokens tokens of the workload,
    repeating the pass until at least min_seconds of CPU work have been
    timed.  The experts' plain weights are staged on the host before the
    clock starts; the oracle widens them to fp64 itself as part of its work."""
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
    return {"value": round(len(tokens) * reps / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(tokens)} of the {wl.T} tokens of {wl.name} through the whole layer (router, "
                      f"selection, the {len(need)} experts they use as fp64 SwiGLU MLPs"
                      f"{' with e4m3 activations' if fp8 else ''}, combine, norm boundary), "
                      f"{reps} passes, {dt:.1f} s on {cores} host threads"}


def time_dense(wl, steps, warmup, hipev, dev):
    """Dense layer step: beam_moe_dense_mlp + beam_moe_norm_boundary."""
    import torch
    import expert_routed_ffn_amd as beam
    import synth
    cfg = lcfg(wl)
    w_gu, w_d, _, _ = synth.make_expert(wl, 0, dev)
    pgu, pd = torch.empty_like(w_gu), torch.empty_like(w_d)
    beam.beam_moe_pack_weights(cfg, w_gu.unsqueeze(0), w_d.unsqueeze(0), pgu.unsqueeze(0), pd.unsqueeze(0))
    del w_gu, w_d
    x, h, gp, gq = synth.make_activations(wl, dev)
    y = torch.empty((wl.T, wl.hidden), dtype=torch.float32, device=dev)
    xn = torch.empty_like(h)
    ws = beam.dense_workspace(cfg, wl.T, wl.d_ff)
    stream = torch.cuda.current_stream().cuda_stream

    def step(evs=None):
        if evs:
            hipev.record(evs[0], stream)
        beam.beam_moe_dense_mlp(cfg, x, pgu, pd, y, ws)
        if evs:
            hipev.record(evs[1], stream)
        beam.beam_moe_norm_boundary(cfg, y, h, xn, gp, gq, wl.n)
        if evs:
            hipev.record(evs[2], stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[hipev.create() for _ in range(3)] for _ in range(steps)]
    t0, t1 = hipev.create(), hipev.create()
    hipev.record(t0, stream)
    for i in range(steps):
        step(evs[i])
    hipev.record(t1, stream)
    torch.cuda.synchronize()
    mlp = [hipev.elapsed_ms(e[0], e[1]) * 1e3 for e in evs]
    nb = [hipev.elapsed_ms(e[1], e[2]) * 1e3 for e in evs]
    layer = [hipev.elapsed_ms(e[0], e[2]) * 1e3 for e in evs]
    us = hipev.elapsed_ms(t0, t1) * 1e3 / steps
    H, Fd, T = wl.hidden, wl.d_ff, wl.T
    mlp_us = sum(mlp) / len(mlp)
    wbytes = 3 * H * Fd * 2 + T * H * 2
    flops = 6 * H * Fd * T
    if T >= RIDGE_ROWS:
        ach = flops / (mlp_us / 1e6) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_MFMA_TFLOPS, 4), "algorithmic_flops": flops}
    else:
        ach = wbytes / (mlp_us / 1e6) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "algorithmic_bytes": wbytes}
    roof.update({"traffic": traffic_for(wl.name, "dense_mlp"),
                 "kernel": "beam_moe_dense_mlp call (GEMM1 + SwiGLU, GEMM2" +
                 (", K-slice sum" if T <= 16 else "") + ")", "kernel_avg_us": round(mlp_us, 2)})
    return {"us_per_layer": round(us, 1), "tokens_per_s": round(T / (us / 1e6), 1), "T": T, "d_ff": Fd,
            "expert_weights": "bf16 (dense)", "layer_us": stats(layer),
            "stages_us_median": {"dense_mlp": round(statistics.median(mlp), 2),
                                 "norm_boundary": round(statistics.median(nb), 2)},
            "roofline": roof}


def time_ep_shards(wl, stacks, steps, warmup, hipev, dev, n_shards=8):
    """One GPU's share of the layer under EP8, for each of the 8 groups of 32
    experts in turn: beam_moe_permute_shard, beam_moe_experts on the group's
    slice of the stacks, beam_moe_combine_partial (the routes computed once,
    as every GPU computes the same routes).  The all-reduce and the norm
    boundary that follows it are not part of a shard."""
    import torch
    import expert_routed_ffn_amd as beam
    s = layer_setup(wl, stacks, dev)
    run_step(wl, s)                       # routes and the unsharded layer
    torch.cuda.synchronize()
    cfg, b = s["cfg"], s["bufs"]
    per = wl.n_experts // n_shards
    scfg = beam.LayerCfg(wl.hidden, per, 1, 1, wl.topk, wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)
    T, K, H = wl.T, wl.topk, wl.hidden
    off = torch.empty(per + 1, dtype=torch.int32, device=dev)
    rt = torch.empty(T * K, dtype=torch.int32, device=dev)
    pr = torch.empty(T * K, dtype=torch.int32, device=dev)
    m = torch.empty((T, H), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    shards = []
    for r in range(n_shards):
        eb = r * per
        wg, wdn = s["wgu"][eb:eb + per], s["wd"][eb:eb + per]

        def step(evs=None):
            if evs:
                hipev.record(evs[0], stream)
            beam.beam_moe_permute_shard(cfg, b.topk_ids, eb, per, off, rt, pr, ws=b.ws)
            if evs:
                hipev.record(evs[1], stream)
            beam.beam_moe_experts(scfg, T, s["x"], off, rt, wg, wdn, b.y, ws=b.ws)
            if evs:
                hipev.record(evs[2], stream)
            beam.beam_moe_combine_partial(cfg, b.y, pr, b.topk_w, m)
            if evs:
                hipev.record(evs[3], stream)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        evs = [[hipev.create() for _ in range(4)] for _ in range(steps)]
        for i in range(steps):
            step(evs[i])
        torch.cuda.synchronize()
        tot = sum(hipev.elapsed_ms(e[0], e[3]) for e in evs) * 1e3 / steps
        ex = sum(hipev.elapsed_ms(e[1], e[2]) for e in evs) * 1e3 / steps
        D = int(((off[1:] - off[:-1]) > 0).sum())
        alg = D * 3 * H * wl.d_ff * 2 + T * H * 2
        shards.append({"shard": r, "us": round(tot, 1), "experts_us": round(ex, 1), "experts_touched": D,
                       "experts_hbm_frac": round(alg / (ex / 1e6) / 1e9 / HBM_PEAK_GBS, 4)})
    worst = max(shards, key=lambda d: d["us"])
    ach = worst["experts_touched"] * 3 * H * wl.d_ff * 2 + T * H * 2
    return {"T": T, "shards": n_shards, "experts_per_shard": per,
            "shard_us_max": worst["us"], "shard_us_mean": round(sum(d["us"] for d in shards) / n_shards, 1),
            "roofline": {"bound": "hbm", "achieved": round(ach / (worst["experts_us"] / 1e6) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": worst["experts_hbm_frac"], "algorithmic_bytes": ach,
                         "traffic": None,   # counters are taken per layer workload, not per shard
                         "kernel": f"beam_moe_experts call of the slowest shard ({worst['shard']})",
                         "kernel_avg_us": worst["experts_us"]},
            "per_shard": shards}


def entry(wl, r):
    roof, layer = roofline_entry(wl, r)
    sec = r["ms_per_step"] / 1e3
    e = {"us_per_layer": round(r["ms_per_step"] * 1e3, 1),
         "tokens_per_s": round(wl.T / sec, 1),
         "T": wl.T, "expert_weights": wl.w_dtype, "experts_touched": r["touched"],
         "layer_us": stats(r["per"]["layer"]),
         "stages_us_median": {k: round(statistics.median(v), 2) for k, v in r["per"].items() if k != "layer"},
         "roofline": roof, "layer_roofline": layer}
    if "graph_us_per_layer" in r:
        e["graph_us_per_layer"] = round(r["graph_us_per_layer"], 1)
    return e


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
    if args.gemm_reference:
        gemm_reference()
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

    EP_BASE = {"ep8_shard_t8": "decode_t8", "ep8_shard_t2048": "prefill_t2048"}
    if args.workload in EP_BASE or synth.WORKLOADS[args.workload].dense:
        # one dense-layer or EP8-shard row on its own (for profiling runs):
        # its entry as one JSON line, not the metric line
        if args.workload in EP_BASE:
            w1 = synth.WORKLOADS[EP_BASE[args.workload]]
            e1 = time_ep_shards(w1, packed_stacks(w1, dev), args.steps, args.warmup, hipev, dev)
        else:
            e1 = time_dense(synth.WORKLOADS[args.workload], args.steps, args.warmup, hipev, dev)
        print(json.dumps({"workload": args.workload, **e1}), flush=True)
        return
    wl = synth.WORKLOADS[args.workload]
    by_dtype = {wl.w_dtype: packed_stacks(wl, dev)}
    r = time_workload(wl, by_dtype[wl.w_dtype], args.steps, args.warmup, hipev, dev, graph=not args.no_graph)
    main_entry = entry(wl, r)
    print(f"# {wl.name}: {main_entry['us_per_layer']} us/layer", file=sys.stderr, flush=True)
    fp8 = wl.w_dtype == "fp8"
    out = {
        "metric": METRIC,
        "value": main_entry["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "us_per_layer": main_entry["us_per_layer"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3" if fp8 else "bf16",
        "data": "synthetic (seeded; all 256 experts resident in HBM)",
        "config": {"workload": wl.name, "T": wl.T, "hidden": wl.hidden, "n_experts": wl.n_experts,
                   "groups": f"{wl.topk_groups}/{wl.n_groups}", "topk": wl.topk, "d_ff": wl.d_ff,
                   "expert_weights": wl.w_dtype, "router": "fp32", "experts_touched": r["touched"],
                   "parallelism": "single GPU"},
        "roofline": main_entry["roofline"],
        "layer_roofline": main_entry["layer_roofline"],
        "layer_us": main_entry["layer_us"],
        "stages_us_median": main_entry["stages_us_median"],
    }
    if "graph_us_per_layer" in main_entry:
        out["graph_us_per_layer"] = main_entry["graph_us_per_layer"]
    state_main = r["state"]
    names = [] if args.configs == "none" else [n for n in args.configs.split(",") if n and n != wl.name]
    cfgs = {}
    for name in names:
        if name.startswith("ep8_shard_"):
            base = {"ep8_shard_t8": "decode_t8", "ep8_shard_t2048": "prefill_t2048"}[name]
            w2 = synth.WORKLOADS[base]
            if w2.w_dtype not in by_dtype:
                by_dtype[w2.w_dtype] = packed_stacks(w2, dev)
            cfgs[name] = time_ep_shards(w2, by_dtype[w2.w_dtype], args.steps, min(args.warmup, 3), hipev, dev)
            print(f"# {name}: slowest shard {cfgs[name]['shard_us_max']} us", file=sys.stderr, flush=True)
            continue
        w2 = synth.WORKLOADS[name]
        if w2.dense:
            cfgs[name] = time_dense(w2, args.steps, min(args.warmup, 3), hipev, dev)
            print(f"# {name}: {cfgs[name]['us_per_layer']} us/layer", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
            continue
        if w2.w_dtype not in by_dtype:
            by_dtype[w2.w_dtype] = packed_stacks(w2, dev)
        r2 = time_workload(w2, by_dtype[w2.w_dtype], args.steps, min(args.warmup, 3), hipev, dev,
                           graph=not args.no_graph)
        cfgs[name] = entry(w2, r2)
        print(f"# {name}: {cfgs[name]['us_per_layer']} us/layer", file=sys.stderr, flush=True)
        del r2
        torch.cuda.empty_cache()
    if cfgs:
        out["configs"] = cfgs
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, state_main, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
