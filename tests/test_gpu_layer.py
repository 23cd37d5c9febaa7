"""GPU parity of the whole layer (route -> permute -> experts ->
combine_norm, in the launch configuration the bench times) against the CPU
oracle, for every workload: the tiny all-fp32 layer in full, and the Beam
shapes (T = 8, 64 skewed, 2048 prefill, 16384 fp8) with all 256 experts
resident.  Routing and the permutation are compared for every token; the
layer outputs on all tokens (T <= 8) or a seeded sample of tokens."""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (check_output, check_permutation_props, check_routes, oracle_cfg,
                         sample_tokens, say)

beam = pytest.importorskip("expert_routed_ffn_amd")
pytestmark = pytest.mark.gpu
DEV = "cuda"

_stacks = {}


def stacks(wl, cfg):
    """Packed device stacks, generated expert by expert."""
    key = (wl.w_dtype, wl.seed, wl.hidden, wl.d_ff, wl.n_experts)
    if key not in _stacks:
        say(f"  generating packed expert stacks {key}")
        _stacks.clear()
        torch.cuda.empty_cache()
        _stacks[key] = beam.packed_expert_stacks(cfg, lambda e: synth.make_expert(wl, e, DEV), wl.n_experts, DEV)
        torch.cuda.synchronize()
    return _stacks[key]


def run_layer(wname, n_sample):
    wl = synth.WORKLOADS[wname]
    say(f"layer {wname}: T={wl.T} w={wl.w_dtype}")
    cfg = beam.LayerCfg(wl.hidden, wl.n_experts, wl.n_groups, wl.topk_groups, wl.topk,
                        wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)
    wgu, wd, sgu, sd = stacks(wl, cfg)
    w_r, bias = synth.make_router(wl, DEV)
    x, h, gp, gq = synth.make_activations(wl, DEV)
    fp8 = wl.w_dtype == "fp8"
    w_dt = {"f32": beam.BEAM_F32, "bf16": beam.BEAM_BF16, "fp8": beam.BEAM_FP8_E4M3}[wl.w_dtype]
    y_dt = torch.bfloat16 if fp8 else torch.float32
    bufs = beam.alloc_buffers(cfg, wl.T, x.dtype, w_dt, y_dtype=y_dt, keep_logits=True,
                              keep_moe_out=True, device=DEV)
    h_dev = h.clone()
    beam.moe_layer(cfg, x, w_r, bias, wgu, wd, h_dev, gp, gq, wl.n, bufs, s_gate_up=sgu, s_down=sd)
    torch.cuda.synchronize()
    say("  gpu layer done")

    ocfg = oracle_cfg(wl)
    xn = synth.to_f64(x)
    logits = oracle.router_logits(xn, synth.to_f64(w_r))
    routes = oracle.route(logits, synth.to_f64(bias), ocfg)
    gids = bufs.topk_ids.cpu().numpy()
    n_near, differ = check_routes(gids, bufs.topk_w.cpu().numpy(), routes, ocfg)

    off, rt, pr = (bufs.expert_offsets.cpu().numpy(), bufs.row_token.cpu().numpy(),
                   bufs.pair_row.cpu().numpy())
    if not differ:
        o_off, o_rt, o_pr = oracle.permutation(np.array([r.ids for r in routes]), wl.n_experts)
        assert np.array_equal(off, o_off) and np.array_equal(rt, o_rt) and np.array_equal(pr, o_pr)
    else:
        check_permutation_props(gids, off, rt, pr, wl.n_experts)
    counts = np.diff(off)
    say(f"  experts touched: {int((counts > 0).sum())}, max rows per expert {int(counts.max())}")

    if fp8:
        q_gpu = oracle.e4m3_decode(bufs.x_q.cpu().numpy())
        s_gpu = bufs.x_scale.cpu().double().numpy()
        for t in sample_tokens(wl.T, 64, seed=1):
            s, q = oracle.quantize_row_e4m3(xn[t])
            assert s_gpu[t] == s and np.array_equal(q_gpu[t], q), t

    tokens = [t for t in sample_tokens(wl.T, n_sample, seed=2) if t not in differ]
    # the oracle reads the plain row-major weights, regenerated per expert
    def ew(e):
        a, b, c, d = synth.make_expert(wl, e, DEV)
        if fp8:
            return {"q_gu": a.cpu().numpy(), "s_gu": synth.to_f64(c), "q_d": b.cpu().numpy(), "s_d": synth.to_f64(d)}
        return {"w_gu": synth.to_f64(a), "w_d": synth.to_f64(b)}
    rnd = oracle.round_f32 if wl.act_dtype == "f32" else oracle.round_bf16
    ref = oracle.layer_tokens(ocfg, xn, synth.to_f64(w_r), synth.to_f64(bias), ew, synth.to_f64(h),
                              synth.to_f64(gp), synth.to_f64(gq), wl.n, tokens=tokens,
                              w_dtype=wl.w_dtype, rnd=rnd)
    kind = {"f32": "f32", "bf16": "bf16", "fp8": "fp8"}[wl.w_dtype]
    say(f"  compared tokens: {tokens}")
    check_output("m", bufs.moe_out.cpu().double().numpy()[tokens], ref["m"], kind)
    check_output("h_new", h_dev.cpu().double().numpy()[tokens], ref["h_new"], kind)
    check_output("x_next", bufs.x_next.cpu().double().numpy()[tokens], ref["x_next"], kind)
    return n_near


def test_layer_tiny_fp32():
    run_layer("tiny_fp32", 4)


def test_layer_decode_t8():
    run_layer("decode_t8", 8)


def test_layer_skew_t64():
    run_layer("skew_t64", 6)


def test_layer_prefill_t2048():
    run_layer("prefill_t2048", 4)


def test_layer_prefill_fp8_t16384():
    run_layer("prefill_fp8_t16384", 4)
    _stacks.clear()
    torch.cuda.empty_cache()
