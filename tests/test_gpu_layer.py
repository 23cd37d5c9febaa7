"""GPU parity of the whole layer (route -> permute -> experts ->
combine_norm, in the launch configuration the bench times) against the CPU
oracle, for every workload: the tiny all-fp32 layer in full, and the Beam
shapes (T = 8, 64 skewed, 2048 prefill, 16384 with bf16 and with fp8
experts; T = 8 and 64 with 4-bit MXFP4 experts) with all 256 experts
resident.

Per workload:
  * routing of every token (ids exact outside near-ties, weights 1e-5);
    a near-tie token whose GPU choice differs must hold a valid choice, and
    the oracle then re-evaluates it with that choice (ids_override);
  * the permutation of every pair, bit-exact against the oracle's counting
    sort of those ids;
  * the expert outputs y of EVERY row of a few chosen experts: the most
    loaded one (several 128-row work items), one whose item reaches rows
    64..127, and the least loaded one;
  * the layer outputs m, h', x_next of all tokens (T <= 64) or of a seeded
    sample of at least 32 tokens that includes tokens whose pairs sit in
    rows 64..127 of their work items;
  * for fp8 and MXFP4 experts also the quantisation "floor" (the quantised
    oracle against the unquantised-activation oracle on the same weights),
    printed beside the GPU's parity; the run-time activation codes are
    compared bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (check_output, check_routes, oracle_cfg, rel_l2, sample_tokens, say)

beam = pytest.importorskip("expert_routed_ffn_amd")
pytestmark = pytest.mark.gpu
DEV = "cuda"
ITEM_ROWS = 128      # rows per work item of the prefill expert GEMMs

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


def expert_weights_fn(wl):
    """Plain row-major weights of expert e for the oracle, regenerated per
    expert (a progress line every 32 experts)."""
    fp8 = wl.w_dtype == "fp8"
    mx = wl.w_dtype == "mxfp4"
    calls = [0]

    def ew(e):
        calls[0] += 1
        if calls[0] % 32 == 0:
            say(f"    oracle: {calls[0]} experts evaluated")
        a, b, c, d = synth.make_expert(wl, e, DEV)
        if fp8:
            return {"q_gu": a.cpu().numpy(), "s_gu": synth.to_f64(c), "q_d": b.cpu().numpy(), "s_d": synth.to_f64(d)}
        if mx:
            return {"c_gu": oracle.unpack_fp4(a.cpu().numpy()), "s_gu": c.cpu().numpy(),
                    "c_d": oracle.unpack_fp4(b.cpu().numpy()), "s_d": d.cpu().numpy()}
        return {"w_gu": synth.to_f64(a), "w_d": synth.to_f64(b)}
    return ew


def pick_tokens(T, n_sample, off, pair_row, K, seed, all_small=True):
    """All tokens if T <= 64 (and all_small), else n_sample tokens: half of
    them owners of a pair that sits in rows 64..127 of its 128-row work item,
    half a seeded sample (including the first and last token)."""
    if T <= 64 and all_small:
        return list(range(T))
    E = len(off) - 1
    start = np.repeat(off[:-1], np.diff(off))            # first row of each row's expert
    item_pos = (np.arange(off[-1]) - start) % ITEM_ROWS   # row index inside its work item
    deep_rows = np.flatnonzero(item_pos >= 64)
    inv = np.empty(len(pair_row), dtype=np.int64)
    inv[pair_row] = np.arange(len(pair_row))
    deep_tok = sorted({int(inv[r]) // K for r in deep_rows})
    rng = np.random.default_rng(seed)
    n_deep = min(len(deep_tok), n_sample // 2)
    chosen = set(int(t) for t in rng.choice(deep_tok, n_deep, replace=False)) if n_deep else set()
    chosen |= set(sample_tokens(T, n_sample - len(chosen), seed=seed))
    return sorted(chosen)


def pick_experts(off):
    """Most loaded expert, an expert with 65..128 rows in one of its items
    (rows 64..127 of an item), and the least loaded touched expert."""
    counts = np.diff(off)
    touched = np.flatnonzero(counts > 0)
    heavy = int(np.argmax(counts))
    out = [heavy]
    deep = [int(e) for e in touched if counts[e] > 64 and int(e) != heavy]
    if deep:
        out.append(deep[0])
    light = int(touched[np.argmin(counts[touched])])
    if light not in out:
        out.append(light)
    return out


def run_layer(wname, n_sample, check_experts=True, all_small=True):
    wl = synth.WORKLOADS[wname]
    say(f"layer {wname}: T={wl.T} w={wl.w_dtype}")
    cfg = beam.LayerCfg(wl.hidden, wl.n_experts, wl.n_groups, wl.topk_groups, wl.topk,
                        wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)
    wgu, wd, sgu, sd = stacks(wl, cfg)
    w_r, bias = synth.make_router(wl, DEV)
    x, h, gp, gq = synth.make_activations(wl, DEV)
    fp8 = wl.w_dtype == "fp8"
    mx = wl.w_dtype == "mxfp4"
    w_dt = {"f32": beam.BEAM_F32, "bf16": beam.BEAM_BF16, "fp8": beam.BEAM_FP8_E4M3,
            "mxfp4": beam.BEAM_MXFP4}[wl.w_dtype]
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
    # Where several results are correct -- a near-tie token whose GPU set
    # differs (validated above), or neighbours within 1e-6 reported in the
    # other order (validated above) -- the oracle continues with the GPU's
    # choice: its permutation and, for differing sets, its layer outputs.
    ids = np.array([r.ids for r in routes])
    override = {t: [int(v) for v in gids[t]] for t in range(wl.T) if list(gids[t]) != list(ids[t])}
    for t, v in override.items():
        ids[t] = v

    off, rt, pr = (bufs.expert_offsets.cpu().numpy(), bufs.row_token.cpu().numpy(),
                   bufs.pair_row.cpu().numpy())
    o_off, o_rt, o_pr = oracle.permutation(ids, wl.n_experts)
    assert np.array_equal(off, o_off) and np.array_equal(rt, o_rt) and np.array_equal(pr, o_pr)
    counts = np.diff(o_off)
    say(f"  experts touched: {int((counts > 0).sum())}, max rows per expert {int(counts.max())}")

    if fp8:
        q_gpu = oracle.e4m3_decode(bufs.x_q.cpu().numpy())
        s_gpu = bufs.x_scale.cpu().double().numpy()
        for t in sample_tokens(wl.T, 64, seed=1):
            s, q = oracle.quantize_row_e4m3(xn[t])
            assert s_gpu[t] == s and np.array_equal(q_gpu[t], q), t
    if mx:
        # run-time MXFP4 codes and block scales of x, bit for bit
        s_o, q_o = oracle.quantize_mx_fp4(xn)
        np.testing.assert_array_equal(bufs.x_scale.cpu().numpy(), s_o)
        np.testing.assert_array_equal(oracle.unpack_fp4(bufs.x_q.cpu().numpy()), oracle.e2m1_encode(q_o))

    kind = {"f32": "f32", "bf16": "bf16", "fp8": "fp8", "mxfp4": "mx"}[wl.w_dtype]
    ew = expert_weights_fn(wl)
    rnd = oracle.round_f32 if wl.act_dtype == "f32" else oracle.round_bf16

    if check_experts:
        # every row of the chosen experts, through the oracle's expert MLP
        y_gpu = bufs.y
        for e in pick_experts(o_off):
            lo, hi = int(o_off[e]), int(o_off[e + 1])
            w = ew(e)
            u = xn[o_rt[lo:hi]]
            if fp8:
                ref = oracle.expert_ffn_w8a8(u, w["q_gu"], w["s_gu"], w["q_d"], w["s_d"])
            elif mx:
                ref = oracle.expert_ffn_w4a4(u, w["c_gu"], w["s_gu"], w["c_d"], w["s_d"])
            else:
                ref = oracle.expert_ffn(u, w["w_gu"], w["w_d"], round_a=rnd)
            got = y_gpu[lo:hi].double().cpu().numpy()
            check_output(f"y expert {e} ({hi - lo} rows, {(hi - lo + ITEM_ROWS - 1) // ITEM_ROWS} items)",
                         got, ref, kind if y_dt == torch.float32 or kind == "fp8" else "bf16")

    tokens = sorted(set(pick_tokens(wl.T, n_sample, o_off, o_pr, wl.topk, seed=2, all_small=all_small)) | differ)
    ref = oracle.layer_tokens(ocfg, xn, synth.to_f64(w_r), synth.to_f64(bias), ew, synth.to_f64(h),
                              synth.to_f64(gp), synth.to_f64(gq), wl.n, tokens=tokens,
                              w_dtype=wl.w_dtype, rnd=rnd, ids_override={t: override[t] for t in differ})
    say(f"  compared {len(tokens)} tokens ({len([t for t in tokens if t in differ])} re-evaluated "
        f"near-tie tokens): {tokens[:12]}{' ...' if len(tokens) > 12 else ''}")
    check_output("m", bufs.moe_out.cpu().double().numpy()[tokens], ref["m"], kind)
    check_output("h_new", h_dev.cpu().double().numpy()[tokens], ref["h_new"], kind)
    check_output("x_next", bufs.x_next.cpu().double().numpy()[tokens], ref["x_next"], kind)
    if fp8:
        # the floor: W8A8 oracle against the same layer with unquantised
        # activations on the same (dequantised) weights
        table = oracle.e4m3_decode(np.arange(256))

        def ew_float(e):
            w = ew(e)
            return {"w_gu": table[w["q_gu"]] * w["s_gu"][:, None],
                    "w_d": table[w["q_d"]] * w["s_d"][:, None]}
        flo = oracle.layer_tokens(ocfg, xn, synth.to_f64(w_r), synth.to_f64(bias), ew_float,
                                  synth.to_f64(h), synth.to_f64(gp), synth.to_f64(gq), wl.n,
                                  tokens=tokens, w_dtype="bf16", rnd=lambda v: np.asarray(v, np.float64),
                                  ids_override={t: override[t] for t in differ})
        say(f"  W8A8 floor (W8A8 oracle vs unquantised activations): rel_l2(m)={rel_l2(ref['m'], flo['m']):.3e}; "
            f"GPU vs W8A8 oracle rel_l2(m)={rel_l2(bufs.moe_out.cpu().double().numpy()[tokens], ref['m']):.3e}")
    if mx:
        # the 4-bit floor: W4A4 oracle against unquantised activations on the
        # same dequantised weights
        def ew_float(e):
            w = ew(e)
            def deq(c, sc):
                return oracle.e2m1_decode(c) * np.repeat(oracle.e8m0_decode(sc), oracle.MX_BLOCK, axis=-1)
            return {"w_gu": deq(w["c_gu"], w["s_gu"]), "w_d": deq(w["c_d"], w["s_d"])}
        flo = oracle.layer_tokens(ocfg, xn, synth.to_f64(w_r), synth.to_f64(bias), ew_float,
                                  synth.to_f64(h), synth.to_f64(gp), synth.to_f64(gq), wl.n,
                                  tokens=tokens, w_dtype="bf16", rnd=lambda v: np.asarray(v, np.float64),
                                  ids_override={t: override[t] for t in differ})
        say(f"  W4A4 floor (W4A4 oracle vs unquantised activations): rel_l2(m)={rel_l2(ref['m'], flo['m']):.3e}; "
            f"GPU vs W4A4 oracle rel_l2(m)={rel_l2(bufs.moe_out.cpu().double().numpy()[tokens], ref['m']):.3e}")
    return n_near


def special_rows(wl):
    """Decode-sized input with an all-zero row, a row holding one NaN and two
    rows holding one +inf / -inf element; the other rows are ordinary."""
    x, h, gp, gq = synth.make_activations(wl, DEV)
    x = x.clone()
    x[2] = 0
    x[4, 100] = float("nan")
    x[6, 7] = float("inf")
    x[7, 5] = float("-inf")
    return x, h, gp, gq, [2, 0, 1, 3, 5], [4, 6, 7]


def run_special_rows(wl):
    """The layer completes on non-finite inputs: finite tokens (the all-zero
    one included) still match the oracle, every token gets K distinct valid
    expert ids, and a token with a NaN or infinite input gets non-finite
    outputs (no hang, no access outside the buffers)."""
    cfg = beam.LayerCfg(wl.hidden, wl.n_experts, wl.n_groups, wl.topk_groups, wl.topk,
                        wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)
    wgu, wd, sgu, sd = stacks(wl, cfg)
    w_r, bias = synth.make_router(wl, DEV)
    x, h, gp, gq, finite, bad = special_rows(wl)
    fp8 = wl.w_dtype == "fp8"
    w_dt = beam.BEAM_FP8_E4M3 if fp8 else beam.BEAM_BF16
    bufs = beam.alloc_buffers(cfg, wl.T, x.dtype, w_dt, y_dtype=torch.bfloat16 if fp8 else torch.float32,
                              keep_moe_out=True, device=DEV)
    h_dev = h.clone()
    beam.moe_layer(cfg, x, w_r, bias, wgu, wd, h_dev, gp, gq, wl.n, bufs, s_gate_up=sgu, s_down=sd)
    torch.cuda.synchronize()
    gids = bufs.topk_ids.cpu().numpy()
    for t in range(wl.T):
        assert len(set(gids[t].tolist())) == wl.topk and gids[t].min() >= 0 and gids[t].max() < wl.n_experts, t
    assert int(bufs.expert_offsets[-1]) == wl.T * wl.topk
    hn, xn_, m = h_dev.cpu().double().numpy(), bufs.x_next.cpu().double().numpy(), bufs.moe_out.cpu().double().numpy()
    for t in bad:
        assert not np.isfinite(hn[t]).any() and not np.isfinite(xn_[t]).any(), t
        assert not np.isfinite(m[t]).all(), t
    say(f"  non-finite rows {bad}: ids {[gids[t].tolist() for t in bad]}, outputs non-finite")
    ocfg = oracle_cfg(wl)
    xd = synth.to_f64(x)
    routes = oracle.route(oracle.router_logits(xd[finite], synth.to_f64(w_r)), synth.to_f64(bias), ocfg)
    _, differ = check_routes(gids[finite], bufs.topk_w.cpu().numpy()[finite], routes, ocfg)
    assert not differ
    ref = oracle.layer_tokens(ocfg, xd, synth.to_f64(w_r), synth.to_f64(bias), expert_weights_fn(wl),
                              synth.to_f64(h), synth.to_f64(gp), synth.to_f64(gq), wl.n, tokens=finite,
                              w_dtype=wl.w_dtype, rnd=oracle.round_bf16)
    kind = "fp8" if fp8 else "bf16"
    check_output("m", m[finite], ref["m"], kind)
    check_output("h_new", hn[finite], ref["h_new"], kind)
    check_output("x_next", xn_[finite], ref["x_next"], kind)
    assert np.all(m[2] == 0)   # the all-zero row: every expert output is exactly zero


def run_graph_replay(wname):
    """The four calls captured in one hipGraph and replayed three times, with
    the program's own eager work and synchronisations in between: every
    replay reproduces the eager layer bit for bit."""
    wl = synth.WORKLOADS[wname]
    cfg = beam.LayerCfg(wl.hidden, wl.n_experts, wl.n_groups, wl.topk_groups, wl.topk,
                        wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)
    wgu, wd, sgu, sd = stacks(wl, cfg)
    w_r, bias = synth.make_router(wl, DEV)
    x, h0, gp, gq = synth.make_activations(wl, DEV)
    bufs = beam.alloc_buffers(cfg, wl.T, x.dtype, beam.BEAM_BF16, keep_moe_out=True, device=DEV)
    h = h0.clone()
    beam.moe_layer(cfg, x, w_r, bias, wgu, wd, h, gp, gq, wl.n, bufs)
    torch.cuda.synchronize()
    want = [t.clone() for t in (bufs.topk_ids, bufs.topk_w, bufs.pair_row, h, bufs.x_next, bufs.moe_out)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        beam.moe_layer(cfg, x, w_r, bias, wgu, wd, h, gp, gq, wl.n, bufs)
    for rep in range(3):
        h.copy_(h0)
        bufs.x_next.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (bufs.topk_ids, bufs.topk_w, bufs.pair_row, h, bufs.x_next, bufs.moe_out)
        for a, b in zip(got, want):
            assert torch.equal(a, b), rep
        # eager work between replays: an ordinary layer call on other data
        h.copy_(h0 * 0.5)
        beam.moe_layer(cfg, x * 2, w_r, bias, wgu, wd, h, gp, gq, wl.n, bufs)
        torch.cuda.synchronize()
    say(f"  {wname}: 3 graph replays identical to the eager layer")
    del g


def run_side_stream(wl):
    """8-bit / 4-bit experts with the input quantisation on a second stream
    (default priority) beside the router and the permutation: the layer is
    bit-identical to the one-stream layer, eagerly and in a captured graph
    replayed twice."""
    cfg = beam.LayerCfg(wl.hidden, wl.n_experts, wl.n_groups, wl.topk_groups, wl.topk,
                        wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)
    wgu, wd, sgu, sd = stacks(wl, cfg)
    w_r, bias = synth.make_router(wl, DEV)
    x, h0, gp, gq = synth.make_activations(wl, DEV)
    fp8 = wl.w_dtype == "fp8"
    w_dt = beam.BEAM_FP8_E4M3 if fp8 else beam.BEAM_MXFP4
    y_dt = torch.bfloat16 if fp8 else torch.float32
    bufs = beam.alloc_buffers(cfg, wl.T, x.dtype, w_dt, y_dtype=y_dt, keep_moe_out=True, device=DEV)
    outs = lambda h: [t.clone() for t in (bufs.topk_ids, bufs.topk_w, bufs.pair_row, bufs.x_q, bufs.x_scale,
                                          bufs.moe_out, h, bufs.x_next)]
    h = h0.clone()
    beam.moe_layer(cfg, x, w_r, bias, wgu, wd, h, gp, gq, wl.n, bufs, s_gate_up=sgu, s_down=sd)
    torch.cuda.synchronize()
    want = outs(h)
    side = torch.cuda.Stream()
    for b in (bufs.x_q, bufs.x_scale):
        b.zero_()
    h = h0.clone()
    beam.moe_layer(cfg, x, w_r, bias, wgu, wd, h, gp, gq, wl.n, bufs, s_gate_up=sgu, s_down=sd,
                   quant_stream=side)
    torch.cuda.synchronize()
    for a, b in zip(outs(h), want):
        assert torch.equal(a, b)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        beam.moe_layer(cfg, x, w_r, bias, wgu, wd, h, gp, gq, wl.n, bufs, s_gate_up=sgu, s_down=sd,
                       quant_stream=side)
    for rep in range(2):
        h.copy_(h0)
        bufs.x_q.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs(h), want):
            assert torch.equal(a, b), rep
    say(f"  {wl.name} T={wl.T}: quantisation on a second stream, eager and 2 graph replays bit-identical")
    del g


def test_layer_tiny_fp32():
    run_layer("tiny_fp32", 4)


def test_layer_decode_t8():
    run_layer("decode_t8", 8)


def test_layer_special_rows_bf16():
    run_special_rows(synth.WORKLOADS["decode_t8"])


def test_layer_graph_replay_decode_t8():
    run_graph_replay("decode_t8")


def test_layer_skew_t64():
    run_layer("skew_t64", 64)


@pytest.mark.timeout(400)
def test_layer_prefill_t2048():
    run_layer("prefill_t2048", 32)


def test_layer_graph_replay_prefill_t2048():
    run_graph_replay("prefill_t2048")


@pytest.mark.timeout(400)
def test_layer_prefill_bf16_t16384():
    run_layer("prefill_bf16_t16384", 32)


@pytest.mark.timeout(400)
def test_layer_prefill_fp8_t16384():
    run_layer("prefill_fp8_t16384", 32)


def test_layer_decode_t8_mxfp4():
    run_layer("decode_t8_mxfp4", 8)


def test_layer_skew_t64_mxfp4():
    # 16 sampled tokens, half of them in rows 64..127 of their items (the
    # oracle decodes every 4-bit expert a token uses); every row of the
    # heaviest experts is still compared
    run_layer("skew_t64_mxfp4", 16, all_small=False)


@pytest.mark.timeout(400)
def test_layer_prefill_mxfp4_t16384():
    # 8 sampled tokens (the oracle decodes every 4-bit expert a token uses);
    # the heaviest experts are still checked row by row
    run_layer("prefill_mxfp4_t16384", 8)


def test_layer_side_stream_mxfp4():
    run_side_stream(synth.WORKLOADS["decode_t8_mxfp4"])


def test_layer_special_rows_fp8():
    run_special_rows(synth.WORKLOADS["prefill_fp8_t16384"].with_T(8))


def test_layer_side_stream_fp8():
    run_side_stream(synth.WORKLOADS["prefill_fp8_t16384"].with_T(300))
    _stacks.clear()
    torch.cuda.empty_cache()
