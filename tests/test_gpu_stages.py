"""GPU parity of each entry point on its own, against the CPU oracle, on
seeded synthetic inputs: router + selection, permutation, per-token e4m3
quantisation, grouped experts (fp32, bf16, fp8) and combine + norm.  Sizes
span several tiles with ragged tails; edge cases include single tokens,
zero-token experts and every token on one expert."""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import (check_output, check_routes, oracle_cfg, rel_l2, say)

beam = pytest.importorskip("expert_routed_ffn_amd")
pytestmark = pytest.mark.gpu
DEV = "cuda"


def lcfg(wl):
    return beam.LayerCfg(wl.hidden, wl.n_experts, wl.n_groups, wl.topk_groups, wl.topk,
                         wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)


# ------------------------------------------------------------------ route

@pytest.mark.parametrize("wname,T", [
    ("tiny_fp32", 1), ("tiny_fp32", 4), ("tiny_fp32", 33),
    ("decode_t8", 1), ("decode_t8", 8), ("decode_t8", 16), ("decode_t8", 17),
    ("skew_t64", 64), ("decode_t8", 300), ("prefill_t2048", 2048), ("decode_t8", 100),
    ("prefill_fp8_t16384", 16384), ("decode_t8", 512), ("decode_t8", 700), ("decode_t8", 1024),
])
def test_route_parity(wname, T):
    say(f"route {wname} T={T}")
    _check_route(synth.WORKLOADS[wname], T)


# The small-batch router (T <= 16) is compiled per chunk count of its K
# slice (1, 2 or 4 chunks of 1024 per thread) and per token batch (8 or
# 16): hidden sizes and token counts that reach each variant, bf16 and fp32.
@pytest.mark.parametrize("wname,H,T", [
    ("decode_t8", 2048, 3), ("decode_t8", 3840, 12), ("decode_t8", 4096, 9), ("decode_t8", 7936, 16),
    ("tiny_fp32", 3840, 5), ("tiny_fp32", 1024, 16), ("tiny_fp32", 4352, 11),
])
def test_route_small_batch_shapes(wname, H, T):
    say(f"route {wname} H={H} T={T}")
    _check_route(dataclasses.replace(synth.WORKLOADS[wname], hidden=H), T)


# The matrix-core router cuts K into as many slices as fill the chip (each a
# multiple of 32 values that divides H, at least 256): hidden sizes whose
# slice counts differ (9 slices of 256 at H=2304 and T=600, 5 at H=1280 and
# T=1000, 1 at T=16384 above) with ragged token tiles.
@pytest.mark.parametrize("H,T", [(2304, 600), (1280, 1000), (5120, 1500)])
def test_route_split_k_shapes(H, T):
    say(f"route split-K H={H} T={T}")
    _check_route(dataclasses.replace(synth.WORKLOADS["decode_t8"], hidden=H), T)


def _check_route(wl, T):
    cfg = lcfg(wl)
    w_r, bias = synth.make_router(wl, DEV)
    x, _, _, _ = synth.make_activations(wl, DEV, T=T)
    ids = torch.empty((T, wl.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((T, wl.topk), dtype=torch.float32, device=DEV)
    logits = torch.empty((T, wl.n_experts), dtype=torch.float32, device=DEV)
    beam.beam_moe_route(cfg, x, w_r, bias, ids, w, logits, ws=beam.workspace(cfg, T, beam.BEAM_BF16))
    torch.cuda.synchronize()
    ref = oracle.router_logits(synth.to_f64(x), synth.to_f64(w_r))
    got = logits.cpu().double().numpy()
    err = np.max(np.abs(got - ref)) / max(1.0, np.max(np.abs(ref)))
    say(f"  logits max err {err:.2e}")
    # The selection is decided on b = sigmoid(logit) + bias (~28).  A token
    # whose fp64 gap is >= 1e-6 relative (2.8e-5 absolute) must get the
    # oracle's experts; that holds while the fp32 error of b (rounding,
    # ~1e-6, plus a quarter of the logit error) stays below 1.4e-5, i.e.
    # for logit errors below ~5e-5.  Ask for 5x headroom.
    assert err < 1e-5
    routes = oracle.route(ref, synth.to_f64(bias), oracle_cfg(wl))
    check_routes(ids.cpu().numpy(), w.cpu().numpy(), routes, oracle_cfg(wl))


@pytest.mark.parametrize("T", [8, 64, 2048])
def test_route_without_logits_output_uses_workspace(T):
    wl = synth.WORKLOADS["decode_t8"].with_T(T)
    cfg = lcfg(wl)
    w_r, bias = synth.make_router(wl, DEV)
    x, _, _, _ = synth.make_activations(wl, DEV)
    ids = torch.empty((wl.T, wl.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((wl.T, wl.topk), dtype=torch.float32, device=DEV)
    ids2, w2 = torch.empty_like(ids), torch.empty_like(w)
    lg = torch.empty((wl.T, wl.n_experts), dtype=torch.float32, device=DEV)
    ws = beam.workspace(cfg, wl.T, beam.BEAM_BF16)
    beam.beam_moe_route(cfg, x, w_r, bias, ids, w, lg, ws=ws)
    beam.beam_moe_route(cfg, x, w_r, bias, ids2, w2, None, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2) and torch.equal(w, w2)


# ------------------------------------------------------------------ permute

def _perm_cfg(E, K):
    if E == 16:
        return beam.LayerCfg(256, 16, 4, 2, K, 2, 128)
    return beam.LayerCfg(topk=K)


def _run_permute(ids_np, E, K):
    T = ids_np.shape[0]
    cfg = _perm_cfg(E, K)
    ids = torch.from_numpy(ids_np.astype(np.int32)).to(DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    rt = torch.empty(T * K, dtype=torch.int32, device=DEV)
    pr = torch.empty(T * K, dtype=torch.int32, device=DEV)
    beam.beam_moe_permute(cfg, ids, off, rt, pr, ws=beam.workspace(cfg, T, beam.BEAM_BF16))
    torch.cuda.synchronize()
    return off.cpu().numpy(), rt.cpu().numpy(), pr.cpu().numpy()


@pytest.mark.parametrize("T,E,K,skew", [
    (1, 16, 4, 0.0), (37, 16, 4, 3.0), (8, 256, 8, 0.0), (64, 256, 8, 1.1), (511, 256, 8, 0.0),
    (512, 256, 8, 0.0), (513, 256, 8, 2.0), (2048, 256, 8, 0.0), (16384, 256, 8, 0.0),
    # multi-block path: 32 and 33 chunks of 1024 pairs, ragged, skewed
    (4096, 256, 8, 1.5), (4097, 256, 8, 0.0), (1000, 256, 8, 3.0),
])
def test_permute_parity(T, E, K, skew):
    say(f"permute T={T} E={E} K={K} skew={skew}")
    ids = synth.random_ids(T, E, K, skew=skew).numpy()
    off, rt, pr = _run_permute(ids, E, K)
    o_off, o_rt, o_pr = oracle.permutation(ids, E)
    assert np.array_equal(off, o_off)
    assert np.array_equal(rt, o_rt)
    assert np.array_equal(pr, o_pr)


def test_permute_every_token_on_one_expert():
    rng = np.random.default_rng(11)
    T, E, K = 1500, 256, 8
    others = np.array([e for e in range(E) if e != 5])
    ids = np.stack([np.concatenate([[5], rng.choice(others, K - 1, replace=False)]) for _ in range(T)])
    ids = np.ascontiguousarray(ids[:, rng.permutation(K)])
    off, rt, pr = _run_permute(ids, E, K)
    o_off, o_rt, o_pr = oracle.permutation(ids, E)
    assert off[6] - off[5] == T
    assert np.array_equal(off, o_off) and np.array_equal(rt, o_rt) and np.array_equal(pr, o_pr)


# hidden sizes that fill the quantiser's chunks exactly (5120) or leave
# lanes past the row (1280, 3328)
@pytest.mark.parametrize("H", [5120, 1280, 3328])
def test_quantize_x_e4m3_bit_exact(H):
    say(f"per-token e4m3 quantisation H={H}")
    T = 37
    g = torch.Generator(device=DEV).manual_seed(3)
    scale = torch.logspace(-3, 3, T, device=DEV).unsqueeze(1)
    x = (torch.randn((T, H), generator=g, device=DEV) * scale)
    x[5] = 0.0                                           # all-zero row
    x[6] = x[6] * torch.logspace(-6, 0, H, device=DEV)   # wide dynamic range -> e4m3 subnormals
    x = x.to(torch.bfloat16)
    cfg = beam.LayerCfg(hidden=H)
    ids = torch.zeros((T, cfg.topk), dtype=torch.int32, device=DEV) + torch.arange(cfg.topk, dtype=torch.int32, device=DEV)
    off = torch.empty(cfg.n_experts + 1, dtype=torch.int32, device=DEV)
    rt = torch.empty(T * cfg.topk, dtype=torch.int32, device=DEV)
    pr = torch.empty_like(rt)
    xq = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    xs = torch.empty(T, dtype=torch.float32, device=DEV)
    beam.beam_moe_permute(cfg, ids, off, rt, pr, x=x, x_q=xq, x_scale=xs)
    # the stand-alone entry point (the one a second stream runs beside the
    # router) writes the same codes and scales
    xq2, xs2 = torch.empty_like(xq), torch.empty_like(xs)
    beam.beam_moe_quantize_fp8(cfg, x, xq2, xs2)
    torch.cuda.synchronize()
    assert torch.equal(xq2, xq) and torch.equal(xs2, xs)
    xn = synth.to_f64(x)
    q_gpu = oracle.e4m3_decode(xq.cpu().numpy())
    s_gpu = xs.cpu().double().numpy()
    for t in range(T):
        s, q = oracle.quantize_row_e4m3(xn[t])
        assert s_gpu[t] == s, (t, s_gpu[t], s)
        assert np.array_equal(q_gpu[t], q), (t, np.flatnonzero(q_gpu[t] != q)[:8])


# ------------------------------------------------------------------ experts

def _stage_wl(w_dtype, H=512, F=256, E=16, K=4):
    return synth.Workload("stage", T=1, hidden=H, n_experts=E, n_groups=4, topk_groups=2, topk=K,
                          group_topn=2, d_ff=F, routed_scale=2.5, rms_eps=1e-6, n=20,
                          act_dtype="f32" if w_dtype == "f32" else "bf16", w_dtype=w_dtype,
                          bias_sigma=0.02, seed=7)


def _run_experts_stage(wl, T, ids_np, y_dtype):
    cfg = lcfg(wl)
    E, K = wl.n_experts, wl.topk
    wgu, wd, sgu, sd = synth.make_expert_stacks(wl, DEV)
    pgu, pd = torch.empty_like(wgu), torch.empty_like(wd)
    mx = wl.w_dtype == "mxfp4"
    beam.beam_moe_pack_weights(cfg, wgu, wd, pgu, pd, mxfp4=mx)
    x, _, _, _ = synth.make_activations(wl, DEV, T=T)
    o_off, o_rt, _ = oracle.permutation(ids_np, E)
    off = torch.from_numpy(o_off.astype(np.int32)).to(DEV)
    rt = torch.from_numpy(o_rt.astype(np.int32)).to(DEV)
    y = torch.empty((T * K, wl.hidden), dtype=y_dtype, device=DEV)
    ws = beam.workspace(cfg, T, beam.BEAM_MXFP4 if mx else beam._dt(wgu))
    if mx:
        xq = torch.empty((T, wl.hidden // 2), dtype=torch.uint8, device=DEV)
        xs = torch.empty((T, wl.hidden // 32), dtype=torch.uint8, device=DEV)
        beam.beam_moe_quantize_mx(cfg, x, xq, xs)
        beam.beam_moe_experts(cfg, T, xq, off, rt, pgu, pd, y, x_scale=xs, s_gate_up=sgu, s_down=sd, ws=ws)
    elif wl.w_dtype == "fp8":
        xq = torch.empty((T, wl.hidden), dtype=torch.uint8, device=DEV)
        xs = torch.empty(T, dtype=torch.float32, device=DEV)
        ids = torch.from_numpy(ids_np.astype(np.int32)).to(DEV)
        tmp = [torch.empty(n, dtype=torch.int32, device=DEV) for n in (E + 1, T * K, T * K)]
        beam.beam_moe_permute(cfg, ids, *tmp, x=x, x_q=xq, x_scale=xs, ws=ws)
        beam.beam_moe_experts(cfg, T, xq, off, rt, pgu, pd, y, x_scale=xs, s_gate_up=sgu, s_down=sd, ws=ws)
    else:
        beam.beam_moe_experts(cfg, T, x, off, rt, pgu, pd, y, ws=ws)
    torch.cuda.synchronize()
    got = y.cpu().double().numpy()
    xn = synth.to_f64(x)
    ref = np.empty_like(got)
    for e in range(E):
        lo, hi = int(o_off[e]), int(o_off[e + 1])
        if lo == hi:
            continue
        u = xn[o_rt[lo:hi]]
        if wl.w_dtype == "fp8":
            ref[lo:hi] = oracle.expert_ffn_w8a8(u, wgu[e].cpu().numpy(), synth.to_f64(sgu[e]),
                                                wd[e].cpu().numpy(), synth.to_f64(sd[e]))
        elif mx:
            ref[lo:hi] = oracle.expert_ffn_w4a4(u, oracle.unpack_fp4(wgu[e].cpu().numpy()), sgu[e].cpu().numpy(),
                                                oracle.unpack_fp4(wd[e].cpu().numpy()), sd[e].cpu().numpy())
        else:
            rnd = oracle.round_f32 if wl.w_dtype == "f32" else oracle.round_bf16
            ref[lo:hi] = oracle.expert_ffn(u, synth.to_f64(wgu[e]), synth.to_f64(wd[e]), round_a=rnd)
    return got, ref


@pytest.mark.parametrize("w_dtype,y_dtype,T,skew", [
    ("bf16", torch.float32, 5, 0.0),      # <= 16 tokens: one row block per item
    ("bf16", torch.float32, 300, 0.5),    # 128-row items, ragged tails, 2+ items per expert
    ("bf16", torch.bfloat16, 300, 0.5),
    ("bf16", torch.float32, 37, 3.0),     # heavy skew: empty experts
    ("fp8", torch.float32, 5, 0.0),
    ("fp8", torch.float32, 300, 0.5),
    ("fp8", torch.bfloat16, 300, 0.5),
    ("f32", torch.float32, 33, 0.5),
    # >= 256 rows per expert on average (T*K >= 256*E): the wide-tile kernel
    # with 256-row items (rows 128..255 included), several per expert, and
    # ragged last items
    ("bf16", torch.float32, 1500, 0.5),
    ("bf16", torch.bfloat16, 1100, 2.0),
    ("fp8", torch.float32, 1500, 0.5),
    ("fp8", torch.bfloat16, 1100, 2.0),
])
def test_experts_parity(w_dtype, y_dtype, T, skew):
    say(f"experts {w_dtype} y={y_dtype} T={T} skew={skew}")
    wl = _stage_wl(w_dtype, H=256 if w_dtype == "f32" else 512, F=128 if w_dtype == "f32" else 256)
    ids = synth.random_ids(T, wl.n_experts, wl.topk, skew=skew).numpy()
    got, ref = _run_experts_stage(wl, T, ids, y_dtype)
    kind = {"bf16": "bf16", "fp8": "fp8", "f32": "f32"}[w_dtype]
    if y_dtype == torch.bfloat16 and kind == "f32":
        kind = "bf16"
    check_output("y", got, ref, kind)
    if kind == "bf16":
        assert rel_l2(got, ref) < 2e-3


@pytest.mark.parametrize("y_dtype,T,skew", [
    (torch.float32, 5, 0.0),       # <= 16 tokens: the direct kernel
    (torch.bfloat16, 12, 0.0),
    (torch.float32, 300, 0.5),     # 128-row items staged in LDS, ragged tails
    (torch.float32, 37, 3.0),      # heavy skew, empty experts
    (torch.float32, 1500, 0.5),    # >= 256 rows per expert: the wide-tile kernel
    (torch.bfloat16, 1100, 2.0),
])
def test_experts_mxfp4_parity(y_dtype, T, skew):
    say(f"experts mxfp4 y={y_dtype} T={T} skew={skew}")
    wl = _stage_wl("mxfp4", H=512, F=512)
    ids = synth.random_ids(T, wl.n_experts, wl.topk, skew=skew).numpy()
    got, ref = _run_experts_stage(wl, T, ids, y_dtype)
    check_output("y", got, ref, "mx")


def test_quantize_mx_bit_exact():
    say("run-time MXFP4 quantisation of x")
    T, H = 37, 5120
    g = torch.Generator(device=DEV).manual_seed(5)
    scale = torch.logspace(-3, 3, T, device=DEV).unsqueeze(1)
    x = torch.randn((T, H), generator=g, device=DEV) * scale
    x[5] = 0.0                                             # all-zero row
    x[6] = x[6] * torch.logspace(-6, 0, H, device=DEV)     # wide range inside a row
    x[7, :32] = 0.0                                        # one all-zero block
    # E2M1 ties: block max 6 * 2^-1 = 3 (scale 2^-1), then ties at 0.25, 0.75, ... x 2^-1
    x[8, :32] = torch.tensor([3.0] + [0.125, 0.375, 0.625, 0.875, 1.25, 1.75, 2.5] * 4 + [0.0] * 3, device=DEV)
    for xdt in (torch.bfloat16, torch.float32):
        xx = x.to(xdt)
        cfg = beam.LayerCfg()
        xq = torch.empty((T, H // 2), dtype=torch.uint8, device=DEV)
        xs = torch.empty((T, H // 32), dtype=torch.uint8, device=DEV)
        beam.beam_moe_quantize_mx(cfg, xx, xq, xs)
        torch.cuda.synchronize()
        s_o, q_o = oracle.quantize_mx_fp4(synth.to_f64(xx))
        np.testing.assert_array_equal(xs.cpu().numpy(), s_o)
        np.testing.assert_array_equal(oracle.unpack_fp4(xq.cpu().numpy()), oracle.e2m1_encode(q_o))


def test_quantizers_special_values():
    # the documented handling of NaN and infinite inputs by the run-time
    # quantisers (include/beam_moe.h): e4m3 -- NaN stays out of the row
    # maximum and gets a NaN code, an infinite element makes the scale
    # infinite, the row's finite elements code 0 and the infinite ones NaN;
    # MXFP4 -- NaN and +-Inf are stored as +-6
    say("quantisers on NaN and infinite inputs")
    T, H = 4, 5120
    g = torch.Generator(device=DEV).manual_seed(9)
    x = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
    x[0, 17] = float("nan")
    x[0, 4000] = -float("nan")
    x[1, 5] = float("inf")
    x[2, 3000] = -float("inf")
    cfg = beam.LayerCfg()
    xq = torch.empty((T, H), dtype=torch.uint8, device=DEV)
    xs = torch.empty(T, dtype=torch.float32, device=DEV)
    beam.beam_moe_quantize_fp8(cfg, x, xq, xs)
    mq = torch.empty((T, H // 2), dtype=torch.uint8, device=DEV)
    ms = torch.empty((T, H // 32), dtype=torch.uint8, device=DEV)
    beam.beam_moe_quantize_mx(cfg, x, mq, ms)
    torch.cuda.synchronize()
    xn = synth.to_f64(x)
    codes = xq.cpu().numpy()
    q_gpu = oracle.e4m3_decode(codes)
    s_gpu = xs.cpu().double().numpy()
    # row 0: scale and codes of the row without its NaN elements
    nan_at = [17, 4000]
    clean = np.delete(xn[0], nan_at)
    s0, q0 = oracle.quantize_row_e4m3(clean)
    assert s_gpu[0] == s0
    assert np.array_equal(np.delete(q_gpu[0], nan_at), q0)
    assert all(np.isnan(q_gpu[0, i]) for i in nan_at)
    # rows 1 and 2: infinite scale, finite elements 0, the infinite one NaN
    for t, i in ((1, 5), (2, 3000)):
        assert np.isinf(s_gpu[t])
        assert np.isnan(q_gpu[t, i])
        assert np.all(np.delete(q_gpu[t], i) == 0.0)
    # row 3 is ordinary
    s3, q3 = oracle.quantize_row_e4m3(xn[3])
    assert s_gpu[3] == s3 and np.array_equal(q_gpu[3], q3)
    # MXFP4: the special elements hold the code of +-6, the other blocks of
    # the rows are the oracle's
    c = oracle.unpack_fp4(mq.cpu().numpy())
    vals = oracle.e2m1_decode(c)
    bits = x.view(torch.int16).cpu().numpy()   # the sign bit as stored (a NaN's too)
    for t, i in ((0, 17), (0, 4000), (1, 5), (2, 3000)):
        sign = -1.0 if bits[t, i] < 0 else 1.0
        assert vals[t, i] == 6.0 * sign, (t, i, vals[t, i])
    s_o, q_o = oracle.quantize_mx_fp4(xn[3:4])
    assert np.array_equal(ms.cpu().numpy()[3:4], s_o)
    assert np.array_equal(c[3:4], oracle.e2m1_encode(q_o))
    special_blocks = {(0, 17 // 32), (0, 4000 // 32), (1, 5 // 32), (2, 3000 // 32)}
    for t in range(3):
        for b in range(H // 32):
            if (t, b) in special_blocks:
                continue
            s_b, q_b = oracle.quantize_mx_fp4(xn[t:t + 1, 32 * b:32 * b + 32])
            assert ms.cpu().numpy()[t, b] == s_b[0, 0], (t, b)
            assert np.array_equal(c[t, 32 * b:32 * b + 32], oracle.e2m1_encode(q_b)[0]), (t, b)


def test_experts_every_token_on_one_expert():
    say("experts: 150 rows on one expert (items of 128 + 22 rows)")
    wl = _stage_wl("bf16", H=512, F=256)
    rng = np.random.default_rng(12)
    T, E, K = 150, wl.n_experts, wl.topk
    others = np.array([e for e in range(E) if e != 3])
    ids = np.stack([np.concatenate([[3], rng.choice(others, K - 1, replace=False)]) for _ in range(T)])
    got, ref = _run_experts_stage(wl, T, ids, torch.float32)
    check_output("y", got, ref, "bf16")


@pytest.mark.parametrize("w_dtype,E,G,T,case", [
    ("bf16", 6, 3, 5, "ends"),      # E not a multiple of 4 (a lane's last experts are past E)
    ("bf16", 6, 3, 16, "one"),      # every token on the last expert: one 16-row item
    ("fp8", 12, 3, 9, "ends"),
    ("mxfp4", 6, 3, 3, "ends"),
])
def test_experts_direct_items(w_dtype, E, G, T, case):
    # At T <= 16 each wave finds its item (the i-th touched expert) in the
    # offsets; cover the first and last expert, untouched experts between,
    # and expert counts that do not fill a lane's four slots
    say(f"experts direct items {w_dtype} E={E} T={T} {case}")
    K = 2
    wl = synth.Workload("stage", T=1, hidden=512, n_experts=E, n_groups=G, topk_groups=G, topk=K,
                        group_topn=1, d_ff=512 if w_dtype == "mxfp4" else 256, routed_scale=2.5, rms_eps=1e-6,
                        n=20, act_dtype="bf16", w_dtype=w_dtype, bias_sigma=0.02, seed=11)
    if case == "ends":
        ids = np.array([[0, E - 1] if t % 2 == 0 else [E - 1, 1 + t % (E - 2)] for t in range(T)])
    else:
        ids = np.array([[E - 1, t % (E - 1)] for t in range(T)])
    got, ref = _run_experts_stage(wl, T, ids, torch.float32)
    check_output("y", got, ref, {"bf16": "bf16", "fp8": "fp8", "mxfp4": "mx"}[w_dtype])


def test_experts_beam_shape_few_tokens():
    say("experts: Beam shape, bf16, T=3")
    wl = synth.WORKLOADS["decode_t8"]
    small = synth.Workload("beam_e8", T=3, hidden=5120, n_experts=8, n_groups=8, topk_groups=4, topk=4,
                           group_topn=1, d_ff=2560, routed_scale=2.5, rms_eps=1e-6, n=20,
                           act_dtype="bf16", w_dtype="bf16", bias_sigma=0.02, seed=wl.seed)
    ids = np.array([[0, 1, 2, 3], [3, 4, 5, 6], [7, 0, 3, 5]])
    got, ref = _run_experts_stage(small, 3, ids, torch.float32)
    check_output("y", got, ref, "bf16")


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8", "f32"])
def test_pack_layout(w_dtype):
    # packed tile (row block rb, 256-byte chunk c) = [piece s][lane r+16g][16 B]
    # holding bytes [256c + 64s + 16g, +16) of row 16rb + r
    say(f"pack layout {w_dtype}")
    wl = _stage_wl(w_dtype, H=512 if w_dtype != "f32" else 256, F=256 if w_dtype != "f32" else 128, E=4)
    cfg = lcfg(wl)
    wgu, wd, _, _ = synth.make_expert_stacks(wl, DEV)
    pgu, pd = torch.empty_like(wgu), torch.empty_like(wd)
    beam.beam_moe_pack_weights(cfg, wgu, wd, pgu, pd)
    torch.cuda.synchronize()
    for src, dst in ((wgu, pgu), (wd, pd)):
        a = src.cpu().contiguous().view(torch.uint8).numpy().reshape(src.shape[0], src.shape[1], -1)
        b = dst.cpu().contiguous().view(torch.uint8).numpy().reshape(-1)
        if w_dtype == "f32":
            assert np.array_equal(a.reshape(-1), b)
            continue
        E, R, KB = a.shape
        ref = a.reshape(E, R // 16, 16, KB // 256, 4, 4, 16)          # e, rb, r, c, s, g, byte
        ref = ref.transpose(0, 1, 3, 4, 5, 2, 6).reshape(-1)          # e, rb, c, s, g, r, byte
        assert np.array_equal(ref, b)


# ------------------------------------------------------------------ combine + norm

@pytest.mark.parametrize("H,K,T,y_dtype,act,n", [
    (5120, 8, 37, torch.float32, "bf16", 20),      # up to 256 tokens: all K rows per load batch
    (5120, 8, 37, torch.bfloat16, "bf16", 20),
    (5120, 8, 3, torch.float32, "bf16", 1),
    (256, 4, 4, torch.float32, "f32", 5),
    (5120, 8, 300, torch.float32, "bf16", 20),     # more tokens: one row at a time
    (5120, 8, 300, torch.bfloat16, "bf16", 20),
    # rows that end part-way through a thread's chunks, on both load paths
    (1280, 8, 300, torch.bfloat16, "bf16", 20),
    (1280, 8, 300, torch.float32, "f32", 7),
    (3328, 6, 5, torch.float32, "bf16", 3),
])
def test_combine_norm_parity(H, K, T, y_dtype, act, n):
    say(f"combine_norm H={H} K={K} T={T} y={y_dtype} act={act} n={n}")
    cfg = beam.LayerCfg(hidden=H, topk=K) if H != 256 else beam.LayerCfg(256, 16, 4, 2, K, 2, 128)
    g = torch.Generator(device=DEV).manual_seed(21)
    TK = T * K
    adt = torch.bfloat16 if act == "bf16" else torch.float32
    y = (torch.randn((TK, H), generator=g, device=DEV) * 0.6).to(y_dtype)
    pair_row = torch.randperm(TK, generator=g, device=DEV).to(torch.int32)
    w = torch.rand((T, K), generator=g, device=DEV) + 0.05
    w = (w / w.sum(dim=1, keepdim=True) * 2.5).contiguous()
    h = torch.randn((T, H), generator=g, device=DEV).to(adt)
    gp = (1 + 0.1 * torch.randn(H, generator=g, device=DEV)).to(adt)
    gq = (1 + 0.1 * torch.randn(H, generator=g, device=DEV)).to(adt)
    h_dev = h.clone()
    xn = torch.empty_like(h)
    m = torch.empty((T, H), dtype=torch.float32, device=DEV)
    beam.beam_moe_combine_norm(cfg, y, pair_row, w, h_dev, xn, gp, gq, n, moe_out=m)
    torch.cuda.synchronize()
    yn, prn, wn = synth.to_f64(y), pair_row.cpu().numpy(), synth.to_f64(w)
    hn, gpn, gqn = synth.to_f64(h), synth.to_f64(gp), synth.to_f64(gq)
    rnd = oracle.round_bf16 if act == "bf16" else oracle.round_f32
    ms, hs, xs = [], [], []
    for t in range(T):
        mt = oracle.combine(yn[prn[t * K:(t + 1) * K]], wn[t])
        _, ht, xt = oracle.norm_boundary(mt, hn[t], gpn, gqn, n, 1e-6, rnd=rnd)
        ms.append(mt); hs.append(ht); xs.append(xt)
    kind = "bf16" if act == "bf16" else "f32"
    check_output("m", m.cpu().double().numpy(), np.array(ms), "f32")
    check_output("h_new", h_dev.cpu().double().numpy(), np.array(hs), kind)
    check_output("x_next", xn.cpu().double().numpy(), np.array(xs), kind)
