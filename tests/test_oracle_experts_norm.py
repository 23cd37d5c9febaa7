"""Pins of the oracle's expert MLP, fp8 (W8A8) expert, combine and norm
boundary: hand-derived closed forms, a torch-library dense SwiGLU, the
identical-experts invariant of the whole layer, the unit-variance property
of the depth-scaled residual, and exactness of W8A8 where quantisation is
lossless."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ident(v):
    return np.asarray(v, np.float64)


def test_swiglu_hand_example_gate_up_order():
    # H=2, F=1: u=[1,2]; gate row [1,0] -> g=1; up row [0,1] -> v=2;
    # a = silu(1)*2 = 2*sigmoid(1); down [[1],[3]] -> y = [a, 3a].
    # Swapping gate and up would give silu(2)*1 instead.
    w_gu = np.array([[1.0, 0.0], [0.0, 1.0]])
    w_d = np.array([[1.0], [3.0]])
    y = oracle.expert_ffn(np.array([1.0, 2.0]), w_gu, w_d, round_a=None)[0]
    a = 2.0 / (1.0 + math.exp(-1.0))
    assert abs(y[0] - a) < 1e-15 and abs(y[1] - 3 * a) < 1e-15
    assert abs(a - 1.4621171572600098) < 1e-15


def test_expert_matches_torch_dense_swiglu():
    rng = np.random.default_rng(0)
    H, F, m = 96, 40, 5
    u = rng.standard_normal((m, H))
    w_gu = rng.standard_normal((2 * F, H)) / math.sqrt(H)
    w_d = rng.standard_normal((H, F)) / math.sqrt(F)
    got = oracle.expert_ffn(u, w_gu, w_d, round_a=None)
    lin = torch.nn.functional.linear
    tu = torch.from_numpy(u)
    ref = lin(torch.nn.functional.silu(lin(tu, torch.from_numpy(w_gu[:F]))) * lin(tu, torch.from_numpy(w_gu[F:])),
              torch.from_numpy(w_d)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_expert_rounds_a_to_bf16():
    rng = np.random.default_rng(1)
    H, F = 64, 32
    u = rng.standard_normal(H)
    w_gu = rng.standard_normal((2 * F, H)) / 8
    w_d = np.eye(H, F)          # y[:F] = a exactly
    y = oracle.expert_ffn(u, w_gu, w_d)[0]
    ref = torch.from_numpy(oracle.expert_ffn(u, w_gu, w_d, round_a=None)[0][:F].astype(np.float32)).to(torch.bfloat16)
    # a from fp64 vs a from fp32 -> bf16 agree except at (vanishingly rare) double-rounding cases
    np.testing.assert_array_equal(y[:F], ref.to(torch.float64).numpy())


def test_w8a8_exact_when_quantisation_is_lossless():
    # u has entries on the e4m3 grid and amax 448 -> activation scale 1, codes = u.
    # Every gate row equal and every up row equal -> a is constant over F, so
    # its quantisation maps every entry to +-448 exactly.  Then the W8A8
    # expert must equal the float expert on the decoded weights up to the
    # fp32 rounding of the scale of a.
    rng = np.random.default_rng(2)
    H, F = 64, 32
    grid = oracle.e4m3_decode(np.arange(0, 126))
    u = rng.choice(grid, H) * rng.choice([-1, 1], H)
    u[7] = 448.0
    qg = rng.integers(0, 0x7E, H)
    qu = rng.integers(0, 0x7E, H) | (rng.integers(0, 2, H) << 7)
    q_gu = np.concatenate([np.tile(qg, (F, 1)), np.tile(qu, (F, 1))]).astype(np.uint8)
    s_gu = np.concatenate([np.full(F, 2.0 ** -12), np.full(F, 2.0 ** -11)])
    q_d = rng.integers(0, 0xFE, (H, F)).astype(np.uint8)
    q_d[(q_d & 0x7F) == 0x7F] = 0x10
    s_d = rng.uniform(1e-3, 2e-3, H).astype(np.float32).astype(np.float64)
    y8 = oracle.expert_ffn_w8a8(u, q_gu, s_gu, q_d, s_d)[0]
    w_gu = oracle.e4m3_decode(q_gu) * s_gu[:, None]
    w_d = oracle.e4m3_decode(q_d) * s_d[:, None]
    yf = oracle.expert_ffn(u, w_gu, w_d, round_a=None)[0]
    np.testing.assert_allclose(y8, yf, rtol=1e-7, atol=1e-12 * np.abs(yf).max())


def test_w8a8_floor_against_full_precision():
    # quantisation error of W8A8 relative to the unquantised expert: a few percent, not more
    rng = np.random.default_rng(3)
    H, F = 512, 256
    u = rng.standard_normal((4, H))
    w_gu = rng.standard_normal((2 * F, H)) / math.sqrt(H)
    w_d = rng.standard_normal((H, F)) / math.sqrt(F)

    def q(w):
        s = np.abs(w).max(axis=1) / 448.0
        codes = torch.from_numpy((w / s[:, None]).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return codes, s.astype(np.float32).astype(np.float64)

    qgu, sgu = q(w_gu)
    qd, sd = q(w_d)
    y8 = oracle.expert_ffn_w8a8(u, qgu, sgu, qd, sd)
    yf = oracle.expert_ffn(u, w_gu, w_d, round_a=None)
    rel = np.linalg.norm(y8 - yf) / np.linalg.norm(yf)
    assert 1e-3 < rel < 0.08, rel


def test_combine_is_weighted_sum():
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0]])
    np.testing.assert_array_equal(oracle.combine(y, [0.5, 0.25, 2.0]), [203.0, 406.0])


def test_norm_boundary_hand_golden():
    g = json.load(open(os.path.join(GOLDEN, "norm_hand.json")))
    p, hn, xn = oracle.norm_boundary(np.array(g["m"]), np.array(g["h"]), np.ones(4), np.ones(4),
                                     g["n"], 0.0, rnd=ident)
    np.testing.assert_allclose(p, g["p"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(hn, g["h_new"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(xn, g["x_next"], rtol=0, atol=1e-15)


def test_norm_first_residual_is_post_norm_output():
    rng = np.random.default_rng(4)
    m, h = rng.standard_normal(64), rng.standard_normal(64)
    gp, gq = 1 + 0.1 * rng.standard_normal(64), 1 + 0.1 * rng.standard_normal(64)
    p, hn, _ = oracle.norm_boundary(m, h, gp, gq, 1, 1e-6)
    np.testing.assert_array_equal(hn, p)


def test_rmsnorm_constant_vector_and_scale_invariance():
    v = np.full(10, -3.0)
    np.testing.assert_allclose(oracle.rmsnorm(v, np.ones(10), 1e-6), -3.0 / math.sqrt(9.0 + 1e-6), rtol=1e-15)
    rng = np.random.default_rng(5)
    m = rng.standard_normal(512)
    np.testing.assert_allclose(oracle.rmsnorm(7.5 * m, np.ones(512), 0.0), oracle.rmsnorm(m, np.ones(512), 0.0), rtol=1e-13)
    # RMS of the gamma=1 output is 1 (eps=0)
    r = oracle.rmsnorm(m, np.ones(512), 0.0)
    assert abs(np.sqrt(np.mean(r * r)) - 1) < 1e-14
    # gamma multiplies per channel
    gm = rng.uniform(0.5, 2, 512)
    np.testing.assert_allclose(oracle.rmsnorm(m, gm, 0.0), r * gm, rtol=1e-14)


def test_residual_update_keeps_unit_variance():
    # independent unit-variance h and sublayer output: the depth-scaled update
    # keeps mean(h'^2) at 1 for every n (no rounding, gamma = 1).
    rng = np.random.default_rng(6)
    H = 1 << 16
    for n in (2, 5, 20, 104):
        h = rng.standard_normal(H)
        m = rng.standard_normal(H)
        _, hn, _ = oracle.norm_boundary(m, h, np.ones(H), np.ones(H), n, 0.0, rnd=ident)
        assert abs(np.mean(hn * hn) - 1.0) < 4 * math.sqrt(2.0 / H) + 1e-3, (n, np.mean(hn * hn))
        # exact identity before rounding: |h'|^2 = (n-1)/n |h|^2 + |p|^2/n + 2 sqrt(n-1)/n <h,p>
        p = m / np.sqrt(np.mean(m * m))
        lhs = np.dot(hn, hn)
        rhs = (n - 1) / n * np.dot(h, h) + np.dot(p, p) / n + 2 * math.sqrt(n - 1) / n * np.dot(h, p)
        assert abs(lhs - rhs) < 1e-9 * lhs


def _tiny_inputs():
    wl = synth.WORKLOADS["tiny_fp32"]
    cfg = dict(n_experts=wl.n_experts, n_groups=wl.n_groups, topk_groups=wl.topk_groups, topk=wl.topk,
               group_topn=wl.group_topn, routed_scale=wl.routed_scale, hidden=wl.hidden, d_ff=wl.d_ff,
               rms_eps=wl.rms_eps)
    w_r, bias = synth.make_router(wl)
    x, h, gp, gq = synth.make_activations(wl)
    return wl, cfg, w_r, bias, x, h, gp, gq


def test_layer_identical_experts_gives_scaled_single_ffn():
    # all experts equal -> m = 2.5 * FFN(x) for any routing (weights sum to 2.5)
    wl, cfg, w_r, bias, x, h, gp, gq = _tiny_inputs()
    w_gu, w_d, _, _ = synth.make_expert(wl, 3)
    w_gu, w_d = synth.to_f64(w_gu), synth.to_f64(w_d)
    out = oracle.layer_tokens(cfg, synth.to_f64(x), synth.to_f64(w_r), synth.to_f64(bias),
                              lambda e: {"w_gu": w_gu, "w_d": w_d}, synth.to_f64(h), synth.to_f64(gp),
                              synth.to_f64(gq), wl.n, rnd=ident)
    ref = 2.5 * oracle.expert_ffn(synth.to_f64(x), w_gu, w_d, round_a=None)
    np.testing.assert_allclose(out["m"], ref, rtol=1e-12, atol=1e-12)


def test_layer_outputs_are_per_token():
    # evaluating a subset of tokens gives the same rows as the full batch
    wl, cfg, w_r, bias, x, h, gp, gq = _tiny_inputs()
    experts = {e: synth.make_expert(wl, e) for e in range(wl.n_experts)}
    ew = lambda e: {"w_gu": synth.to_f64(experts[e][0]), "w_d": synth.to_f64(experts[e][1])}
    args = (cfg, synth.to_f64(x), synth.to_f64(w_r), synth.to_f64(bias), ew, synth.to_f64(h),
            synth.to_f64(gp), synth.to_f64(gq), wl.n)
    full = oracle.layer_tokens(*args, rnd=oracle.round_f32)
    sub = oracle.layer_tokens(*args, tokens=[2], rnd=oracle.round_f32)
    # fp64 BLAS may sum in another order for another row count: compare to 1e-12
    np.testing.assert_allclose(sub["m"][0], full["m"][2], rtol=1e-12, atol=1e-14)
    assert list(sub["routes"][0].ids) == list(full["routes"][2].ids)


def test_ids_override_equals_bias_forced_selection():
    # The correction bias only decides which experts are picked; the weights
    # use the unbiased scores ([TS] "Architecture").  So overriding a token's
    # experts with a set S must give exactly what the unmodified layer gives
    # when S's experts get +100 bias (which forces S through both the group
    # and the expert stage).  Sizes: tiny layer, 16 experts in 4 groups, keep
    # 2 groups, K = 4; S spans groups 1 and 3 and is not the oracle's choice.
    wl, cfg, w_r, bias, x, h, gp, gq = _tiny_inputs()
    experts = {e: synth.make_expert(wl, e) for e in range(wl.n_experts)}
    ew = lambda e: {"w_gu": synth.to_f64(experts[e][0]), "w_d": synth.to_f64(experts[e][1])}
    xd, wr, b = synth.to_f64(x), synth.to_f64(w_r), synth.to_f64(bias)
    args = (synth.to_f64(h), synth.to_f64(gp), synth.to_f64(gq), wl.n)
    S = [13, 5, 4, 15]
    plain = oracle.layer_tokens(cfg, xd, wr, b, ew, *args, rnd=ident)
    assert set(plain["routes"][1].ids) != set(S)
    over = oracle.layer_tokens(cfg, xd, wr, b, ew, *args, rnd=ident, ids_override={1: S})
    b_forced = b.copy()
    b_forced[S] += 100.0
    forced = oracle.layer_tokens(cfg, xd, wr, b_forced, ew, *args, rnd=ident)
    assert set(forced["routes"][1].ids) == set(S)
    assert list(over["routes"][1].ids) == S
    order = [list(forced["routes"][1].ids).index(e) for e in S]
    np.testing.assert_allclose(over["routes"][1].weights, forced["routes"][1].weights[order], rtol=1e-15)
    for k in ("m", "h_new", "x_next"):
        np.testing.assert_allclose(over[k][1], forced[k][1], rtol=1e-13, atol=1e-13)
    # tokens without an override are untouched
    for t in (0, 2, 3):
        assert list(over["routes"][t].ids) == list(plain["routes"][t].ids)
        np.testing.assert_array_equal(over["m"][t], plain["m"][t])
    # weights still sum to the routed scale and follow the unbiased scores
    w = over["routes"][1].weights
    assert abs(w.sum() - 2.5) < 1e-14
    s = plain["routes"][1].scores[S]
    np.testing.assert_allclose(w / w[0], s / s[0], rtol=1e-14)


def test_w8a8_rows_are_independent():
    # the batched W8A8 evaluation of several rows equals evaluating each row
    # on its own (per-row activation and intermediate scales)
    rng = np.random.default_rng(8)
    H, F = 256, 128
    u = rng.standard_normal((5, H)) * rng.uniform(0.1, 10, (5, 1))
    q_gu = rng.integers(0, 0x7E, (2 * F, H)).astype(np.uint8) | (rng.integers(0, 2, (2 * F, H)) << 7).astype(np.uint8)
    q_d = rng.integers(0, 0x7E, (H, F)).astype(np.uint8)
    s_gu = rng.uniform(1e-4, 1e-3, 2 * F)
    s_d = rng.uniform(1e-4, 1e-3, H)
    full = oracle.expert_ffn_w8a8(u, q_gu, s_gu, q_d, s_d)
    for r in range(5):
        np.testing.assert_array_equal(full[r], oracle.expert_ffn_w8a8(u[r], q_gu, s_gu, q_d, s_d)[0])


def test_dense_layer_matches_torch_swiglu_and_boundary():
    # the dense MLP against torch's own linear / silu at a d_ff several times
    # the hidden size, then the boundary on its output
    rng = np.random.default_rng(9)
    H, F, T = 64, 320, 3
    x = rng.standard_normal((T, H))
    w_gu = rng.standard_normal((2 * F, H)) / math.sqrt(H)
    w_d = rng.standard_normal((H, F)) / math.sqrt(F)
    h = rng.standard_normal((T, H))
    gp, gq = 1 + 0.1 * rng.standard_normal(H), 1 + 0.1 * rng.standard_normal(H)
    cfg = {"rms_eps": 1e-6}
    out = oracle.dense_layer_tokens(cfg, x, w_gu, w_d, h, gp, gq, 3, rnd=ident)
    lin = torch.nn.functional.linear
    tx = torch.from_numpy(x)
    y = lin(torch.nn.functional.silu(lin(tx, torch.from_numpy(w_gu[:F]))) * lin(tx, torch.from_numpy(w_gu[F:])),
            torch.from_numpy(w_d)).numpy()
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-13)
    rms = torch.nn.functional.rms_norm(torch.from_numpy(y), (H,), torch.from_numpy(gp), eps=1e-6).numpy()
    np.testing.assert_allclose(out["p"], rms, rtol=1e-12, atol=1e-13)
    hn = math.sqrt(2 / 3) * h + rms / math.sqrt(3)
    np.testing.assert_allclose(out["h_new"], hn, rtol=1e-12, atol=1e-13)
    xn = torch.nn.functional.rms_norm(torch.from_numpy(hn), (H,), torch.from_numpy(gq), eps=1e-6).numpy()
    np.testing.assert_allclose(out["x_next"], xn, rtol=1e-12, atol=1e-13)


def test_shard_partials_sum_to_the_combine():
    # 8 contiguous shards of 32 experts partition every token's K experts:
    # their partial sums add up to the full combine, a shard without the
    # token's experts contributes zero, and each partial is the combine of
    # exactly its own experts
    rng = np.random.default_rng(10)
    K, H = 8, 16
    for _ in range(20):
        ids = rng.choice(256, K, replace=False)
        w = rng.uniform(0.1, 1, K)
        y = rng.standard_normal((K, H))
        parts = [oracle.combine_shard(y, ids, w, 32 * r, 32) for r in range(8)]
        np.testing.assert_allclose(sum(parts), oracle.combine(y, w), rtol=1e-13, atol=1e-14)
        for r in range(8):
            own = (ids >= 32 * r) & (ids < 32 * r + 32)
            if not own.any():
                assert np.all(parts[r] == 0)
            else:
                np.testing.assert_allclose(parts[r], oracle.combine(y[own], w[own]), rtol=1e-13, atol=1e-14)
