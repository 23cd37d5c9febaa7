"""Pins of the oracle's router, selection and permutation: hand-derived
golden cases, brute-force enumeration of group/expert choices, reductions
to plain top-k, invariants, and a library (stable sort / bincount)
construction of the permutation."""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(wl):
    return dict(n_experts=wl.n_experts, n_groups=wl.n_groups, topk_groups=wl.topk_groups,
                topk=wl.topk, group_topn=wl.group_topn, routed_scale=wl.routed_scale,
                hidden=wl.hidden, d_ff=wl.d_ff, rms_eps=wl.rms_eps)


def _logit(sig):
    sig = np.asarray(sig, np.float64)
    return np.log(sig / (1 - sig))


def test_router_logits_one_hot_reads_expert_rows():
    # x = unit vector i picks column i of the stored [E,H] weight: catches a transposed operand
    rng = np.random.default_rng(0)
    E, H = 16, 24
    w = rng.standard_normal((E, H))
    for i in (0, 5, 23):
        x = np.zeros((1, H))
        x[0, i] = 1.0
        np.testing.assert_array_equal(oracle.router_logits(x, w)[0], w[:, i])
    x = np.zeros((2, H))
    x[0, 3], x[1, 7] = 2.0, -1.0
    got = oracle.router_logits(x, w)
    np.testing.assert_array_equal(got[0], 2.0 * w[:, 3])
    np.testing.assert_array_equal(got[1], -w[:, 7])


def test_sigmoid_silu_match_torch():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(oracle.sigmoid(z), torch.sigmoid(torch.from_numpy(z)).numpy(), rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(oracle.silu(z), torch.nn.functional.silu(torch.from_numpy(z)).numpy(), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("case", range(3))
def test_routing_hand_golden(case):
    c = json.load(open(os.path.join(GOLDEN, "routing_hand.json")))["cases"][case]
    r = oracle.route_token(_logit(c["logit_sigmoids"]), np.array(c["bias"]), c["cfg"])
    assert list(r.ids) == c["ids"]
    np.testing.assert_allclose(r.weights, c["weights"], rtol=1e-12)
    for key in ("margin_group", "margin_expert"):
        exp = c[key]
        got = getattr(r, key)
        if math.isinf(exp):
            assert math.isinf(got)
        else:
            assert abs(got - exp) < 1e-12, (key, got, exp)


def _brute_select(b, cfg):
    """Exhaustive: the chosen group set maximises the summed group scores,
    where each group score is the best sum over `group_topn`-subsets of its
    members; the chosen experts maximise the summed biased score over
    K-subsets of the candidates.  Ties: lexicographically smallest set."""
    E, G = cfg["n_experts"], cfg["n_groups"]
    per = E // G
    gs = []
    for g in range(G):
        best = max(sum(c) for c in itertools.combinations(b[g * per:(g + 1) * per], cfg["group_topn"]))
        gs.append(best)
    best_set, best_val = None, -math.inf
    for gset in itertools.combinations(range(G), cfg["topk_groups"]):
        v = sum(gs[g] for g in gset)
        if v > best_val:
            best_set, best_val = gset, v
    cand = [e for g in best_set for e in range(g * per, (g + 1) * per)]
    eset, ev = None, -math.inf
    for s in itertools.combinations(sorted(cand), cfg["topk"]):
        v = sum(b[e] for e in s)
        if v > ev:
            eset, ev = s, v
    return set(best_set), set(eset)


def test_selection_brute_force_tiny():
    wl = synth.WORKLOADS["tiny_fp32"]
    cfg = _cfg(wl)
    rng = np.random.default_rng(5)
    for trial in range(300):
        logit = rng.standard_normal(wl.n_experts) * rng.uniform(0.1, 3)
        bias = 28.0 + rng.standard_normal(wl.n_experts) * rng.choice([0.05, 0.5])
        r = oracle.route_token(logit, bias, cfg)
        groups, experts = _brute_select(r.biased, cfg)
        assert set(r.groups) == groups
        assert set(int(e) for e in r.ids) == experts


def test_selection_brute_force_beam_groups():
    # Beam shape (256 experts, 8 groups, 4 kept, top-8): enumerate all C(8,4)=70
    # group choices; the expert stage is checked against a stable argsort.
    wl = synth.WORKLOADS["decode_t8"]
    cfg = _cfg(wl)
    w_r, bias = synth.make_router(wl)
    x, _, _, _ = synth.make_activations(wl, T=3)
    logits = oracle.router_logits(synth.to_f64(x), synth.to_f64(w_r))
    per = wl.n_experts // wl.n_groups
    for t in range(3):
        r = oracle.route_token(logits[t], synth.to_f64(bias), cfg)
        b = r.biased
        gscore = [sum(sorted(b[g * per:(g + 1) * per])[-2:]) for g in range(wl.n_groups)]
        best = max(itertools.combinations(range(wl.n_groups), 4), key=lambda s: sum(gscore[g] for g in s))
        assert set(r.groups) == set(best)
        mask = np.full(wl.n_experts, -np.inf)
        for g in best:
            mask[g * per:(g + 1) * per] = 0
        order = np.argsort(-(b + mask), kind="stable")[:wl.topk]
        assert list(r.ids) == list(order)


def test_all_groups_kept_is_plain_topk():
    rng = np.random.default_rng(6)
    cfg = dict(n_experts=64, n_groups=8, topk_groups=8, topk=6, group_topn=2, routed_scale=2.5)
    for _ in range(50):
        logit = rng.standard_normal(64)
        bias = rng.standard_normal(64) * 0.1
        r = oracle.route_token(logit, bias, cfg)
        b = oracle.sigmoid(logit) + bias
        assert list(r.ids) == list(np.argsort(-b, kind="stable")[:6])


def test_one_expert_per_group_is_plain_topk():
    rng = np.random.default_rng(7)
    cfg = dict(n_experts=32, n_groups=32, topk_groups=5, topk=5, group_topn=1, routed_scale=2.5)
    for _ in range(50):
        logit = rng.standard_normal(32)
        bias = rng.standard_normal(32) * 0.1
        r = oracle.route_token(logit, bias, cfg)
        b = oracle.sigmoid(logit) + bias
        assert list(r.ids) == list(np.argsort(-b, kind="stable")[:5])


def test_routing_invariants_beam_shape():
    wl = synth.WORKLOADS["skew_t64"]
    cfg = _cfg(wl)
    w_r, bias = synth.make_router(wl)
    x, _, _, _ = synth.make_activations(wl, T=16)
    logits = oracle.router_logits(synth.to_f64(x), synth.to_f64(w_r))
    bias = synth.to_f64(bias)
    per = wl.n_experts // wl.n_groups
    for t in range(16):
        r = oracle.route_token(logits[t], bias, cfg)
        ids = [int(e) for e in r.ids]
        assert len(set(ids)) == wl.topk
        assert all(e // per in r.groups for e in ids)           # chosen experts lie in chosen groups
        assert np.all(r.weights > 0)
        assert abs(r.weights.sum() - 2.5) < 1e-12               # weights sum to the routed scale
        # weights follow the unbiased scores, not the biased ones
        s = oracle.sigmoid(logits[t])[ids]
        np.testing.assert_allclose(r.weights / r.weights[0], s / s[0], rtol=1e-12)
        # descending biased score
        assert all(r.biased[ids[i]] >= r.biased[ids[i + 1]] for i in range(len(ids) - 1))
        # a constant bias shift changes neither the choice nor the weights
        r2 = oracle.route_token(logits[t], bias + 3.0, cfg)
        assert list(r2.ids) == ids
        np.testing.assert_allclose(r2.weights, r.weights, rtol=1e-14)


def test_single_expert_gets_whole_scale():
    rng = np.random.default_rng(8)
    cfg = dict(n_experts=16, n_groups=4, topk_groups=2, topk=1, group_topn=2, routed_scale=2.5)
    r = oracle.route_token(rng.standard_normal(16), np.zeros(16), cfg)
    assert r.weights[0] == 2.5


def test_exact_tie_gives_zero_margin_and_lower_index():
    cfg = dict(n_experts=16, n_groups=4, topk_groups=4, topk=3, group_topn=2, routed_scale=2.5)
    logit = np.zeros(16)
    bias = np.zeros(16)
    bias[[3, 9, 12, 14]] = 1.0
    r = oracle.route_token(logit, bias, cfg)
    assert list(r.ids) == [3, 9, 12] and r.margin_expert == 0.0


# ---------------------------------------------------------------- permutation

def test_permutation_hand_golden():
    g = json.load(open(os.path.join(GOLDEN, "permutation_hand.json")))
    off, rt, pr = oracle.permutation(np.array(g["ids"]), g["n_experts"])
    assert list(off) == g["offsets"] and list(rt) == g["row_token"] and list(pr) == g["pair_row"]


@pytest.mark.parametrize("T,E,K,skew", [(1, 8, 2, 0.0), (37, 16, 4, 0.0), (300, 256, 8, 1.1), (513, 64, 8, 2.0)])
def test_permutation_against_stable_sort(T, E, K, skew):
    ids = synth.random_ids(T, E, K, skew=skew).numpy()
    off, rt, pr = oracle.permutation(ids, E)
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")          # library stable sort of pairs by expert
    np.testing.assert_array_equal(rt, order // K)
    np.testing.assert_array_equal(pr[order], np.arange(T * K))
    np.testing.assert_array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert sorted(pr) == list(range(T * K))           # each pair gets exactly one row
