"""GPU parity of the norm boundary on a given m, the dense SwiGLU layers
(d_ff 20480) and the expert-parallel shards against the CPU oracle.

Dense layer: beam_moe_dense_mlp then beam_moe_norm_boundary against
oracle.dense_layer_tokens, at the decode size (all tokens; the down
projection split over K) and at T = 2048 (a sample that includes rows
64..127 of the 128-row work items).

EP8 shards on one GPU: for each of the 8 groups of 32 experts,
beam_moe_permute_shard (bit-exact against the oracle's permutation
restricted to the group), beam_moe_experts on the group's slice of the
stacks and beam_moe_combine_partial against oracle.combine_shard; the sum of
the 8 partials through beam_moe_norm_boundary against the oracle's layer.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from parity_util import check_output, check_routes, oracle_cfg, sample_tokens, say

beam = pytest.importorskip("expert_routed_ffn_amd")
pytestmark = pytest.mark.gpu
DEV = "cuda"
N_SHARDS, PER_SHARD = 8, 32


def lcfg(wl, **kw):
    c = dict(hidden=wl.hidden, n_experts=wl.n_experts, n_groups=wl.n_groups, topk_groups=wl.topk_groups,
             topk=wl.topk, group_topn=wl.group_topn, d_ff=wl.d_ff, routed_scale=wl.routed_scale,
             rms_eps=wl.rms_eps)
    c.update(kw)
    return beam.LayerCfg(**c)


@pytest.mark.parametrize("m_dtype,act", [(torch.float32, "bf16"), (torch.bfloat16, "bf16"), (torch.float32, "f32")])
def test_norm_boundary_parity(m_dtype, act):
    say(f"norm boundary m={m_dtype} act={act}")
    T, H, n = 37, 5120, 7
    g = torch.Generator(device=DEV).manual_seed(31)
    adt = torch.bfloat16 if act == "bf16" else torch.float32
    m = (torch.randn((T, H), generator=g, device=DEV) * 0.7).to(m_dtype)
    h = torch.randn((T, H), generator=g, device=DEV).to(adt)
    gp = (1 + 0.1 * torch.randn(H, generator=g, device=DEV)).to(adt)
    gq = (1 + 0.1 * torch.randn(H, generator=g, device=DEV)).to(adt)
    h_dev, xn = h.clone(), torch.empty_like(h)
    beam.beam_moe_norm_boundary(beam.LayerCfg(), m, h_dev, xn, gp, gq, n)
    torch.cuda.synchronize()
    rnd = oracle.round_bf16 if act == "bf16" else oracle.round_f32
    _, hn, xo = oracle.norm_boundary(synth.to_f64(m), synth.to_f64(h), synth.to_f64(gp), synth.to_f64(gq), n,
                                     1e-6, rnd=rnd)
    kind = "bf16" if act == "bf16" else "f32"
    check_output("h_new", h_dev.cpu().double().numpy(), hn, kind)
    check_output("x_next", xn.cpu().double().numpy(), xo, kind)


def run_dense(wname, n_sample):
    wl = synth.WORKLOADS[wname]
    say(f"dense layer {wname}: T={wl.T} d_ff={wl.d_ff}")
    cfg = lcfg(wl)
    w_gu, w_d, _, _ = synth.make_expert(wl, 0, DEV)
    pgu, pd = torch.empty_like(w_gu), torch.empty_like(w_d)
    beam.beam_moe_pack_weights(cfg, w_gu.unsqueeze(0), w_d.unsqueeze(0), pgu.unsqueeze(0), pd.unsqueeze(0))
    x, h, gp, gq = synth.make_activations(wl, DEV)
    y = torch.empty((wl.T, wl.hidden), dtype=torch.float32, device=DEV)
    h_dev, xn = h.clone(), torch.empty_like(h)
    ws = beam.dense_workspace(cfg, wl.T, wl.d_ff)
    beam.beam_moe_dense_mlp(cfg, x, pgu, pd, y, ws)
    beam.beam_moe_norm_boundary(cfg, y, h_dev, xn, gp, gq, wl.n)
    torch.cuda.synchronize()
    say("  gpu dense layer done")
    if wl.T <= n_sample:
        tokens = list(range(wl.T))
    else:   # half of them in rows 64..127 of a 128-row work item
        rng = np.random.default_rng(4)
        deep = [t for t in range(wl.T) if t % 128 >= 64]
        tokens = sorted(set(sample_tokens(wl.T, n_sample // 2, seed=3)) |
                        {int(t) for t in rng.choice(deep, n_sample // 2, replace=False)})
    ref = oracle.dense_layer_tokens(oracle_cfg(wl), synth.to_f64(x), synth.to_f64(w_gu), synth.to_f64(w_d),
                                    synth.to_f64(h), synth.to_f64(gp), synth.to_f64(gq), wl.n, tokens=tokens)
    check_output("y", y.cpu().double().numpy()[tokens], ref["y"], "bf16")
    check_output("h_new", h_dev.cpu().double().numpy()[tokens], ref["h_new"], "bf16")
    check_output("x_next", xn.cpu().double().numpy()[tokens], ref["x_next"], "bf16")


def test_dense_layer_t8():
    run_dense("dense_t8", 8)


@pytest.mark.timeout(400)
def test_dense_layer_t2048():
    run_dense("dense_t2048", 48)


_stacks = {}


def run_shards(wname, n_sample):
    wl = synth.WORKLOADS[wname]
    say(f"EP8 shards {wname}: T={wl.T}")
    cfg = lcfg(wl)
    if "bf16" not in _stacks:
        _stacks["bf16"] = beam.packed_expert_stacks(cfg, lambda e: synth.make_expert(wl, e, DEV), wl.n_experts, DEV)
    wgu, wd, _, _ = _stacks["bf16"]
    w_r, bias = synth.make_router(wl, DEV)
    x, h, gp, gq = synth.make_activations(wl, DEV)
    T, K, H = wl.T, wl.topk, wl.hidden
    bufs = beam.alloc_buffers(cfg, T, x.dtype, beam.BEAM_BF16, keep_moe_out=True, device=DEV)
    h_full = h.clone()
    beam.moe_layer(cfg, x, w_r, bias, wgu, wd, h_full, gp, gq, wl.n, bufs)   # the unsharded layer
    # every shard on this GPU, as each of 8 GPUs would run it
    lcfg_shard = lcfg(wl, n_experts=PER_SHARD, n_groups=1, topk_groups=1)
    parts, perms = [], []
    ws = bufs.ws
    y = torch.empty((T * K, H), dtype=torch.float32, device=DEV)
    for r in range(N_SHARDS):
        eb = r * PER_SHARD
        off = torch.empty(PER_SHARD + 1, dtype=torch.int32, device=DEV)
        rt = torch.empty(T * K, dtype=torch.int32, device=DEV)
        pr = torch.empty(T * K, dtype=torch.int32, device=DEV)
        beam.beam_moe_permute_shard(cfg, bufs.topk_ids, eb, PER_SHARD, off, rt, pr, ws=ws)
        beam.beam_moe_experts(lcfg_shard, T, x, off, rt, wgu[eb:eb + PER_SHARD], wd[eb:eb + PER_SHARD], y, ws=ws)
        m_r = torch.empty((T, H), dtype=torch.float32, device=DEV)
        beam.beam_moe_combine_partial(cfg, y, pr, bufs.topk_w, m_r)
        torch.cuda.synchronize()
        parts.append(m_r)
        perms.append((off.cpu().numpy(), rt.cpu().numpy(), pr.cpu().numpy()))
    m_sum = parts[0].clone()
    for m_r in parts[1:]:
        m_sum += m_r
    h_ep, xn_ep = h.clone(), torch.empty_like(h)
    beam.beam_moe_norm_boundary(cfg, m_sum, h_ep, xn_ep, gp, gq, wl.n)
    torch.cuda.synchronize()
    say("  gpu shards done")

    ocfg = oracle_cfg(wl)
    xd = synth.to_f64(x)
    routes = oracle.route(oracle.router_logits(xd, synth.to_f64(w_r)), synth.to_f64(bias), ocfg)
    gids = bufs.topk_ids.cpu().numpy()
    _, differ = check_routes(gids, bufs.topk_w.cpu().numpy(), routes, ocfg)
    ids = np.array([r.ids for r in routes])
    override = {t: [int(v) for v in gids[t]] for t in range(T) if list(gids[t]) != list(ids[t])}
    for t, v in override.items():
        ids[t] = v
    # each shard's permutation: the oracle's counting sort restricted to the group
    o_off, o_rt, o_pr = oracle.permutation(ids, wl.n_experts)
    touched = []
    for r in range(N_SHARDS):
        eb = r * PER_SHARD
        lo, hi = int(o_off[eb]), int(o_off[eb + PER_SHARD])
        want_off = o_off[eb:eb + PER_SHARD + 1] - lo
        want_pr = np.where((o_pr >= lo) & (o_pr < hi), o_pr - lo, -1)
        off, rt, pr = perms[r]
        assert np.array_equal(off, want_off), r
        assert np.array_equal(rt[:hi - lo], o_rt[lo:hi]), r
        assert np.array_equal(pr, want_pr), r
        touched.append(int((np.diff(want_off) > 0).sum()))
    say(f"  shard permutations bit-exact; experts touched per shard {touched}")
    tokens = sorted(set(sample_tokens(T, n_sample, seed=5)) | differ)
    def ew(e):
        a, b, _, _ = synth.make_expert(wl, e, DEV)
        return {"w_gu": synth.to_f64(a), "w_d": synth.to_f64(b)}
    ref = oracle.layer_tokens(ocfg, xd, synth.to_f64(w_r), synth.to_f64(bias), ew,
                              synth.to_f64(h), synth.to_f64(gp), synth.to_f64(gq), wl.n, tokens=tokens,
                              ids_override={t: override[t] for t in differ})
    for r in range(N_SHARDS):
        want = np.array([oracle.combine_shard(ref["y"][i], ref["routes"][i].ids, ref["routes"][i].weights,
                                              r * PER_SHARD, PER_SHARD) for i in range(len(tokens))])
        got = parts[r].cpu().double().numpy()[tokens]
        # partials can be zero for a token with no expert in the shard
        assert np.all(got[np.all(want == 0, axis=1)] == 0)
        check_output(f"m shard {r}", got, want, "f32" if np.abs(want).max() == 0 else "bf16")
    check_output("sum of shard partials vs m", m_sum.cpu().double().numpy()[tokens], ref["m"], "bf16")
    check_output("h_new (EP)", h_ep.cpu().double().numpy()[tokens], ref["h_new"], "bf16")
    check_output("x_next (EP)", xn_ep.cpu().double().numpy()[tokens], ref["x_next"], "bf16")
    # the sharded layer equals the unsharded one up to the fp32 summation order
    d = (m_sum - bufs.moe_out).abs().max().item()
    say(f"  max |sum of shards - unsharded m| = {d:.3e}")
    assert d < 1e-4


def test_ep8_shards_t8():
    run_shards("decode_t8", 8)


@pytest.mark.timeout(400)
def test_ep8_shards_t2048():
    run_shards("prefill_t2048", 24)
    _stacks.clear()
    torch.cuda.empty_cache()
