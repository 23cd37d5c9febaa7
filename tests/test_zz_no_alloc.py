"""The allocation-free experts entry point (beam_moe_experts_static, which
works in the library's per-GPU static scratch array) against the entry
point with a caller workspace (beam_moe_experts): identical outputs on two
calls in a row, the second with fewer tokens, for bf16 and fp8 experts, on
a small expert shape and on the Beam decode shape.  (Its size limit and
argument checks are host-side: tests/test_abi_host.py.)"""

import pytest
import torch

import synth

beam = pytest.importorskip("expert_routed_ffn_amd")
pytestmark = pytest.mark.gpu
DEV = "cuda"


def _wl(w_dtype, H, F, E, K):
    return synth.Workload("static", T=1, hidden=H, n_experts=E, n_groups=4 if E % 4 == 0 else 1,
                          topk_groups=2 if E % 4 == 0 else 1, topk=K, group_topn=2, d_ff=F,
                          routed_scale=2.5, rms_eps=1e-6, n=20, act_dtype="bf16", w_dtype=w_dtype,
                          bias_sigma=0.02, seed=11)


def _run(wl, Ts, skew):
    cfg = beam.LayerCfg(wl.hidden, wl.n_experts, wl.n_groups, wl.topk_groups, wl.topk,
                        wl.group_topn, wl.d_ff, wl.routed_scale, wl.rms_eps)
    E, K = wl.n_experts, wl.topk
    wgu, wd, sgu, sd = synth.make_expert_stacks(wl, DEV)
    pgu, pd = torch.empty_like(wgu), torch.empty_like(wd)
    beam.beam_moe_pack_weights(cfg, wgu, wd, pgu, pd)
    fp8 = wl.w_dtype == "fp8"
    for T in Ts:
        print(f"static experts {wl.w_dtype} H={wl.hidden} F={wl.d_ff} E={E} T={T}", flush=True)
        x, _, _, _ = synth.make_activations(wl, DEV, T=T)
        ids = synth.random_ids(T, E, K, skew=skew).to(DEV)
        off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        rt = torch.empty(T * K, dtype=torch.int32, device=DEV)
        pr = torch.empty(T * K, dtype=torch.int32, device=DEV)
        ws = beam.workspace(cfg, T, beam.BEAM_FP8_E4M3 if fp8 else beam.BEAM_BF16)
        xq = torch.empty((T, wl.hidden), dtype=torch.uint8, device=DEV) if fp8 else None
        xs = torch.empty(T, dtype=torch.float32, device=DEV) if fp8 else None
        beam.beam_moe_permute(cfg, ids, off, rt, pr, x=x if fp8 else None, x_q=xq, x_scale=xs, ws=ws)
        y_ref = torch.empty((T * K, wl.hidden), dtype=torch.float32, device=DEV)
        y_st = torch.full_like(y_ref, float("nan"))
        xin = xq if fp8 else x
        beam.beam_moe_experts(cfg, T, xin, off, rt, pgu, pd, y_ref, x_scale=xs, s_gate_up=sgu, s_down=sd, ws=ws)
        beam.beam_moe_experts_static(cfg, T, xin, off, rt, pgu, pd, y_st, x_scale=xs, s_gate_up=sgu, s_down=sd)
        torch.cuda.synchronize()
        assert torch.isfinite(y_ref).all()
        assert torch.equal(y_st, y_ref), (T, (y_st - y_ref).abs().max().item())


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
def test_static_experts_small_shape(w_dtype):
    _run(_wl(w_dtype, 512, 256, 16, 4), (300, 37), 0.5)


@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
def test_static_experts_beam_decode_shape(w_dtype):
    _run(_wl(w_dtype, 5120, 2560, 8, 4), (12, 3), 0.0)
