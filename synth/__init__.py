"""Seeded synthetic inputs for the Beam-style MoE layer.

This module only draws random tensors and stores them in the formats the
layer consumes (bf16, fp32, or e4m3 codes with per-row fp32 scales).  It
holds none of the layer's arithmetic: no routing, no permutation, no GEMM,
no normalisation.  Both the CPU oracle (through the tests and the bench's
CPU baseline) and the HIP path consume exactly the tensors made here.

Workloads follow the five layer shapes the pages describe (hidden 5120,
256 routed experts in 8 groups, top-4 groups then top-8 experts, routed
scale 2.5, SwiGLU d_ff 2560; TokenSpeed x Reflection Beam blog, section
"Architecture"; vLLM Beam summary, section on the MoE and residual stream),
plus a tiny all-fp32 layer used for exhaustive checks.

Every tensor comes from its own torch.Generator, seeded from
(workload seed, tensor id, expert id), so any expert can be regenerated on
its own and generation on the GPU never needs the host.
"""

from __future__ import annotations

import dataclasses
import hashlib
import math

import torch

# tensor ids used in the seed tuple
_X, _WR, _BIAS, _ZIPF, _WG, _WU, _WD, _H, _GPOST, _GPRE, _XSCALE = range(11)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    hidden: int
    n_experts: int
    n_groups: int
    topk_groups: int
    topk: int
    group_topn: int
    d_ff: int
    routed_scale: float
    rms_eps: float
    n: int                   # residual index of the norm boundary (1-based)
    act_dtype: str           # "f32" or "bf16": x, h, gamma, outputs
    w_dtype: str             # "f32", "bf16" or "fp8"
    bias_sigma: float
    zipf_s: float = 0.0      # >0: add a Zipf(s) per-expert offset spanning +-0.5
    token_lognormal: float = 0.0  # >0: scale each x row by LogNormal(0, this)
    seed: int = 0
    dense: bool = False      # a dense SwiGLU layer (one MLP of width d_ff over all tokens)

    def with_T(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T)


_BEAM = dict(hidden=5120, n_experts=256, n_groups=8, topk_groups=4, topk=8,
             group_topn=2, d_ff=2560, routed_scale=2.5, rms_eps=1e-6)

WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", T=4, hidden=256, n_experts=16, n_groups=4,
                          topk_groups=2, topk=4, group_topn=2, d_ff=128,
                          routed_scale=2.5, rms_eps=1e-6, n=5, act_dtype="f32",
                          w_dtype="f32", bias_sigma=0.05, seed=0),
    "decode_t8": Workload("decode_t8", T=8, n=20, act_dtype="bf16", w_dtype="bf16",
                          bias_sigma=0.02, seed=1, **_BEAM),
    "skew_t64": Workload("skew_t64", T=64, n=20, act_dtype="bf16", w_dtype="bf16",
                         bias_sigma=0.02, zipf_s=1.1, seed=1, **_BEAM),
    "prefill_t2048": Workload("prefill_t2048", T=2048, n=20, act_dtype="bf16",
                              w_dtype="bf16", bias_sigma=0.02, token_lognormal=0.5,
                              seed=1, **_BEAM),
    "prefill_fp8_t16384": Workload("prefill_fp8_t16384", T=16384, n=20, act_dtype="bf16",
                                   w_dtype="fp8", bias_sigma=0.02, seed=1, **_BEAM),
    # the decode shapes with 4-bit (MXFP4) experts quantised from the same
    # float weights as the bf16 ones
    "decode_t8_mxfp4": Workload("decode_t8_mxfp4", T=8, n=20, act_dtype="bf16", w_dtype="mxfp4",
                                bias_sigma=0.02, seed=1, **_BEAM),
    "skew_t64_mxfp4": Workload("skew_t64_mxfp4", T=64, n=20, act_dtype="bf16", w_dtype="mxfp4",
                               bias_sigma=0.02, zipf_s=1.1, seed=1, **_BEAM),
    # the dense layers (0-2): one SwiGLU MLP of width 20480 over all tokens,
    # bf16 weights, the same norm boundary
    "dense_t8": Workload("dense_t8", T=8, hidden=5120, n_experts=1, n_groups=1, topk_groups=1, topk=1,
                         group_topn=1, d_ff=20480, routed_scale=1.0, rms_eps=1e-6, n=2, act_dtype="bf16",
                         w_dtype="bf16", bias_sigma=0.0, seed=2, dense=True),
    "dense_t2048": Workload("dense_t2048", T=2048, hidden=5120, n_experts=1, n_groups=1, topk_groups=1,
                            topk=1, group_topn=1, d_ff=20480, routed_scale=1.0, rms_eps=1e-6, n=2,
                            act_dtype="bf16", w_dtype="bf16", bias_sigma=0.0, token_lognormal=0.5, seed=2,
                            dense=True),
    # the fp8 prefill shape with the bf16 experts of the other Beam workloads:
    # about 512 rows per expert, past the point where bf16 matrix-core
    # throughput rather than HBM bandwidth bounds the expert GEMMs
    "prefill_bf16_t16384": Workload("prefill_bf16_t16384", T=16384, n=20, act_dtype="bf16",
                                    w_dtype="bf16", bias_sigma=0.02, seed=1, **_BEAM),
    # the same prefill shape with 4-bit (MXFP4) experts
    "prefill_mxfp4_t16384": Workload("prefill_mxfp4_t16384", T=16384, n=20, act_dtype="bf16",
                                     w_dtype="mxfp4", bias_sigma=0.02, seed=1, **_BEAM),
}
# the order the workloads are listed in (index = position in that list; the
# bf16 16384-token shape, the 4-bit decode shapes and the dense layers came
# after the first five)
WORKLOAD_ORDER = ["tiny_fp32", "decode_t8", "skew_t64", "prefill_t2048", "prefill_fp8_t16384",
                  "prefill_bf16_t16384", "decode_t8_mxfp4", "skew_t64_mxfp4", "dense_t8", "dense_t2048",
                  "prefill_mxfp4_t16384"]


def _seed(*parts: int) -> int:
    h = hashlib.sha256(",".join(str(int(p)) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def _randn(shape, std, device, *parts) -> torch.Tensor:
    g = _gen(device, *parts)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _act(t: torch.Tensor, wl: Workload) -> torch.Tensor:
    return t.to(torch.bfloat16) if wl.act_dtype == "bf16" else t.contiguous()


def make_router(wl: Workload, device="cpu"):
    """Router weight [E,H] fp32 (row e feeds expert e) and correction bias [E] fp32."""
    E, H = wl.n_experts, wl.hidden
    w_r = _randn((E, H), 1.0 / math.sqrt(H), device, wl.seed, _WR)
    bias = 28.0 + _randn((E,), wl.bias_sigma, device, wl.seed, _BIAS)
    if wl.zipf_s > 0:
        # experts get Zipf ranks 1..E from a seeded permutation; the rank's
        # weight r^-s is mapped affinely onto [-0.5, +0.5]
        g = _gen("cpu", wl.seed, _ZIPF)
        ranks = torch.randperm(E, generator=g).to(torch.float64) + 1.0
        z = ranks ** (-wl.zipf_s)
        zmin, zmax = float(E) ** (-wl.zipf_s), 1.0
        off = -0.5 + (z - zmin) / (zmax - zmin)
        bias = bias + off.to(torch.float32).to(device)
    return w_r.contiguous(), bias.to(torch.float32).contiguous()


def make_activations(wl: Workload, device="cpu", T: int | None = None):
    """x [T,H], residual h [T,H], gamma_post [H], gamma_pre [H] in act dtype."""
    T = wl.T if T is None else T
    H = wl.hidden
    x = _randn((T, H), 1.0, device, wl.seed, _X, T)
    if wl.token_lognormal > 0:
        c = torch.exp(_randn((T, 1), wl.token_lognormal, device, wl.seed, _XSCALE, T))
        x = x * c
    h = _randn((T, H), 1.0, device, wl.seed, _H, T)
    gp = 1.0 + _randn((H,), 0.1, device, wl.seed, _GPOST)
    gq = 1.0 + _randn((H,), 0.1, device, wl.seed, _GPRE)
    return _act(x, wl), _act(h, wl), _act(gp, wl), _act(gq, wl)


def _quantize_rows_e4m3(w: torch.Tensor):
    """Offline per-output-channel e4m3 weight format: codes and fp32 scales.

    Uses torch's own float8_e4m3fn conversion; this is a checkpoint format
    step, not part of the layer."""
    amax = w.abs().amax(dim=-1, keepdim=True)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (w / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s.squeeze(-1).to(torch.float32)


_E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _quantize_rows_mxfp4(w: torch.Tensor):
    """Offline MXFP4 weight format (OCP microscaling): every block of 32
    consecutive weights of a row shares the power-of-two scale
    2^(floor(log2(amax)) - 2); each weight becomes the nearest E2M1 value of
    w / scale (ties to the even code, saturating at 6).  Returns packed codes
    [rows, cols/2] uint8 (element 2i in the low nibble of byte i) and the
    E8M0 scale codes [rows, cols/32] uint8.  A checkpoint format step, not
    part of the layer."""
    rows, cols = w.shape
    blk = w.reshape(rows, cols // 32, 32).to(torch.float64)
    amax = blk.abs().amax(dim=-1)
    _, ex = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
    e = torch.where(amax > 0, ex.to(torch.int64) - 3, torch.full_like(ex, -127, dtype=torch.int64)).clamp(-127, 127)
    y = (blk.abs() / torch.exp2(e.to(torch.float64)).unsqueeze(-1)).clamp(max=6.0)
    grid = torch.tensor(_E2M1_GRID, dtype=torch.float64, device=w.device)
    mids = (grid[1:] + grid[:-1]) / 2
    idx = torch.bucketize(y, mids, right=False)            # y <= mid -> lower code
    tie = (idx < 7) & (y == mids[idx.clamp(max=6)])
    idx = idx + (tie & (idx % 2 == 1)).to(idx.dtype)       # ties to the even code
    code = idx | torch.where(blk < 0, 8, 0)
    code = code.reshape(rows, cols).to(torch.uint8)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), (e + 127).to(torch.uint8).contiguous()


def make_expert(wl: Workload, e: int, device="cpu"):
    """Weights of expert e.

    Returns (w_gate_up [2F,H], w_down [H,F], s_gate_up [2F] | None, s_down [H] | None).
    Rows [0,F) of w_gate_up are the gate projection, rows [F,2F) the up
    projection.  bf16/f32 stacks carry no scales; fp8 stacks are uint8 e4m3
    codes with one fp32 scale per output row; mxfp4 stacks are packed E2M1
    codes [2F,H/2] / [H,F/2] with E8M0 scale codes [2F,H/32] / [H,F/32]."""
    H, F = wl.hidden, wl.d_ff
    wg = _randn((F, H), 1.0 / math.sqrt(H), device, wl.seed, _WG, e)
    wu = _randn((F, H), 1.0 / math.sqrt(H), device, wl.seed, _WU, e)
    wd = _randn((H, F), 1.0 / math.sqrt(F), device, wl.seed, _WD, e)
    wgu = torch.cat([wg, wu], dim=0)
    if wl.w_dtype == "f32":
        return wgu.contiguous(), wd.contiguous(), None, None
    if wl.w_dtype == "bf16":
        return wgu.to(torch.bfloat16), wd.to(torch.bfloat16), None, None
    if wl.w_dtype == "fp8":
        qgu, sgu = _quantize_rows_e4m3(wgu)
        qd, sd = _quantize_rows_e4m3(wd)
        return qgu, qd, sgu, sd
    if wl.w_dtype == "mxfp4":
        cgu, sgu = _quantize_rows_mxfp4(wgu)
        cd, sd = _quantize_rows_mxfp4(wd)
        return cgu, cd, sgu, sd
    raise ValueError(wl.w_dtype)


def make_expert_stacks(wl: Workload, device="cpu"):
    """All E experts stacked: w_gate_up [E,2F,H], w_down [E,H,F] (+ scales for fp8)."""
    E, H, F = wl.n_experts, wl.hidden, wl.d_ff
    wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8, "mxfp4": torch.uint8}[wl.w_dtype]
    cdiv = 2 if wl.w_dtype == "mxfp4" else 1
    wgu = torch.empty((E, 2 * F, H // cdiv), dtype=wdt, device=device)
    wd = torch.empty((E, H, F // cdiv), dtype=wdt, device=device)
    sgu = sd = None
    if wl.w_dtype == "fp8":
        sgu = torch.empty((E, 2 * F), dtype=torch.float32, device=device)
        sd = torch.empty((E, H), dtype=torch.float32, device=device)
    if wl.w_dtype == "mxfp4":
        sgu = torch.empty((E, 2 * F, H // 32), dtype=torch.uint8, device=device)
        sd = torch.empty((E, H, F // 32), dtype=torch.uint8, device=device)
    for e in range(E):
        a, b, c, d = make_expert(wl, e, device)
        wgu[e].copy_(a)
        wd[e].copy_(b)
        if sgu is not None:
            sgu[e].copy_(c)
            sd[e].copy_(d)
    return wgu, wd, sgu, sd


def random_ids(T: int, E: int, K: int, device="cpu", seed=0, skew=0.0):
    """Random routes [T,K] int32 with K distinct experts per token (for testing
    the permutation on its own).  skew>0 biases towards low expert ids."""
    g = _gen("cpu", seed, 99, T, E, K)
    w = torch.ones(E, dtype=torch.float64)
    if skew > 0:
        w = (torch.arange(E, dtype=torch.float64) + 1.0) ** (-skew)
    ids = torch.multinomial(w.expand(T, E), K, replacement=False, generator=g)
    return ids.to(torch.int32).to(device).contiguous()


def to_f64(t: torch.Tensor):
    """Host fp64 numpy copy of a tensor (bf16/f32 values are exact in fp64)."""
    return t.detach().to("cpu").to(torch.float64).numpy()

