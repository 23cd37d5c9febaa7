"""Plain fp64 CPU oracle of the Beam MoE layer.  TEST INFRASTRUCTURE ONLY.

Everything is numpy float64 unless a step states otherwise.  Rounding to a
storage format (bf16, fp32, e4m3) is done by this module's own functions,
written from the formats' definitions, and happens only at the points listed
in `layer_tokens`.

Readings taken where the pages leave a step open (each is listed with its
reason in the design notes of the repository):
  * group score = sum of the two largest biased scores in the group, groups
    are contiguous blocks of E/G experts;
  * ties (equal scores) go to the lower group / expert index; the K chosen
    experts are reported in descending biased score;
  * routing weights use the unbiased sigmoid scores, renormalised over the
    K chosen experts, times the routed scale (so they sum to the scale);
  * SwiGLU is silu(gate) * up with rows [0,F) of the stacked weight the gate
    and rows [F,2F) the up projection;
  * bf16 rounding points: the SwiGLU output a (GEMM2 input), the post-norm
    output p, the new residual h' and the next sublayer input x_next; the
    expert outputs y and their weighted sum m stay unrounded;
  * each RMSNorm is v / sqrt(mean(v^2) + eps) * gamma with learned gamma;
  * fp8 path: dynamic per-row scale amax/448 for the token activations and
    for each (token, expert) SwiGLU output over all F columns, e4m3 codes by
    round-to-nearest-even with saturation at +-448.  The scale and the
    division that picks each code are fp32 operations: the Gaudi port's
    W8A8 reference is an fp32 CPU program that models per-token FP8
    activations ([GD] "Correctness"), so its scales are fp32 numbers.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "round_bf16", "round_f32", "e4m3_decode", "e4m3_round", "quantize_row_e4m3",
    "router_logits", "sigmoid", "silu", "Route", "route_token", "route",
    "permutation", "expert_ffn", "expert_ffn_w8a8", "combine", "rmsnorm",
    "norm_boundary", "layer_tokens", "E4M3_MAX",
    "E2M1_MAX", "MX_BLOCK", "e2m1_decode", "e2m1_round", "e2m1_encode", "e8m0_decode",
    "quantize_mx_fp4", "unpack_fp4", "expert_ffn_w4a4",
    "dense_layer_tokens", "combine_shard",
]

E4M3_MAX = 448.0

# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(v):
    """Nearest bfloat16 value of each element (ties to even), as float64.

    bfloat16 keeps 8 significant bits and fp32's exponent range (smallest
    normal 2^-126, subnormal spacing 2^-133).  The value is rounded straight
    from fp64, not through fp32, so no double rounding happens.  Magnitudes
    that round past the largest finite bf16 become infinities; NaN stays NaN.
    Used at the bf16 rounding points the Gaudi port lists ([GD] "What was
    built") and that vLLM's fused norm keeps ([VL], kernel change 1).
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    fin = np.isfinite(v) & (v != 0)
    x = v[fin]
    _, e = np.frexp(x)                 # x = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)            # below 2^-126 the spacing stays 2^-133
    q = np.ldexp(np.round(np.ldexp(x, 8 - e)), e - 8)   # np.round: half to even
    q = np.where(np.abs(q) > _BF16_MAX, np.copysign(np.inf, q), q)
    out[fin] = q
    return out


def round_f32(v):
    """Nearest fp32 value (IEEE round-to-nearest-even), as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def e4m3_decode(codes):
    """Values of OCP FP8 E4M3FN codes (uint8) as float64.

    Layout: sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent
    field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; there is no
    infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = (c & 0x7).astype(np.float64)
    mag = np.where(ef == 0, mf / 8.0 * 2.0 ** -6, (1.0 + mf / 8.0) * np.exp2(ef - 7.0))
    mag = np.where((ef == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def e4m3_round(v):
    """Nearest E4M3FN value (ties to even mantissa), saturating at +-448.

    The grid spacing is 2^(E-3) for |v| in [2^E, 2^(E+1)), E >= -6, and
    2^-9 in the subnormal range below 2^-6.  NaN stays NaN; anything whose
    magnitude exceeds 448 (infinities included) saturates, the scaled-FP8
    convention of the per-channel FP8 checkpoint ([GD] "What was built").
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    fin = np.isfinite(v)
    x = np.abs(v[fin])
    _, e = np.frexp(x)                 # x in [2^(e-1), 2^e)
    E = np.maximum(e - 1, -6)
    step = np.exp2(E - 3.0)
    q = np.round(x / step) * step      # exact: division by a power of two
    q = np.minimum(q, E4M3_MAX)
    out[fin] = np.copysign(q, v[fin])
    inf = np.isinf(v)
    out[inf] = np.copysign(E4M3_MAX, v[inf])
    return out


def quantize_row_e4m3(v):
    """Dynamic per-row e4m3 quantisation: returns (scale, quantised values).

    scale = amax / 448 so that the row's largest magnitude maps onto the
    largest code; q = e4m3(v / scale).  v is taken as fp32 values and the
    scale and the division are fp32 operations (correctly rounded), the
    precision of the W8A8 reference program ([GD] "Correctness": an fp32
    CPU oracle with a W8A8 variant modelling per-token FP8 activations).
    An all-zero row gets scale 1 and codes 0.  ([GD] "What was built":
    per-channel FP8 weights with dynamic per-token activations; "EP vs TP
    quality": the down-projection input is quantised per token over the
    whole 2560-wide intermediate.)
    """
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    amax = np.float32(np.max(np.abs(v32))) if v32.size else np.float32(0)
    if amax == 0:
        return 1.0, np.zeros(v32.shape, dtype=np.float64)
    s = np.float32(amax / np.float32(E4M3_MAX))
    q = e4m3_round((v32 / s).astype(np.float64))
    return float(s), q


# --------------------------------------------------------------------------
# routing  ([TS] "Architecture", "Fused FP32 routing"; [VL] MoE section)
# --------------------------------------------------------------------------

def router_logits(x, w_r):
    """Router projection logit[t,e] = sum_i x[t,i] * W_r[e,i], in fp64.

    The router is FP32 end to end on the pages (bf16 activations times fp32
    weights, fp32 accumulation and logits; [TS] "Fused FP32 routing", [VL]
    MoE section); the oracle evaluates the same products exactly enough in
    fp64.  W_r is stored one row per expert.
    """
    return np.asarray(x, np.float64) @ np.asarray(w_r, np.float64).T


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


def silu(z):
    z = np.asarray(z, np.float64)
    return z * sigmoid(z)


@dataclass
class Route:
    ids: np.ndarray           # [K] int, descending biased score
    weights: np.ndarray       # [K] fp64, sum = routed_scale
    scores: np.ndarray        # [E] sigmoid(logit)
    biased: np.ndarray        # [E] scores + bias
    group_scores: np.ndarray  # [G]
    groups: list              # chosen groups, descending group score
    margin_group: float       # relative gap between the last chosen and first rejected group
    margin_expert: float      # relative gap between the K-th and (K+1)-th candidate

    @property
    def margin(self):
        return min(self.margin_group, self.margin_expert)


def route_token(logit, bias, cfg):
    """Sigmoid scores, correction bias, group-limited top-k, weights x scale.

    Steps ([TS] "Architecture": sigmoid scores plus a learned per-expert
    bias that only affects which experts are picked, top 4 of 8 groups then
    top 8 experts, routed output scaled by 2.5; [TS] "Fused FP32 routing":
    the 2.5 is folded into the routing weights; [VL] MoE section: the
    routing matches DeepSeek-V3, weights renormalised):
      s = sigmoid(logit);  b = s + bias
      group score = sum of the `group_topn` largest b in each contiguous group
      keep the `topk_groups` best groups (ties: lower group index)
      among their experts keep the `topk` largest b (ties: lower expert index)
      w_k = routed_scale * s[e_k] / sum_j s[e_j]
    """
    E, G = cfg["n_experts"], cfg["n_groups"]
    per = E // G
    s = sigmoid(logit)
    b = s + np.asarray(bias, np.float64)
    gs = np.empty(G)
    for g in range(G):
        members = sorted(b[g * per:(g + 1) * per], reverse=True)
        gs[g] = sum(members[:cfg["group_topn"]])
    gorder = sorted(range(G), key=lambda g: (-gs[g], g))
    chosen = gorder[:cfg["topk_groups"]]
    cand = [e for g in chosen for e in range(g * per, (g + 1) * per)]
    eorder = sorted(cand, key=lambda e: (-b[e], e))
    K = cfg["topk"]
    ids = np.array(eorder[:K], dtype=np.int64)
    sk = s[ids]
    w = cfg["routed_scale"] * sk / sk.sum()

    def rel_gap(hi, lo):
        return (hi - lo) / abs(hi) if hi != 0 else (math.inf if hi != lo else 0.0)

    mg = rel_gap(gs[gorder[len(chosen) - 1]], gs[gorder[len(chosen)]]) if len(chosen) < G else math.inf
    me = rel_gap(b[eorder[K - 1]], b[eorder[K]]) if len(eorder) > K else math.inf
    return Route(ids, w, s, b, gs, chosen, mg, me)


def route(logits, bias, cfg):
    """route_token for every row of logits [T,E]."""
    return [route_token(logits[t], bias, cfg) for t in range(np.asarray(logits).shape[0])]


# --------------------------------------------------------------------------
# permutation  ([VL] kernel list: the MoE path's routing kernels group the
# tokens by expert; [TS] "TensorRT-LLM NVFP4 MoE")
# --------------------------------------------------------------------------

def permutation(ids, n_experts):
    """Stable counting sort of the (token, slot) pairs by expert.

    ids [T,K]; pair p = t*K + k.  Returns
      offsets [E+1]: exclusive running count of pairs per expert,
      row_token [T*K]: permuted row r -> token t,
      pair_row [T*K]: pair p -> permuted row r.
    Within one expert the pairs keep ascending p, so the order is unique.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, K = ids.shape
    flat = ids.reshape(-1)
    counts = [0] * n_experts
    for e in flat:
        counts[int(e)] += 1
    offsets = [0] * (n_experts + 1)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    nxt = list(offsets[:n_experts])
    row_token = np.empty(T * K, dtype=np.int64)
    pair_row = np.empty(T * K, dtype=np.int64)
    for p in range(T * K):
        e = int(flat[p])
        r = nxt[e]
        nxt[e] += 1
        row_token[r] = p // K
        pair_row[p] = r
    return np.array(offsets, dtype=np.int64), row_token, pair_row


# --------------------------------------------------------------------------
# experts  ([TS] "TensorRT-LLM NVFP4 MoE": GEMM1 with SwiGLU fused, GEMM2,
# per-token weighted sum; [VL] MoE section: SwiGLU experts, d_ff 2560, no
# shared expert)
# --------------------------------------------------------------------------

def expert_ffn(u, w_gu, w_d, round_a=round_bf16):
    """One expert's SwiGLU MLP on rows u [m,H] (float weights).

    g = u W_g^T, v = u W_u^T (W_gu rows [0,F) gate, [F,2F) up),
    a = round_a(silu(g) * v), y = a W_d^T (y unrounded).
    """
    u = np.atleast_2d(np.asarray(u, np.float64))
    F = np.asarray(w_gu).shape[0] // 2
    gv = u @ np.asarray(w_gu, np.float64).T
    a = silu(gv[:, :F]) * gv[:, F:]
    if round_a is not None:
        a = round_a(a)
    return a @ np.asarray(w_d, np.float64).T


def expert_ffn_w8a8(u, q_gu, s_gu, q_d, s_d):
    """One expert's SwiGLU MLP with e4m3 weights and activations (W8A8).

    q_gu [2F,H] / q_d [H,F] are e4m3 codes with per-output-row fp32 scales
    s_gu [2F] / s_d [H] ([GD] "What was built": per-channel FP8 weights,
    dynamic per-token activations).  For each row of u:
      (sx, qx) = quantize_row_e4m3(u)
      g_j = sx * s_gu[j] * sum_i qx_i * q_gu[j,i]    (v likewise)
      a = silu(g) * v;  (sa, qa) = quantize_row_e4m3(a) over all F
      y_o = sa * s_d[o] * sum_j qa_j * q_d[o,j]
    The fp64 sums of e4m3 products are exact at these sizes (every product
    is a multiple of 2^-18 below 2^18, so a sum of up to 2^17 of them needs
    fewer than 53 bits), which makes the order of the summation irrelevant:
    the rows go through one matrix product per projection.
    """
    u = np.atleast_2d(np.asarray(u, np.float64))
    table = e4m3_decode(np.arange(256))          # value of every code
    wgu = table[np.asarray(q_gu, np.uint8)]
    wd = table[np.asarray(q_d, np.uint8)]
    s_gu = np.asarray(s_gu, np.float64)
    s_d = np.asarray(s_d, np.float64)
    F = wgu.shape[0] // 2
    m = u.shape[0]
    sx = np.empty(m)
    qx = np.empty_like(u)
    for r in range(m):
        sx[r], qx[r] = quantize_row_e4m3(u[r])
    gv = sx[:, None] * s_gu[None, :] * (qx @ wgu.T)
    a = silu(gv[:, :F]) * gv[:, F:]
    sa = np.empty(m)
    qa = np.empty_like(a)
    for r in range(m):
        sa[r], qa[r] = quantize_row_e4m3(a[r])
    return sa[:, None] * s_d[None, :] * (qa @ wd.T)


# --------------------------------------------------------------------------
# 4-bit experts.  The pages' 4-bit checkpoint stores every expert weight as a
# 4-bit float (E2M1) with an FP8 scale per 16 weights and an FP32 scale per
# expert ([TS] "NVFP4 and FP8 checkpoints"), and the 4-bit MoE kernel
# quantises its inputs to 4 bits at run time ([TS] "TensorRT-LLM NVFP4
# MoE").  This build re-encodes the weights in the OCP microscaling format
# MXFP4, which the target's matrix cores consume natively: E2M1 elements
# with one power-of-two (E8M0) scale per block of 32 consecutive elements of
# a row (OCP Microscaling Formats (MX) specification v1.0).
# --------------------------------------------------------------------------

E2M1_MAX = 6.0
MX_BLOCK = 32
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes):
    """Values of FP4 E2M1 codes (the low 4 bits of each integer).

    Layout: sign bit 3, exponent bits 2..1 with bias 1, mantissa bit 0.
    Exponent field 0 is subnormal (m * 0.5); otherwise (1 + m/2) * 2^(E-1).
    There is no infinity or NaN; the largest magnitude is 1.5 * 4 = 6.
    """
    c = np.asarray(codes, dtype=np.int64) & 0xF
    ef = (c >> 1) & 0x3
    mf = (c & 0x1).astype(np.float64)
    mag = np.where(ef == 0, mf * 0.5, (1.0 + mf / 2.0) * np.exp2(ef - 1.0))
    return np.where(c & 0x8, -mag, mag)


def e8m0_decode(codes):
    """Values of E8M0 scale codes: 2^(c - 127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def e2m1_round(v):
    """Nearest E2M1 value of each element, ties to the even mantissa,
    saturating at +-6 (the conversion rule of the MX specification for FP4
    elements).  NaN stays NaN.

    The non-negative grid is 0, 0.5, 1, 1.5, 2, 3, 4, 6; its spacing is 0.5
    below 2, 1 in [2, 4) and 2 in [4, 6]."""
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    fin = np.isfinite(v)
    x = np.minimum(np.abs(v[fin]), E2M1_MAX)
    step = np.where(x < 2.0, 0.5, np.where(x < 4.0, 1.0, 2.0))
    q = np.round(x / step) * step        # np.round: half to even (in units of step)
    # a tie at a spacing change (e.g. 1.75 -> 1.5 / 2) is decided by
    # np.round in the lower spacing; the even mantissa there is correct too
    out[fin] = np.copysign(np.minimum(q, E2M1_MAX), v[fin])
    inf = np.isinf(v)
    out[inf] = np.copysign(E2M1_MAX, v[inf])
    return out


def e2m1_encode(values):
    """E2M1 codes of values that lie on the grid (uint8, one code per value)."""
    v = np.asarray(values, dtype=np.float64)
    mag = np.abs(v)
    idx = np.searchsorted(_E2M1_MAG, mag)
    if not np.all(_E2M1_MAG[np.minimum(idx, 7)] == mag):
        raise ValueError("value not on the E2M1 grid")
    return (idx | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def quantize_mx_fp4(v):
    """MX quantisation of each block of 32 consecutive elements (last axis).

    Per block: amax = max |v_i|; shared exponent e = floor(log2(amax)) - 2
    (2 = the largest exponent of E2M1, so amax / 2^e lies in [4, 8));
    scale X = 2^e, kept within the E8M0 range [2^-127, 2^127];
    elements = e2m1_round(v_i / X) (division by a power of two is exact).
    An all-zero block gets the smallest scale and zero elements.
    Returns (scale codes uint8 [..., n/32], quantised element values
    float64 [..., n]) -- the dequantised value is element * 2^(code - 127).
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("length must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))    # amax = m * 2^ex, m in [0.5, 1)
    e = np.where(amax > 0, ex - 1 - 2, -127)
    e = np.clip(e, -127, 127)
    q = e2m1_round(blk / np.exp2(e)[..., None])
    return (e + 127).astype(np.uint8), q.reshape(v.shape)


def unpack_fp4(packed):
    """E2M1 codes of a packed array: byte i holds element 2i in its low
    nibble and element 2i + 1 in its high nibble."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def expert_ffn_w4a4(u, c_gu, s_gu, c_d, s_d, intermediates=False):
    """One expert's SwiGLU MLP with MXFP4 weights and activations.

    c_gu [2F,H] / c_d [H,F]: E2M1 codes (one per element); s_gu [2F,H/32] /
    s_d [H,F/32]: E8M0 codes of the blocks of 32 along each row.  For each
    row of u (taken in fp32, as stored):
      (sx, qx) = quantize_mx_fp4(u);  x~ = qx * 2^(sx - 127) per block
      g = x~ W_g~^T, v = x~ W_u~^T   with W~ = E2M1 value * 2^(s - 127)
      a = fp32(silu(g) * v);  (sa, qa) = quantize_mx_fp4(a) over all F
      y = a~ W_d~^T
    The rounding of a to fp32 before its quantisation is the reading taken
    for where the intermediate is stored (the run-time activation
    quantisation reads fp32 values; the decision that picks each code is
    then taken on the same fp32 value the kernel holds).  The products are
    exact and their sums are taken in fp64.
    """
    u = np.atleast_2d(np.asarray(u, np.float64)).astype(np.float32).astype(np.float64)
    def deq(c, s):
        vals = e2m1_decode(c)
        sc = np.repeat(e8m0_decode(s), MX_BLOCK, axis=-1)
        return vals * sc
    wgu = deq(c_gu, s_gu)
    wd = deq(c_d, s_d)
    F = wgu.shape[0] // 2
    sx, qx = quantize_mx_fp4(u)
    xq = qx * np.repeat(e8m0_decode(sx), MX_BLOCK, axis=-1)
    gv = xq @ wgu.T
    a = (silu(gv[:, :F]) * gv[:, F:]).astype(np.float32).astype(np.float64)
    sa, qa = quantize_mx_fp4(a)
    aq = qa * np.repeat(e8m0_decode(sa), MX_BLOCK, axis=-1)
    y = aq @ wd.T
    if intermediates:
        return y, {"xq": xq, "g": gv[:, :F], "v": gv[:, F:], "a": a, "aq": aq, "sx": sx, "sa": sa}
    return y


def combine(y, w):
    """Weighted combine m = sum_k w_k y_k of one token's K expert outputs
    ([TS] "TensorRT-LLM NVFP4 MoE": weighted sum per token; [VL] kernel
    change 3: the norm kernel also combines the top-8 outputs)."""
    y = np.asarray(y, np.float64)
    w = np.asarray(w, np.float64)
    return (w[:, None] * y).sum(axis=0)


# --------------------------------------------------------------------------
# sandwich-norm boundary  ([VL] MoE and residual section: RMSNorm before and
# after every sublayer, n-th residual update h <- sqrt((n-1)/n) h + x/sqrt(n);
# [TS] "MNNVL all-reduce and SandwichNorm fusion": post-norm, depth-scaled
# residual, next pre-norm in one step)
# --------------------------------------------------------------------------

def rmsnorm(v, gamma, eps):
    v = np.asarray(v, np.float64)
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * np.asarray(gamma, np.float64)


def norm_boundary(m, h, gamma_post, gamma_pre, n, eps, rnd=round_bf16):
    """p = rnd(RMSNorm(m) * gamma_post); h' = rnd(sqrt((n-1)/n) h + p/sqrt(n));
    x_next = rnd(RMSNorm(h') * gamma_pre).  Returns (p, h', x_next)."""
    p = rnd(rmsnorm(m, gamma_post, eps))
    h_new = rnd(math.sqrt((n - 1) / n) * np.asarray(h, np.float64) + p / math.sqrt(n))
    x_next = rnd(rmsnorm(h_new, gamma_pre, eps))
    return p, h_new, x_next


# --------------------------------------------------------------------------
# the dense layers and one expert-parallel shard
# --------------------------------------------------------------------------

def dense_layer_tokens(cfg, x, w_gu, w_d, h, gamma_post, gamma_pre, n, tokens=None, rnd=round_bf16):
    """A dense layer's MLP and its sandwich-norm boundary, for the listed tokens.

    The first three layers use a dense SwiGLU MLP with d_ff 20480 instead of
    the MoE ([VL] MoE section; [TS] "Architecture": three dense layers, then
    49 MoE layers), with the same norm before and after every block
    ([TS] "Architecture": SandwichNorm and depth-scaled residuals).  Reading:
    the MLP is the expert MLP of this module over all tokens (a = silu(g) * v
    rounded by rnd, output unrounded) and its output takes the place of the
    MoE output m in the boundary.  Returns dict with y (= m), p, h_new, x_next.
    """
    x = np.asarray(x, np.float64)
    tokens = list(range(x.shape[0])) if tokens is None else list(tokens)
    y = expert_ffn(x[tokens], w_gu, w_d, round_a=rnd)
    p, hn, xn = norm_boundary(y, np.asarray(h, np.float64)[tokens], gamma_post, gamma_pre, n,
                              cfg["rms_eps"], rnd)
    return {"tokens": tokens, "y": y, "p": p, "h_new": hn, "x_next": xn}


def combine_shard(y, ids, w, expert_begin, n_local):
    """One expert-parallel shard's part of a token's combine: the weighted
    sum over the token's experts in [expert_begin, expert_begin + n_local).

    Under EP8 each GPU holds 32 complete experts, processes the tokens routed
    to them and an all-reduce sums the partial MoE outputs; normalisation
    runs after it ([TS] "Tensor parallelism and expert parallelism"; [GD]
    "At a glance": EP 8, 32 experts per card).  The shards' partial sums add
    up to combine(y, w).
    """
    y = np.asarray(y, np.float64)
    ids = np.asarray(ids)
    keep = (ids >= expert_begin) & (ids < expert_begin + n_local)
    w = np.where(keep, np.asarray(w, np.float64), 0.0)
    return (w[:, None] * y).sum(axis=0)


# --------------------------------------------------------------------------
# the layer, for a subset of tokens
# --------------------------------------------------------------------------

def layer_tokens(cfg, x, w_r, bias, expert_weights, h, gamma_post, gamma_pre, n,
                 tokens=None, w_dtype="bf16", rnd=round_bf16, ids_override=None):
    """Whole layer for the listed tokens (default: all).

    x, h [T,H]; w_r [E,H]; bias [E]; gammas [H] (numpy, any float dtype).
    expert_weights(e) returns {"w_gu","w_d"} (float),
    {"q_gu","s_gu","q_d","s_d"} (w_dtype "fp8") or {"c_gu","s_gu","c_d","s_d"}
    (w_dtype "mxfp4": E2M1 codes and E8M0 block scales).  rnd is the storage
    rounding of a, p, h', x_next (round_bf16, or round_f32 for the all-fp32
    layer).  ids_override {t: ids} replaces a token's chosen experts (used
    to re-evaluate near-tie tokens with another valid choice).

    Returns a dict with, per listed token: route, y [K,H], m, p, h_new, x_next.
    """
    x = np.asarray(x, np.float64)
    T = x.shape[0]
    tokens = list(range(T)) if tokens is None else list(tokens)
    logits = router_logits(x[tokens], w_r)
    routes = [route_token(logits[i], bias, cfg) for i in range(len(tokens))]
    if ids_override:
        for i, t in enumerate(tokens):
            if t in ids_override:
                r = routes[i]
                ids = np.asarray(ids_override[t], dtype=np.int64)
                sk = r.scores[ids]
                r.ids = ids
                r.weights = cfg["routed_scale"] * sk / sk.sum()
    need = sorted({int(e) for r in routes for e in r.ids})
    y = {i: np.empty((cfg["topk"], cfg["hidden"])) for i in range(len(tokens))}
    for e in need:
        wts = expert_weights(e)
        for i, r in enumerate(routes):
            for k, ek in enumerate(r.ids):
                if ek != e:
                    continue
                u = x[tokens[i]]
                if w_dtype == "fp8":
                    y[i][k] = expert_ffn_w8a8(u, wts["q_gu"], wts["s_gu"], wts["q_d"], wts["s_d"])[0]
                elif w_dtype == "mxfp4":
                    y[i][k] = expert_ffn_w4a4(u, wts["c_gu"], wts["s_gu"], wts["c_d"], wts["s_d"])[0]
                else:
                    y[i][k] = expert_ffn(u, wts["w_gu"], wts["w_d"], round_a=rnd)[0]
    out = {"tokens": tokens, "routes": routes, "logits": logits, "y": [], "m": [],
           "p": [], "h_new": [], "x_next": []}
    h = np.asarray(h, np.float64)
    for i, t in enumerate(tokens):
        m = combine(y[i], routes[i].weights)
        p, hn, xn = norm_boundary(m, h[t], gamma_post, gamma_pre, n, cfg["rms_eps"], rnd)
        out["y"].append(y[i])
        out["m"].append(m)
        out["p"].append(p)
        out["h_new"].append(hn)
        out["x_next"].append(xn)
    for k in ("y", "m", "p", "h_new", "x_next"):
        out[k] = np.array(out[k])
    return out
