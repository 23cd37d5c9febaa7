"""Pins of the oracle's 4-bit (MXFP4) path: the E2M1 element codec against
the format's value table and a brute-force nearest-value search, the E8M0
scale decode against the table and torch's own float8_e8m0fnu type, the
block quantisation's defining properties, and the W4A4 expert's structure
(lossless cases, gate/up order, transposition, scale placement)."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _spec():
    return json.load(open(os.path.join(GOLDEN, "e2m1_spec.json")))


def test_e2m1_decode_all_codes():
    g = _spec()
    got = oracle.e2m1_decode(np.array(g["codes"]))
    np.testing.assert_array_equal(got, np.array(g["values"]))
    assert np.all(np.signbit(got[8:]))


def test_e8m0_decode_table_and_torch():
    g = _spec()
    got = oracle.e8m0_decode(np.array(g["scale_codes"]))
    want = np.array([np.nan if v is None else v for v in g["scale_values"]])
    np.testing.assert_array_equal(got, want)
    codes = np.arange(255, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e8m0_decode(codes), t)


def _brute_nearest(x):
    """Nearest E2M1 value by exhaustive search over the 15 distinct values,
    ties to the code with even mantissa bit, saturating beyond +-6."""
    vals = oracle.e2m1_decode(np.arange(16))
    out = np.empty_like(x)
    for i, v in enumerate(x):
        if abs(v) >= 6:
            out[i] = math.copysign(6.0, v)
            continue
        d = np.abs(vals - v)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            best = [c for c in best if (c & 1) == 0] or best
        out[i] = abs(vals[best[0]]) * (1 if v >= 0 else -1) if vals[best[0]] != 0 else 0.0
    return out


def test_e2m1_round_matches_brute_force():
    rng = np.random.default_rng(0)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    grid = oracle.e2m1_decode(np.arange(8))
    x = np.concatenate([rng.uniform(-8, 8, 20000), mids, -mids, grid, -grid,
                        np.nextafter(mids, 0), np.nextafter(mids, 9), [6.0, 6.5, 100.0, -1e9]])
    got = oracle.e2m1_round(x)
    want = _brute_nearest(x)
    np.testing.assert_array_equal(np.abs(got), np.abs(want))
    nz = got != 0
    np.testing.assert_array_equal(np.sign(got[nz]), np.sign(x[nz]))
    assert np.isnan(oracle.e2m1_round([np.nan]))[0]
    np.testing.assert_array_equal(oracle.e2m1_round([np.inf, -np.inf]), [6.0, -6.0])


def test_e2m1_encode_round_trip():
    codes = np.arange(16, dtype=np.uint8)
    vals = oracle.e2m1_decode(codes)
    back = oracle.e2m1_encode(vals)
    # -0 encodes as 8 (sign bit set), the rest exactly
    np.testing.assert_array_equal(back, codes)
    with pytest.raises(ValueError):
        oracle.e2m1_encode([0.7])


def test_quantize_mx_block_properties():
    rng = np.random.default_rng(1)
    v = rng.standard_normal((5, 256)) * np.exp2(rng.integers(-20, 20, (5, 1)))
    v[2, 32:64] = 0.0                                   # an all-zero block
    s, q = oracle.quantize_mx_fp4(v)
    assert s.shape == (5, 8) and q.shape == v.shape
    scale = np.repeat(oracle.e8m0_decode(s), 32, axis=-1)
    blk = np.abs(v).reshape(5, 8, 32).max(axis=-1)
    r = np.where(blk > 0, blk / oracle.e8m0_decode(s), 4.0)
    assert np.all((r >= 4) & (r < 8))                   # amax lands in [4, 8) before rounding
    np.testing.assert_array_equal(q, oracle.e2m1_round(v / scale))
    assert np.all(q[2, 32:64] == 0) and s[2, 1] == 0
    # each block is quantised on its own
    v2 = v.copy()
    v2[:, :32] *= 1000.0
    s2, q2 = oracle.quantize_mx_fp4(v2)
    np.testing.assert_array_equal(s2[:, 1:], s[:, 1:])
    np.testing.assert_array_equal(q2[:, 32:], q[:, 32:])


def test_quantize_mx_lossless_on_grid():
    # blocks whose values are E2M1 values times 2^e with a block maximum of 4
    # or 6 (times 2^e) are reproduced exactly with scale 2^e
    rng = np.random.default_rng(2)
    grid = oracle.e2m1_decode(np.arange(16))
    e = rng.integers(-30, 30, 4)
    el = rng.choice(grid, (4, 32))
    el[:, 5] = rng.choice([4.0, -6.0, 6.0, -4.0], 4)
    v = el * np.exp2(e)[:, None]
    s, q = oracle.quantize_mx_fp4(v.reshape(1, -1))
    np.testing.assert_array_equal(s[0], (e + 127).astype(np.uint8))
    np.testing.assert_array_equal(q.reshape(4, 32), el)


def test_unpack_fp4_nibble_order():
    np.testing.assert_array_equal(oracle.unpack_fp4(np.array([[0x21, 0xF0]], np.uint8)), [[1, 2, 0, 15]])


def _mx_weights(rng, rows, cols, emin=-9, emax=-6):
    c = rng.integers(0, 16, (rows, cols)).astype(np.uint8)
    s = rng.integers(127 + emin, 127 + emax + 1, (rows, cols // 32)).astype(np.uint8)
    return c, s


def _deq(c, s):
    return oracle.e2m1_decode(c) * np.repeat(oracle.e8m0_decode(s), 32, axis=-1)


def test_w4a4_gemm1_lossless_and_layout():
    # activations already on the MX grid are quantised losslessly, so the
    # gate/up pre-activations equal plain fp64 products with the dequantised
    # weights.  Non-square, non-symmetric weights with per-row per-block
    # scales: a transposed operand, a wrong scale block or a swapped gate/up
    # half changes the result.
    rng = np.random.default_rng(3)
    H, F = 128, 64
    grid = oracle.e2m1_decode(np.arange(16))
    el = rng.choice(grid, (3, H))
    el[:, ::32] = 6.0
    ex = rng.integers(-3, 3, (3, H // 32))
    u = el * np.repeat(np.exp2(ex), 32, axis=-1)
    c_gu, s_gu = _mx_weights(rng, 2 * F, H)
    c_d, s_d = _mx_weights(rng, H, F)
    y, it = oracle.expert_ffn_w4a4(u, c_gu, s_gu, c_d, s_d, intermediates=True)
    np.testing.assert_array_equal(it["xq"], u)
    w = _deq(c_gu, s_gu)
    np.testing.assert_allclose(it["g"], u @ w[:F].T, rtol=1e-15, atol=1e-300)
    np.testing.assert_allclose(it["v"], u @ w[F:].T, rtol=1e-15, atol=1e-300)
    a = (it["g"] / (1 + np.exp(-it["g"])) * it["v"]).astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(it["a"], a)
    sa, qa = oracle.quantize_mx_fp4(a)
    np.testing.assert_array_equal(it["aq"], qa * np.repeat(oracle.e8m0_decode(sa), 32, axis=-1))
    np.testing.assert_allclose(y, it["aq"] @ _deq(c_d, s_d).T, rtol=1e-15, atol=1e-300)


def test_w4a4_floor_against_full_precision():
    # W4A4 against the unquantised expert on the same (dequantised) weights:
    # the activation quantisation costs some percent, not more
    rng = np.random.default_rng(4)
    H, F = 512, 256
    u = rng.standard_normal((4, H))
    w_gu = rng.standard_normal((2 * F, H)) / math.sqrt(H)
    w_d = rng.standard_normal((H, F)) / math.sqrt(F)
    s1, q1 = oracle.quantize_mx_fp4(w_gu)
    s2, q2 = oracle.quantize_mx_fp4(w_d)
    c_gu, c_d = oracle.e2m1_encode(q1), oracle.e2m1_encode(q2)
    y4 = oracle.expert_ffn_w4a4(u, c_gu, s1, c_d, s2)
    yf = oracle.expert_ffn(u, _deq(c_gu, s1), _deq(c_d, s2), round_a=None)
    rel = np.linalg.norm(y4 - yf) / np.linalg.norm(yf)
    assert 1e-2 < rel < 0.3, rel


def test_mx_quantiser_matches_independent_checkpoint_quantiser():
    # the MXFP4 checkpoint of the seeded inputs is produced by a separate
    # torch implementation (bucketize over the E2M1 grid); on Gaussian
    # weights the oracle's quantiser must give the same scales and codes
    import dataclasses
    import synth
    wl = synth.Workload("t", T=2, hidden=512, n_experts=4, n_groups=2, topk_groups=1, topk=2,
                        group_topn=2, d_ff=256, routed_scale=2.5, rms_eps=1e-6, n=2, act_dtype="bf16",
                        w_dtype="mxfp4", bias_sigma=0.02, seed=3)
    cgu, cd, sgu, sd = synth.make_expert(wl, 1)
    wgu, wd, _, _ = synth.make_expert(dataclasses.replace(wl, w_dtype="f32"), 1)
    for c, s, w in ((cgu, sgu, wgu), (cd, sd, wd)):
        s_o, q_o = oracle.quantize_mx_fp4(w.double().numpy())
        np.testing.assert_array_equal(s.numpy(), s_o)
        np.testing.assert_array_equal(oracle.e2m1_decode(oracle.unpack_fp4(c.numpy())), q_o)
