"""Pins of the oracle's storage formats (bf16, fp32, e4m3) against library
conversions, brute force over the code table and the OCP FP8 spec values."""

import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_bf16(v32):
    return torch.from_numpy(np.asarray(v32, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_matches_torch_on_fp32_inputs():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(100000) * 10.0 ** rng.integers(-38, 38, 100000),
        rng.standard_normal(1000) * 1e-40,            # fp32 subnormals
        np.array([3.38e38, 3.39e38, -3.3895e38, 1e-45, 0.0, -0.0]),
    ]).astype(np.float32)
    got = oracle.round_bf16(v.astype(np.float64))
    ref = _torch_bf16(v)
    np.testing.assert_array_equal(got, ref)


def test_bf16_rounds_from_fp64_without_double_rounding():
    # 1 + 2^-8 + 2^-30 lies above the midpoint between the bf16 neighbours
    # 1 and 1 + 2^-7, but rounds to that midpoint in fp32 (then to even: 1).
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.round_bf16(np.array([v]))[0] == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0        # exact tie -> even
    assert oracle.round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


def test_bf16_specials():
    v = np.array([np.nan, np.inf, -np.inf, 0.0, 1e300])
    r = oracle.round_bf16(v)
    assert np.isnan(r[0]) and r[1] == np.inf and r[2] == -np.inf and r[3] == 0.0 and r[4] == np.inf


def test_f32_matches_numpy_cast_semantics():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(1000) * 1e3
    r = oracle.round_f32(v)
    assert np.all(np.abs(r - v) <= np.abs(v) * 2.0 ** -24)
    assert np.all(r.astype(np.float32).astype(np.float64) == r)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])


def test_e4m3_decode_spec_table():
    spec = json.load(open(os.path.join(GOLDEN, "e4m3_spec.json")))
    for code, val in spec["codes"].items():
        got = oracle.e4m3_decode(np.array([int(code)]))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)
    for code in spec["nan_codes"]:
        assert np.isnan(oracle.e4m3_decode(np.array([code]))[0])


def _nearest_code_brute(v, finite_vals, finite_codes):
    """Nearest finite e4m3 value by exhaustive search; ties pick the even
    mantissa (code with bit 0 clear); |v| > 448 saturates."""
    out = np.empty_like(v)
    for i, x in enumerate(v):
        d = np.abs(finite_vals - x)
        best = np.flatnonzero(d == d.min())
        if len(best) > 1:
            even = [b for b in best if (finite_codes[b] & 1) == 0]
            # +0 and -0 are both at distance |x| from x=0-ish values; prefer
            # the one with the sign of x
            best = even if even else list(best)
        vals = finite_vals[best]
        if len(vals) > 1:
            vals = vals[np.signbit(vals) == np.signbit(x)] if np.any(np.signbit(vals) == np.signbit(x)) else vals
        out[i] = vals[0]
    return out


def test_e4m3_round_matches_brute_force_nearest():
    codes = np.arange(256)
    vals = oracle.e4m3_decode(codes)
    fin = np.isfinite(vals)
    fvals, fcodes = vals[fin], codes[fin]
    rng = np.random.default_rng(2)
    # dense sweep over the whole range incl. subnormals, exact midpoints, and saturation
    mids = (np.sort(np.unique(fvals))[1:] + np.sort(np.unique(fvals))[:-1]) / 2
    v = np.concatenate([
        rng.uniform(-460, 460, 20000),
        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 9, 20000),
        mids, -mids, np.unique(fvals),
    ])
    got = oracle.e4m3_round(v)
    ref = _nearest_code_brute(np.clip(v, -448, 448), fvals, fcodes)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_round_matches_torch_in_range():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(200000) * 2.0 ** rng.integers(-12, 8, 200000)).astype(np.float32)
    v = np.clip(v, -448, 448)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_round(v.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_e4m3_round_saturates_and_keeps_nan():
    r = oracle.e4m3_round(np.array([500.0, -1e9, np.inf, -np.inf, np.nan, 464.0, 465.0]))
    assert list(r[:4]) == [448.0, -448.0, 448.0, -448.0]
    assert np.isnan(r[4]) and r[5] == 448.0 and r[6] == 448.0


def test_quantize_row_maps_amax_to_448():
    rng = np.random.default_rng(4)
    for _ in range(20):
        v = rng.standard_normal(777) * rng.uniform(1e-3, 1e3)
        s, q = oracle.quantize_row_e4m3(v)
        i = np.argmax(np.abs(v))
        assert abs(q[i]) == 448.0
        assert np.all(np.abs(q) <= 448.0)
        # every quantised value is an e4m3 grid value
        assert np.array_equal(oracle.e4m3_round(q), q)
        # dequantised error of the largest entries is within half an e4m3 step (2^-4 relative)
        big = np.abs(v) > np.abs(v).max() / 4
        assert np.all(np.abs(q[big] * s - v[big]) <= np.abs(v[big]) * 2.0 ** -4 * 1.0001)


def test_quantize_row_zero():
    s, q = oracle.quantize_row_e4m3(np.zeros(16))
    assert s == 1.0 and np.all(q == 0)
