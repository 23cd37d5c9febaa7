"""Host-side checks of bench.py's contract and of the figures it reports:
the one-GPU refusal, the algorithmic bytes and flops behind `roofline`, and
the choice between the HBM and the matrix-core roof.  No GPU is used."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

H, F, E, K = 5120, 2560, 256, 8


def test_multi_gpu_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_ridge_rows():
    # flops per weight byte at MFMA peak / HBM peak; 2 flops per weight per row
    assert bench.ridge_rows("bf16") == pytest.approx(2500e12 / 8000e9 / (2 / 2.0))
    assert bench.ridge_rows("bf16") == pytest.approx(312.5)
    assert bench.ridge_rows("fp8") == pytest.approx(312.5)
    # E2M1 half-bytes plus one E8M0 byte per 32 weights
    assert bench.ridge_rows("mxfp4") == pytest.approx(10100e12 / 8000e9 * (0.5 + 1 / 32) / 2)


def test_algorithmic_bf16_decode():
    wl = synth.WORKLOADS["decode_t8"]
    D = 60
    a = bench.algorithmic(wl, D)
    # gate, up and down projections of one expert: 3 * H * F bf16 weights
    assert a["w_expert"] == 3 * 5120 * 2560 * 2 == 78_643_200
    assert a["experts_bytes"] == D * 78_643_200 + 8 * H * 2
    # W_r in fp32, and x, h in / h', x_next out in bf16
    assert a["layer_bytes"] == D * 78_643_200 + E * H * 4 + 4 * 8 * H * 2
    # GEMM1 2*H*2F + GEMM2 2*F*H per (token, expert) pair; router 2*H*E per token
    assert a["experts_flops"] == 8 * K * (2 * H * 2 * F + 2 * F * H)
    assert a["layer_flops"] == a["experts_flops"] + 8 * 2 * H * E


def test_algorithmic_fp8_and_mxfp4():
    fp8 = synth.WORKLOADS["prefill_fp8_t16384"]
    a = bench.algorithmic(fp8, 256)
    # e4m3 weights and one fp32 scale per output row (2F rows of GEMM1, H of GEMM2)
    assert a["w_expert"] == 3 * H * F + (2 * F + H) * 4
    # e4m3 activation codes and one fp32 scale per token
    assert a["experts_bytes"] == 256 * a["w_expert"] + 16384 * H + 16384 * 4
    mx = synth.WORKLOADS["decode_t8_mxfp4"]
    b = bench.algorithmic(mx, 10)
    n_w = 3 * H * F
    assert b["w_expert"] == n_w // 2 + n_w // 32
    assert b["experts_bytes"] == 10 * b["w_expert"] + 8 * H // 2 + 8 * H // 32


def fake_run(us, touched, ms_per_step):
    return {"touched": touched, "per": {"experts": [us, us]}, "ms_per_step": ms_per_step}


def test_roofline_bound_choice():
    # decode: 8 tokens * 8 / 60 experts is far below the ridge -> HBM roof
    wl = synth.WORKLOADS["decode_t8"]
    roof, layer = bench.roofline_entry(wl, fake_run(700.0, 60, 0.75))
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    want = (60 * 78_643_200 + 8 * H * 2) / 700e-6 / 1e9
    assert roof["achieved"] == pytest.approx(want, abs=0.05)
    assert roof["frac"] == pytest.approx(want / 8000.0, abs=1e-4)
    assert 0 < layer["hbm_frac"] < roof["frac"]
    # T = 16384: 512 rows per expert -> matrix-core roof at the dtype's own peak
    for name, peak in (("prefill_bf16_t16384", 2500.0), ("prefill_fp8_t16384", 5000.0)):
        wl = synth.WORKLOADS[name]
        roof, _ = bench.roofline_entry(wl, fake_run(6000.0, 256, 6.5))
        assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == peak
        flops = 16384 * K * 6 * H * F
        assert roof["achieved"] == pytest.approx(flops / 6000e-6 / 1e12, abs=0.05)
    # T = 2048: 64 rows per expert stays below the ridge
    wl = synth.WORKLOADS["prefill_t2048"]
    roof, _ = bench.roofline_entry(wl, fake_run(3600.0, 256, 3.7))
    assert roof["bound"] == "hbm"


def test_traffic_lookup():
    # an unknown workload or call has no measured traffic
    assert bench.traffic_for("no_such_workload") is None
    assert bench.traffic_for("decode_t8", call="no_such_call") is None
    rec = json.load(open(bench.TRAFFIC_FILE)).get("decode_t8", {}).get("experts")
    got = bench.traffic_for("decode_t8")
    if rec is not None and rec.get("kernel_src_hash") == bench.kernel_hash():
        assert got == rec["bytes_per_call"]
    else:   # counters taken on another expert-kernel source are not reported
        assert got is None
