"""Host-side checks of the C ABI (no GPU needed, no kernel is launched):
the library loads and exports every function the header declares, and
invalid calls are rejected with the documented status before anything is
enqueued."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")

beam = pytest.importorskip("expert_routed_ffn_amd")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(beam.LIB_PATH):
        pytest.skip("library not built")
    return beam.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(beam_moe_\w+)\s*\(", text)))


def test_header_declares_the_layer_calls():
    d = _declared()
    for name in ("beam_moe_route", "beam_moe_permute", "beam_moe_experts", "beam_moe_combine_norm",
                 "beam_moe_workspace_bytes", "beam_moe_status_string"):
        assert name in d


def test_every_declared_symbol_is_exported(L):
    for name in _declared():
        assert hasattr(L, name), name
    assert sorted(beam.SYMBOLS) == _declared()


def test_status_strings(L):
    for code, text in beam.STATUS.items():
        assert L.beam_moe_status_string(code).decode() == text
    assert L.beam_moe_status_string(99).decode() == "unknown status"


def _cfg(**kw):
    return beam.LayerCfg(**kw).c()


FAKE = 0x10000   # never dereferenced: every call below fails validation first


def _route(L, cfg, T=8, x=FAKE, x_dt=beam.BEAM_BF16, w=FAKE, b=FAKE, ids=FAKE, wt=FAKE, lg=None,
           ws=FAKE, wsb=1 << 30):
    return L.beam_moe_route(ctypes.byref(cfg), T, x, x_dt, w, b, ids, wt, lg, ws, wsb, None)


@pytest.mark.parametrize("bad", [
    dict(hidden=100), dict(hidden=8448), dict(n_experts=512), dict(n_groups=3),
    dict(topk_groups=9), dict(topk=33), dict(group_topn=5), dict(d_ff=100),
    dict(routed_scale=0.0), dict(rms_eps=-1.0), dict(topk=0), dict(n_experts=256, n_groups=256, topk_groups=4),
])
def test_invalid_cfg_rejected(L, bad):
    st = _route(L, _cfg(**bad))
    assert st in (1, 2), (bad, st)


def test_route_argument_checks(L):
    c = _cfg()
    assert _route(L, c, T=-1) == 1
    assert _route(L, c, x=None) == 1
    assert _route(L, c, ids=None) == 1
    assert _route(L, c, x_dt=beam.BEAM_FP8_E4M3) == 1
    assert _route(L, c, x=FAKE + 2) == 1                    # misaligned
    assert _route(L, c, ws=None) == 3                       # logits need workspace
    assert _route(L, c, wsb=16) == 3
    assert L.beam_moe_route(None, 8, FAKE, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1


def test_zero_tokens_is_a_no_op(L):
    c = _cfg()
    # T == 0 returns before touching any pointer (all null here)
    assert L.beam_moe_route(ctypes.byref(c), 0, None, 1, None, None, None, None, None, None, 0, None) == 0
    assert L.beam_moe_permute(ctypes.byref(c), 0, None, None, None, None, None, 1, None, None, None, 0, None) == 0
    assert L.beam_moe_experts(ctypes.byref(c), 0, 1, None, 1, None, None, None, None, None, None, None,
                              None, 0, None, 0, None) == 0
    assert L.beam_moe_combine_norm(ctypes.byref(c), 0, None, 0, None, None, None, None, 1, None, None,
                                   1, None, None) == 0


def test_permute_argument_checks(L):
    c = _cfg()
    f = lambda **kw: L.beam_moe_permute(
        ctypes.byref(c), kw.get("T", 8), kw.get("ids", FAKE), FAKE, FAKE, FAKE, kw.get("x", None),
        kw.get("xdt", 1), kw.get("xq", None), kw.get("xs", None), kw.get("ws", None), kw.get("wsb", 0), None)
    assert f(ids=None) == 1
    assert f(xq=FAKE) == 1                 # x_q needs x and x_scale
    assert f(xq=FAKE, x=FAKE, xs=FAKE, xdt=0) == 1
    assert f(T=4096) == 3                  # multi-block permutation needs workspace
    assert f(T=4096, ws=FAKE + 4, wsb=1 << 30) == 3   # ... 16-byte aligned


def test_experts_argument_checks(L):
    c = _cfg()

    def f(T=8, w_dt=1, x_dt=1, xs=None, sgu=None, sd=None, y_dt=0, ws=FAKE, wsb=1 << 40, x=FAKE, y=FAKE):
        return L.beam_moe_experts(ctypes.byref(c), T, w_dt, x, x_dt, xs, FAKE, FAKE, FAKE, sgu, FAKE,
                                  sd, y, y_dt, ws, wsb, None)

    assert f(x_dt=0) == 1                      # activation dtype must match the weights
    assert f(y_dt=2) == 1                      # y cannot be fp8
    assert f(w_dt=2, x_dt=2) == 1              # fp8 needs scales
    assert f(ws=None) == 3
    assert f(wsb=1024) == 3
    assert f(x=None) == 1
    assert f(y=FAKE + 4) == 1
    assert f(w_dt=7, x_dt=7) == 1
    assert f(T=-1) == 1
    assert f(T=(1 << 22) + 1) == 1             # beyond the largest token count
    # 4-bit experts: any batch (all three GEMM paths), hidden and d_ff
    # multiples of 512
    mx = dict(w_dt=3, x_dt=3, xs=FAKE, sgu=FAKE, sd=FAKE)
    assert f(T=8, ws=None, **mx) == 3          # past the shape checks: on to the workspace check
    assert f(T=16384, ws=None, **mx) == 3
    c2 = _cfg(d_ff=2304)
    assert L.beam_moe_experts(ctypes.byref(c2), 8, 3, FAKE, 3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              0, FAKE, 1 << 40, None) == 2


def test_combine_argument_checks(L):
    c = _cfg()

    def f(n=20, y_dt=0, a_dt=1, h=FAKE, xn=FAKE + 4096):
        return L.beam_moe_combine_norm(ctypes.byref(c), 8, FAKE, y_dt, FAKE, FAKE, h, xn, a_dt, FAKE,
                                       FAKE, n, None, None)

    assert f(n=0) == 1
    assert f(y_dt=2) == 1
    assert f(a_dt=2) == 1
    assert f(h=None) == 1
    assert f(xn=FAKE) == 1                     # x_next must not alias h


def test_workspace_bytes(L):
    c = _cfg()
    sizes = [L.beam_moe_workspace_bytes(ctypes.byref(c), T, 1) for T in (1, 8, 64, 2048, 16384)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    # fp8 keeps an fp32 intermediate plus codes
    assert L.beam_moe_workspace_bytes(ctypes.byref(c), 16384, 2) > sizes[-1]
    assert L.beam_moe_workspace_bytes(ctypes.byref(c), -1, 1) == 0
    assert L.beam_moe_workspace_bytes(ctypes.byref(_cfg(hidden=100)), 8, 1) == 0
    # small expert counts (no matrix-core router tiles) and every dtype
    tiny = beam.LayerCfg(256, 16, 4, 2, 4, 2, 128).c()
    for dt in (0, 1):
        for T in (1, 4, 17, 33, 1000):
            assert L.beam_moe_workspace_bytes(ctypes.byref(tiny), T, dt) > 0


def test_pack_argument_checks(L):
    c = _cfg()
    f = lambda n=2, dt=1, a=FAKE, b=FAKE * 1024, pa=FAKE * 4096, pb=FAKE * 8192: L.beam_moe_pack_weights(
        ctypes.byref(c), n, dt, a, b, pa, pb, None)
    assert f(n=0) == 0                        # nothing to do
    assert f(n=-1) == 1
    assert f(dt=5) == 1
    assert f(a=None) == 1
    assert f(pa=FAKE + 8) == 1                # misaligned
    assert f(pa=FAKE) == 1                    # output overlaps its input
    assert f(pb=FAKE * 4096 + 4096) == 1      # outputs overlap each other
    assert L.beam_moe_pack_weights(ctypes.byref(_cfg(d_ff=384)), 1, 2, FAKE, FAKE * 1024, FAKE * 4096,
                                   FAKE * 8192, None) == 2   # fp8 needs d_ff % 256 == 0


def test_experts_static_checks(L):
    c = _cfg()
    f = lambda T=8, x_dt=1, y_dt=0, x=FAKE: L.beam_moe_experts_static(
        ctypes.byref(c), T, 1, x, x_dt, None, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, y_dt, None)
    assert f(T=0, x=None) == 0                 # nothing to do
    assert f(x_dt=0) == 1                      # same argument checks as beam_moe_experts
    assert f(y_dt=2) == 1
    assert f(x=None) == 1
    # the Beam shape at T = 4096 needs more than the 64 MiB static scratch:
    # rejected before anything is enqueued
    assert L.beam_moe_workspace_bytes(ctypes.byref(c), 4096, 1) > beam.STATIC_SCRATCH_BYTES
    assert f(T=4096) == 2


def test_shard_dense_norm_checks(L):
    c = _cfg()
    # permute_shard: the expert range must lie inside the layer's experts
    ps = lambda eb=0, n=32, T=8: L.beam_moe_permute_shard(ctypes.byref(c), T, eb, n, FAKE, FAKE, FAKE, FAKE,
                                                         None, 0, None)
    assert ps(eb=-1) == 1
    assert ps(eb=240, n=32) == 1
    assert ps(n=0) == 1
    assert ps(T=0) == 0
    assert ps(T=4096) == 3                     # multi-block permutation needs workspace
    # combine_partial: fp32 output required, y dtype checked
    cp = lambda y_dt=0, m=FAKE: L.beam_moe_combine_partial(ctypes.byref(c), 8, FAKE, y_dt, FAKE, FAKE, m, None)
    assert cp(y_dt=2) == 1
    assert cp(m=None) == 1
    # norm boundary: residual index >= 1, no aliasing of h and x_next
    nb = lambda n=20, h=FAKE, xn=FAKE + 4096: L.beam_moe_norm_boundary(ctypes.byref(c), 8, FAKE, 0, h, xn, 1,
                                                                       FAKE, FAKE, n, None)
    assert nb(n=0) == 1
    assert nb(xn=FAKE) == 1
    # dense MLP: d_ff a multiple of 128 and at most 32768, bf16 input, workspace
    dm = lambda d_ff=20480, x_dt=1, ws=FAKE, wsb=1 << 40: L.beam_moe_dense_mlp(
        ctypes.byref(c), 8, d_ff, FAKE, x_dt, FAKE, FAKE, FAKE, ws, wsb, None)
    assert dm(d_ff=20000) == 2
    assert dm(d_ff=65536) == 2
    assert dm(x_dt=0) == 1
    assert dm(ws=None) == 3
    assert dm(wsb=1024) == 3
    # at least the bf16 SwiGLU output [T, d_ff] plus the K-split partial sums
    assert L.beam_moe_dense_workspace_bytes(ctypes.byref(c), 8, 20480) >= 8 * 20480 * 2 + 8 * 8 * 5120 * 4
    assert L.beam_moe_dense_workspace_bytes(ctypes.byref(c), 8, 2560) > 0
    assert L.beam_moe_dense_workspace_bytes(ctypes.byref(c), 8, 100) == 0


def test_quantize_argument_checks(L):
    c = _cfg()
    # e4m3 input quantisation: bf16 input, codes and scales required, codes 16-byte aligned
    q8 = lambda T=8, x=FAKE, dt=1, xq=FAKE, xs=FAKE: L.beam_moe_quantize_fp8(ctypes.byref(c), T, x, dt, xq, xs,
                                                                             None)
    assert q8(T=0, x=None, xq=None, xs=None) == 0
    assert q8(T=-1) == 1
    assert q8(dt=0) == 1
    assert q8(xs=None) == 1
    assert q8(xq=FAKE + 4) == 1
    # MXFP4 input quantisation: bf16 or fp32 input, hidden a multiple of 512
    qm = lambda T=8, dt=1, cfg=c: L.beam_moe_quantize_mx(ctypes.byref(cfg), T, FAKE, dt, FAKE, FAKE, None)
    assert qm(dt=2) == 1
    assert qm(cfg=_cfg(hidden=5184, n_experts=256)) == 2
