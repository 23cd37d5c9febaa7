"""Python binding of libbeam_moe.so: one Beam-style MoE layer forward on
MI355X (gfx950).

The functions below carry the C entry points' names and do argument
marshalling only: they check that the torch tensors are contiguous device
tensors of the expected dtype and shape, then pass their data pointers and
the current HIP stream to the library.  Every step of the layer runs in the
library's HIP kernels; there is no fallback of any kind.  If the library is
missing, importing this package still works but every call raises.

Layer (TokenSpeed x Reflection Beam blog, "Architecture"; vLLM Beam summary,
MoE and residual section):
    route -> permute -> experts -> combine_norm
"""

from __future__ import annotations

import ctypes
import dataclasses
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbeam_moe.so")

BEAM_F32, BEAM_BF16, BEAM_FP8_E4M3, BEAM_MXFP4 = 0, 1, 2, 3
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape or dtype",
          3: "workspace missing or too small", 4: "HIP launch failed"}

SYMBOLS = ("beam_moe_route", "beam_moe_permute", "beam_moe_quantize_fp8", "beam_moe_quantize_mx", "beam_moe_experts",
           "beam_moe_experts_static", "beam_moe_combine_norm", "beam_moe_norm_boundary",
           "beam_moe_permute_shard", "beam_moe_combine_partial", "beam_moe_dense_mlp",
           "beam_moe_dense_workspace_bytes", "beam_moe_pack_weights", "beam_moe_workspace_bytes",
           "beam_moe_status_string")
STATIC_SCRATCH_BYTES = 64 << 20   # BEAM_MOE_STATIC_SCRATCH_BYTES


class BeamMoeCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("group_topn", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("routed_scale", ctypes.c_float),
                ("rms_eps", ctypes.c_float)]


@dataclasses.dataclass(frozen=True)
class LayerCfg:
    """Shape of one MoE layer.  Beam defaults."""
    hidden: int = 5120
    n_experts: int = 256
    n_groups: int = 8
    topk_groups: int = 4
    topk: int = 8
    group_topn: int = 2
    d_ff: int = 2560
    routed_scale: float = 2.5
    rms_eps: float = 1e-6

    def c(self) -> BeamMoeCfg:
        return BeamMoeCfg(self.hidden, self.n_experts, self.n_groups, self.topk_groups, self.topk,
                          self.group_topn, self.d_ff, self.routed_scale, self.rms_eps)


class BeamError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first use; raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(BeamMoeCfg)
    L.beam_moe_route.argtypes = [cfgp, i32, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.beam_moe_permute.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    L.beam_moe_experts.argtypes = [cfgp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                   vp, sz, vp]
    L.beam_moe_experts_static.argtypes = [cfgp, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp]
    L.beam_moe_quantize_mx.argtypes = [cfgp, i32, vp, i32, vp, vp, vp]
    L.beam_moe_quantize_fp8.argtypes = [cfgp, i32, vp, i32, vp, vp, vp]
    L.beam_moe_norm_boundary.argtypes = [cfgp, i32, vp, i32, vp, vp, i32, vp, vp, i32, vp]
    L.beam_moe_permute_shard.argtypes = [cfgp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.beam_moe_combine_partial.argtypes = [cfgp, i32, vp, i32, vp, vp, vp, vp]
    L.beam_moe_dense_mlp.argtypes = [cfgp, i32, i32, vp, i32, vp, vp, vp, vp, sz, vp]
    L.beam_moe_dense_workspace_bytes.argtypes = [cfgp, i32, i32]
    L.beam_moe_dense_workspace_bytes.restype = sz
    L.beam_moe_combine_norm.argtypes = [cfgp, i32, vp, i32, vp, vp, vp, vp, i32, vp, vp, i32, vp, vp]
    L.beam_moe_pack_weights.argtypes = [cfgp, i32, i32, vp, vp, vp, vp, vp]
    L.beam_moe_workspace_bytes.argtypes = [cfgp, i32, i32]
    L.beam_moe_workspace_bytes.restype = sz
    L.beam_moe_status_string.argtypes = [i32]
    L.beam_moe_status_string.restype = ctypes.c_char_p
    for f in ("beam_moe_route", "beam_moe_permute", "beam_moe_quantize_mx", "beam_moe_experts",
              "beam_moe_experts_static", "beam_moe_combine_norm", "beam_moe_norm_boundary",
              "beam_moe_permute_shard", "beam_moe_combine_partial", "beam_moe_dense_mlp",
              "beam_moe_pack_weights"):
        getattr(L, f).restype = i32
    _lib = L
    return L


# ------------------------------------------------------------------ helpers

def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return BEAM_F32
    if t.dtype == torch.bfloat16:
        return BEAM_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return BEAM_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _check(t, shape, dtypes, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ok(fn, status):
    if status != 0:
        raise BeamError(fn, status)


def workspace_bytes(cfg: LayerCfg, T: int, w_dtype: int) -> int:
    return int(lib().beam_moe_workspace_bytes(ctypes.byref(cfg.c()), T, w_dtype))


def workspace(cfg: LayerCfg, T: int, w_dtype: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_bytes(cfg, T, w_dtype), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points

def beam_moe_route(cfg: LayerCfg, x, w_router, bias, topk_ids, topk_w, logits_out=None, ws=None,
                   stream=None):
    T = x.shape[0]
    _check(x, (T, cfg.hidden), (torch.bfloat16, torch.float32), "x")
    _check(w_router, (cfg.n_experts, cfg.hidden), (torch.float32,), "w_router")
    _check(bias, (cfg.n_experts,), (torch.float32,), "bias")
    _check(topk_ids, (T, cfg.topk), (torch.int32,), "topk_ids")
    _check(topk_w, (T, cfg.topk), (torch.float32,), "topk_w")
    if logits_out is not None:
        _check(logits_out, (T, cfg.n_experts), (torch.float32,), "logits_out")
    st = lib().beam_moe_route(ctypes.byref(cfg.c()), T, _p(x), _dt(x), _p(w_router), _p(bias),
                              _p(topk_ids), _p(topk_w), _p(logits_out), _p(ws),
                              0 if ws is None else ws.numel(), _stream(stream))
    _ok("beam_moe_route", st)


def beam_moe_permute(cfg: LayerCfg, topk_ids, expert_offsets, row_token, pair_row, x=None,
                     x_q=None, x_scale=None, ws=None, stream=None):
    T = topk_ids.shape[0]
    TK = T * cfg.topk
    _check(topk_ids, (T, cfg.topk), (torch.int32,), "topk_ids")
    _check(expert_offsets, (cfg.n_experts + 1,), (torch.int32,), "expert_offsets")
    _check(row_token, (TK,), (torch.int32,), "row_token")
    _check(pair_row, (TK,), (torch.int32,), "pair_row")
    if x_q is not None:
        _check(x, (T, cfg.hidden), (torch.bfloat16,), "x")
        _check(x_q, (T, cfg.hidden), (torch.uint8, torch.float8_e4m3fn), "x_q")
        _check(x_scale, (T,), (torch.float32,), "x_scale")
    st = lib().beam_moe_permute(ctypes.byref(cfg.c()), T, _p(topk_ids), _p(expert_offsets),
                                _p(row_token), _p(pair_row), _p(x), BEAM_BF16, _p(x_q),
                                _p(x_scale), _p(ws), 0 if ws is None else ws.numel(),
                                _stream(stream))
    _ok("beam_moe_permute", st)


def beam_moe_quantize_fp8(cfg: LayerCfg, x, x_q, x_scale, stream=None):
    """Dynamic per-token e4m3 quantisation of x [T,H] (bf16) into codes x_q
    [T,H] (uint8/float8_e4m3fn) and fp32 scales x_scale [T]."""
    T, H = x.shape[0], cfg.hidden
    _check(x, (T, H), (torch.bfloat16,), "x")
    _check(x_q, (T, H), (torch.uint8, torch.float8_e4m3fn), "x_q")
    _check(x_scale, (T,), (torch.float32,), "x_scale")
    st = lib().beam_moe_quantize_fp8(ctypes.byref(cfg.c()), T, _p(x), _dt(x), _p(x_q), _p(x_scale),
                                     _stream(stream))
    _ok("beam_moe_quantize_fp8", st)


def beam_moe_quantize_mx(cfg: LayerCfg, x, x_q, x_scale, stream=None):
    """Run-time MXFP4 quantisation of x [T,H] (bf16/f32) into packed E2M1
    codes x_q [T,H/2] and E8M0 block scales x_scale [T,H/32] (uint8)."""
    T, H = x.shape[0], cfg.hidden
    _check(x, (T, H), (torch.bfloat16, torch.float32), "x")
    _check(x_q, (T, H // 2), (torch.uint8,), "x_q")
    _check(x_scale, (T, H // 32), (torch.uint8,), "x_scale")
    st = lib().beam_moe_quantize_mx(ctypes.byref(cfg.c()), T, _p(x), _dt(x), _p(x_q), _p(x_scale),
                                    _stream(stream))
    _ok("beam_moe_quantize_mx", st)


def _w_dtype(w_gate_up, s_gate_up):
    """MXFP4 stacks are uint8 E2M1 bytes with uint8 E8M0 scales; fp8 stacks
    carry fp32 row scales."""
    if w_gate_up.dtype == torch.uint8 and s_gate_up is not None and s_gate_up.dtype == torch.uint8:
        return BEAM_MXFP4
    return _dt(w_gate_up)


def beam_moe_experts(cfg: LayerCfg, T, x, expert_offsets, row_token, w_gate_up, w_down, y,
                     x_scale=None, s_gate_up=None, s_down=None, ws=None, stream=None):
    """x: [T,H] f32/bf16 activations, e4m3 codes (uint8) for fp8 weights, or
    packed E2M1 codes [T,H/2] for MXFP4 weights."""
    w_dt = _experts_common(cfg, T, x, expert_offsets, row_token, w_gate_up, w_down, y, x_scale,
                           s_gate_up, s_down)
    st = lib().beam_moe_experts(ctypes.byref(cfg.c()), T, w_dt, _p(x), w_dt, _p(x_scale),
                                _p(expert_offsets), _p(row_token), _p(w_gate_up), _p(s_gate_up),
                                _p(w_down), _p(s_down), _p(y), _dt(y), _p(ws),
                                0 if ws is None else ws.numel(), _stream(stream))
    _ok("beam_moe_experts", st)


def _experts_common(cfg, T, x, expert_offsets, row_token, w_gate_up, w_down, y, x_scale, s_gate_up, s_down):
    E, H, F, TK = cfg.n_experts, cfg.hidden, cfg.d_ff, T * cfg.topk
    w_dt = _w_dtype(w_gate_up, s_gate_up)
    _check(expert_offsets, (E + 1,), (torch.int32,), "expert_offsets")
    _check(row_token, (TK,), (torch.int32,), "row_token")
    _check(y, (TK, H), (torch.float32, torch.bfloat16), "y")
    if w_dt == BEAM_MXFP4:
        _check(x, (T, H // 2), (torch.uint8,), "x")
        _check(w_gate_up, (E, 2 * F, H // 2), (torch.uint8,), "w_gate_up")
        _check(w_down, (E, H, F // 2), (torch.uint8,), "w_down")
        _check(x_scale, (T, H // 32), (torch.uint8,), "x_scale")
        _check(s_gate_up, (E, 2 * F, H // 32), (torch.uint8,), "s_gate_up")
        _check(s_down, (E, H, F // 32), (torch.uint8,), "s_down")
        return w_dt
    _check(x, (T, H), (w_gate_up.dtype,) if w_dt != BEAM_FP8_E4M3 else (torch.uint8, torch.float8_e4m3fn), "x")
    _check(w_gate_up, (E, 2 * F, H), (w_gate_up.dtype,), "w_gate_up")
    _check(w_down, (E, H, F), (w_gate_up.dtype,), "w_down")
    if w_dt == BEAM_FP8_E4M3:
        _check(x_scale, (T,), (torch.float32,), "x_scale")
        _check(s_gate_up, (E, 2 * F), (torch.float32,), "s_gate_up")
        _check(s_down, (E, H), (torch.float32,), "s_down")
    return w_dt


def beam_moe_experts_static(cfg: LayerCfg, T, x, expert_offsets, row_token, w_gate_up, w_down, y,
                            x_scale=None, s_gate_up=None, s_down=None, stream=None):
    """beam_moe_experts working in the library's per-GPU static scratch array
    (no workspace argument, nothing allocated).  Calls that overlap in time
    on one GPU race; calls ordered on one stream are safe."""
    w_dt = _experts_common(cfg, T, x, expert_offsets, row_token, w_gate_up, w_down, y, x_scale,
                           s_gate_up, s_down)
    st = lib().beam_moe_experts_static(ctypes.byref(cfg.c()), T, w_dt, _p(x), w_dt, _p(x_scale),
                                       _p(expert_offsets), _p(row_token), _p(w_gate_up), _p(s_gate_up),
                                       _p(w_down), _p(s_down), _p(y), _dt(y), _stream(stream))
    _ok("beam_moe_experts_static", st)


def beam_moe_combine_norm(cfg: LayerCfg, y, pair_row, topk_w, h, x_next, gamma_post, gamma_pre, n,
                          moe_out=None, stream=None):
    T = h.shape[0]
    H, TK = cfg.hidden, T * cfg.topk
    _check(y, (TK, H), (torch.float32, torch.bfloat16), "y")
    _check(pair_row, (TK,), (torch.int32,), "pair_row")
    _check(topk_w, (T, cfg.topk), (torch.float32,), "topk_w")
    _check(h, (T, H), (torch.float32, torch.bfloat16), "h")
    _check(x_next, (T, H), (h.dtype,), "x_next")
    _check(gamma_post, (H,), (h.dtype,), "gamma_post")
    _check(gamma_pre, (H,), (h.dtype,), "gamma_pre")
    if moe_out is not None:
        _check(moe_out, (T, H), (torch.float32,), "moe_out")
    st = lib().beam_moe_combine_norm(ctypes.byref(cfg.c()), T, _p(y), _dt(y), _p(pair_row),
                                     _p(topk_w), _p(h), _p(x_next), _dt(h), _p(gamma_post),
                                     _p(gamma_pre), int(n), _p(moe_out), _stream(stream))
    _ok("beam_moe_combine_norm", st)


def beam_moe_norm_boundary(cfg: LayerCfg, m, h, x_next, gamma_post, gamma_pre, n, stream=None):
    """Sandwich-norm boundary on a given m [T,H] (fp32/bf16): h updated in
    place, x_next written."""
    T, H = h.shape[0], cfg.hidden
    _check(m, (T, H), (torch.float32, torch.bfloat16), "m")
    _check(h, (T, H), (torch.float32, torch.bfloat16), "h")
    _check(x_next, (T, H), (h.dtype,), "x_next")
    _check(gamma_post, (H,), (h.dtype,), "gamma_post")
    _check(gamma_pre, (H,), (h.dtype,), "gamma_pre")
    st = lib().beam_moe_norm_boundary(ctypes.byref(cfg.c()), T, _p(m), _dt(m), _p(h), _p(x_next), _dt(h),
                                      _p(gamma_post), _p(gamma_pre), int(n), _stream(stream))
    _ok("beam_moe_norm_boundary", st)


def beam_moe_permute_shard(cfg: LayerCfg, topk_ids, expert_begin, n_local, expert_offsets, row_token, pair_row,
                           ws=None, stream=None):
    """Stable grouping of the pairs routed to experts [expert_begin,
    expert_begin + n_local); other pairs get pair_row -1."""
    T = topk_ids.shape[0]
    TK = T * cfg.topk
    _check(topk_ids, (T, cfg.topk), (torch.int32,), "topk_ids")
    _check(expert_offsets, (n_local + 1,), (torch.int32,), "expert_offsets")
    _check(row_token, (TK,), (torch.int32,), "row_token")
    _check(pair_row, (TK,), (torch.int32,), "pair_row")
    st = lib().beam_moe_permute_shard(ctypes.byref(cfg.c()), T, int(expert_begin), int(n_local), _p(topk_ids),
                                      _p(expert_offsets), _p(row_token), _p(pair_row), _p(ws),
                                      0 if ws is None else ws.numel(), _stream(stream))
    _ok("beam_moe_permute_shard", st)


def beam_moe_combine_partial(cfg: LayerCfg, y, pair_row, topk_w, m_out, stream=None):
    """One shard's share of the weighted combine (fp32, no norm)."""
    T = topk_w.shape[0]
    H, TK = cfg.hidden, T * cfg.topk
    _check(y, (TK, H), (torch.float32, torch.bfloat16), "y")
    _check(pair_row, (TK,), (torch.int32,), "pair_row")
    _check(topk_w, (T, cfg.topk), (torch.float32,), "topk_w")
    _check(m_out, (T, H), (torch.float32,), "m_out")
    st = lib().beam_moe_combine_partial(ctypes.byref(cfg.c()), T, _p(y), _dt(y), _p(pair_row), _p(topk_w),
                                        _p(m_out), _stream(stream))
    _ok("beam_moe_combine_partial", st)


def dense_workspace(cfg: LayerCfg, T: int, d_ff: int, device="cuda") -> torch.Tensor:
    n = int(lib().beam_moe_dense_workspace_bytes(ctypes.byref(cfg.c()), T, d_ff))
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def beam_moe_dense_mlp(cfg: LayerCfg, x, w_gate_up, w_down, y, ws, stream=None):
    """Dense SwiGLU MLP of width d_ff = w_gate_up.shape[0] // 2 over all rows
    of x [T,H] bf16; packed weights; y [T,H] fp32."""
    T, H = x.shape[0], cfg.hidden
    Fd = w_gate_up.shape[0] // 2
    _check(x, (T, H), (torch.bfloat16,), "x")
    _check(w_gate_up, (2 * Fd, H), (torch.bfloat16,), "w_gate_up")
    _check(w_down, (H, Fd), (torch.bfloat16,), "w_down")
    _check(y, (T, H), (torch.float32,), "y")
    st = lib().beam_moe_dense_mlp(ctypes.byref(cfg.c()), T, Fd, _p(x), BEAM_BF16, _p(w_gate_up), _p(w_down),
                                  _p(y), _p(ws), ws.numel(), _stream(stream))
    _ok("beam_moe_dense_mlp", st)


def beam_moe_pack_weights(cfg: LayerCfg, w_gate_up, w_down, packed_gate_up, packed_down, stream=None,
                          mxfp4=False):
    """Re-lays out [n,2F,H] / [n,H,F] expert stacks into the tiled layout that
    beam_moe_experts reads (any n >= 1 experts).  mxfp4: the stacks are
    packed E2M1 bytes [n,2F,H/2] / [n,H,F/2]."""
    n = w_gate_up.shape[0]
    H, F = cfg.hidden, cfg.d_ff
    dt = w_gate_up.dtype
    d = 2 if mxfp4 else 1
    _check(w_gate_up, (n, 2 * F, H // d), (dt,), "w_gate_up")
    _check(w_down, (n, H, F // d), (dt,), "w_down")
    _check(packed_gate_up, (n, 2 * F, H // d), (dt,), "packed_gate_up")
    _check(packed_down, (n, H, F // d), (dt,), "packed_down")
    st = lib().beam_moe_pack_weights(ctypes.byref(cfg.c()), n, BEAM_MXFP4 if mxfp4 else _dt(w_gate_up),
                                     _p(w_gate_up), _p(w_down), _p(packed_gate_up), _p(packed_down),
                                     _stream(stream))
    _ok("beam_moe_pack_weights", st)


def packed_expert_stacks(cfg: LayerCfg, make_expert, n_experts: int, device="cuda"):
    """Builds packed [E,2F,H] / [E,H,F] stacks one expert at a time from
    make_expert(e) -> (w_gate_up [2F,H], w_down [H,F], s_gate_up, s_down)
    device tensors (MXFP4: E2M1 bytes [2F,H/2] / [H,F/2] with uint8 E8M0
    scales).  Returns (packed_gate_up, packed_down, s_gate_up, s_down); the
    scales are not re-laid out."""
    a, b, c, d = make_expert(0)
    mx = c is not None and c.dtype == torch.uint8
    pgu = torch.empty((n_experts,) + tuple(a.shape), dtype=a.dtype, device=device)
    pd = torch.empty((n_experts,) + tuple(b.shape), dtype=b.dtype, device=device)
    sgu = sd = None
    if c is not None:
        sgu = torch.empty((n_experts,) + tuple(c.shape), dtype=c.dtype, device=device)
        sd = torch.empty((n_experts,) + tuple(d.shape), dtype=d.dtype, device=device)
    for e in range(n_experts):
        if e:
            a, b, c, d = make_expert(e)
        beam_moe_pack_weights(cfg, a.unsqueeze(0), b.unsqueeze(0), pgu[e:e + 1], pd[e:e + 1], mxfp4=mx)
        if sgu is not None:
            sgu[e].copy_(c)
            sd[e].copy_(d)
    return pgu, pd, sgu, sd


# ------------------------------------------------------------------ whole layer

@dataclasses.dataclass
class LayerBuffers:
    """Device outputs and scratch of one layer call for T tokens."""
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    logits: torch.Tensor | None
    expert_offsets: torch.Tensor
    row_token: torch.Tensor
    pair_row: torch.Tensor
    x_q: torch.Tensor | None
    x_scale: torch.Tensor | None
    y: torch.Tensor
    x_next: torch.Tensor
    moe_out: torch.Tensor | None
    ws: torch.Tensor


def alloc_buffers(cfg: LayerCfg, T: int, act_dtype, w_dtype: int, y_dtype=torch.float32,
                  keep_logits=False, keep_moe_out=False, device="cuda") -> LayerBuffers:
    TK = T * cfg.topk
    d = dict(device=device)
    fp8 = w_dtype == BEAM_FP8_E4M3
    mx = w_dtype == BEAM_MXFP4
    if mx:
        x_q = torch.empty((T, cfg.hidden // 2), dtype=torch.uint8, **d)
        x_scale = torch.empty((T, cfg.hidden // 32), dtype=torch.uint8, **d)
    else:
        x_q = torch.empty((T, cfg.hidden), dtype=torch.uint8, **d) if fp8 else None
        x_scale = torch.empty((T,), dtype=torch.float32, **d) if fp8 else None
    return LayerBuffers(
        topk_ids=torch.empty((T, cfg.topk), dtype=torch.int32, **d),
        topk_w=torch.empty((T, cfg.topk), dtype=torch.float32, **d),
        logits=torch.empty((T, cfg.n_experts), dtype=torch.float32, **d) if keep_logits else None,
        expert_offsets=torch.empty((cfg.n_experts + 1,), dtype=torch.int32, **d),
        row_token=torch.empty((TK,), dtype=torch.int32, **d),
        pair_row=torch.empty((TK,), dtype=torch.int32, **d),
        x_q=x_q,
        x_scale=x_scale,
        y=torch.empty((TK, cfg.hidden), dtype=y_dtype, **d),
        x_next=torch.empty((T, cfg.hidden), dtype=act_dtype, **d),
        moe_out=torch.empty((T, cfg.hidden), dtype=torch.float32, **d) if keep_moe_out else None,
        ws=workspace(cfg, T, w_dtype, device),
    )


def moe_layer(cfg: LayerCfg, x, w_router, bias, w_gate_up, w_down, h, gamma_post, gamma_pre, n,
              bufs: LayerBuffers, s_gate_up=None, s_down=None, stream=None, quant_stream=None):
    """Runs the entry points of one layer in order on one stream.
    w_gate_up/w_down are packed stacks (beam_moe_pack_weights).  h is
    updated in place; the other results land in `bufs`.

    With 8-bit or 4-bit experts and a `quant_stream` (a torch.cuda.Stream
    of the default priority), the input quantisation runs on that stream
    alongside the router and the permutation, and the experts call waits for
    it; `stream` is then None (the current stream) or a torch.cuda.Stream.
    On MI355X that pays off for large batches (fp8, 16384 tokens: about
    60 µs per layer); at decode sizes the fork and join cost more than the
    quantisation they hide, so leave quant_stream None there."""
    T = x.shape[0]
    w_dt = _w_dtype(w_gate_up, s_gate_up)
    fp8 = w_dt == BEAM_FP8_E4M3
    mx = w_dt == BEAM_MXFP4
    side = quant_stream if (fp8 or mx) else None
    main = None
    if side is not None:
        main = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.current_stream()
        side.wait_stream(main)
        if fp8:
            beam_moe_quantize_fp8(cfg, x, bufs.x_q, bufs.x_scale, side)
        else:
            beam_moe_quantize_mx(cfg, x, bufs.x_q, bufs.x_scale, side)
    beam_moe_route(cfg, x, w_router, bias, bufs.topk_ids, bufs.topk_w, bufs.logits, bufs.ws, stream)
    if mx and side is None:
        beam_moe_quantize_mx(cfg, x, bufs.x_q, bufs.x_scale, stream)
    q_in_permute = fp8 and side is None
    beam_moe_permute(cfg, bufs.topk_ids, bufs.expert_offsets, bufs.row_token, bufs.pair_row,
                     x=x if q_in_permute else None, x_q=bufs.x_q if q_in_permute else None,
                     x_scale=bufs.x_scale if q_in_permute else None, ws=bufs.ws, stream=stream)
    if side is not None:
        main.wait_stream(side)
    beam_moe_experts(cfg, T, bufs.x_q if (fp8 or mx) else x, bufs.expert_offsets, bufs.row_token,
                     w_gate_up, w_down, bufs.y, x_scale=bufs.x_scale, s_gate_up=s_gate_up,
                     s_down=s_down, ws=bufs.ws, stream=stream)
    beam_moe_combine_norm(cfg, bufs.y, bufs.pair_row, bufs.topk_w, h, bufs.x_next, gamma_post,
                          gamma_pre, n, bufs.moe_out, stream)
