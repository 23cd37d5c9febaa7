// C ABI entry points: argument validation, workspace carving and launches.
// Every check runs on the host before anything is enqueued.
#include "beam_moe.h"

#include <math.h>

#include <mutex>

#include "kernels.h"

// Workspace of beam_moe_experts_static: one copy of this array per GPU,
// loaded with the library's device code and held until the process ends.
// In host code the name is only a stand-in: kernels get the per-device
// address that hipGetSymbolAddress returns (static_scratch below).
static __device__ __align__(256) uint8_t scratch[BEAM_MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxT = 1 << 22;   // T*K stays far below 2^31
constexpr int kMaxDenseFF = 32768;  // widest dense MLP (the dense layers use 20480)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int epl_of(int E) { return beam::route_epl(E); }

beam_status check_cfg(const beam_moe_cfg* c) {
    if (!c) return BEAM_ERR_INVALID_ARG;
    if (c->hidden <= 0 || c->n_experts <= 0 || c->n_groups <= 0 || c->topk_groups <= 0 ||
        c->topk <= 0 || c->group_topn <= 0 || c->d_ff <= 0)
        return BEAM_ERR_INVALID_ARG;
    if (!(c->routed_scale > 0.f) || !isfinite(c->routed_scale) || !(c->rms_eps >= 0.f) ||
        !isfinite(c->rms_eps))
        return BEAM_ERR_INVALID_ARG;
    if (c->hidden % 256 != 0 || c->hidden > 8192) return BEAM_ERR_UNSUPPORTED;
    if (c->n_experts > beam::kMaxExperts || c->n_experts % c->n_groups != 0) return BEAM_ERR_UNSUPPORTED;
    const int per = c->n_experts / c->n_groups;
    const int epl = epl_of(c->n_experts);
    if (per % epl != 0) return BEAM_ERR_UNSUPPORTED;
    const int lpg = per / epl;
    if ((lpg & (lpg - 1)) != 0 || lpg * c->n_groups > 64) return BEAM_ERR_UNSUPPORTED;
    if (c->topk_groups > c->n_groups) return BEAM_ERR_INVALID_ARG;
    if (c->group_topn > per || c->group_topn > 4) return BEAM_ERR_UNSUPPORTED;
    if (c->topk > c->topk_groups * per) return BEAM_ERR_INVALID_ARG;
    if (c->topk > 32) return BEAM_ERR_UNSUPPORTED;
    if (c->d_ff % 128 != 0 || c->d_ff > 8192) return BEAM_ERR_UNSUPPORTED;
    return BEAM_OK;
}

bool valid_dtype(beam_dtype d) {
    return d == BEAM_F32 || d == BEAM_BF16 || d == BEAM_FP8_E4M3 || d == BEAM_MXFP4;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t route_ws(const beam_moe_cfg* c, int T) {
    return align256(beam::route_partials_bytes(T, c->hidden, c->n_experts));
}

beam::WKind wkind(beam_dtype d) {
    switch (d) {
        case BEAM_BF16: return beam::W_BF16;
        case BEAM_FP8_E4M3: return beam::W_FP8;
        case BEAM_MXFP4: return beam::W_MXFP4;
        default: return beam::W_F32;
    }
}

// 4-bit experts: rows of K values are K/2 bytes in whole 256-byte chunks
bool mx_shape_ok(const beam_moe_cfg* c) { return c->hidden % 512 == 0 && c->d_ff % 512 == 0; }

// Dense MLP: the rows form one "expert".  At decode sizes (direct kernel)
// both projections are split over K so that the chip holds enough waves to
// keep the weight stream going: the smallest slice count >= want / tiles
// that divides the 256-byte K iterations, for the down projection's H/128
// tiles and the gate/up projection's d_ff/64 tiles (measured on MI355X at
// d_ff 20480, T = 8: 16 and 4 slices, 137 -> 122 us per MLP call).
static int ksplit_for(int tiles, int nk, int want) {
    for (int s = (want + tiles - 1) / tiles; s <= nk; ++s)
        if (nk % s == 0) return s;
    return 1;
}
constexpr int kDenseWantWG2 = 512, kDenseWantWG1 = 1024;   // workgroups of 4 waves
int dense_ksplit(int T, int H, int Fd) {
    return T > 16 ? 1 : ksplit_for(H / 128, Fd * 2 / 256, kDenseWantWG2);
}
int dense_ksplit1(int T, int H, int Fd) {
    return T > 16 ? 1 : ksplit_for(Fd / 64, H * 2 / 256, kDenseWantWG1);
}

size_t dense_ws_bytes(int T, int H, int Fd) {
    const int S = dense_ksplit(T, H, Fd), S1 = dense_ksplit1(T, H, Fd);
    size_t b = 256 + align256((size_t)T * sizeof(int32_t));
    b += beam::experts_ws_bytes(T, 1, 1, H, Fd, beam::W_BF16);
    if (S > 1) b += align256((size_t)S * T * H * sizeof(float));
    if (S1 > 1) b += align256((size_t)S1 * T * 2 * Fd * sizeof(float));
    return b;
}

// Checks of beam_moe_experts that do not concern the workspace; fills `a`
// (all but a.ws) and the workspace bytes the call needs.
beam_status experts_prepare(const beam_moe_cfg* cfg, int32_t T, beam_dtype w_dtype, const void* x,
                            beam_dtype x_dtype, const void* x_scale, const int32_t* expert_offsets,
                            const int32_t* row_token, const void* w_gate_up, const void* s_gate_up,
                            const void* w_down, const void* s_down, void* y, beam_dtype y_dtype,
                            beam::ExpertsArgs& a, size_t& need) {
    beam_status st = check_cfg(cfg);
    if (st != BEAM_OK) return st;
    if (T < 0 || T > kMaxT) return BEAM_ERR_INVALID_ARG;
    if (!valid_dtype(w_dtype) || !valid_dtype(x_dtype) || !valid_dtype(y_dtype))
        return BEAM_ERR_INVALID_ARG;
    if (x_dtype != w_dtype) return BEAM_ERR_INVALID_ARG;
    if (y_dtype == BEAM_FP8_E4M3 || y_dtype == BEAM_MXFP4) return BEAM_ERR_INVALID_ARG;
    if (w_dtype == BEAM_FP8_E4M3 && (cfg->hidden % 256 != 0 || cfg->d_ff % 256 != 0))
        return BEAM_ERR_UNSUPPORTED;
    if (w_dtype == BEAM_MXFP4 && !mx_shape_ok(cfg)) return BEAM_ERR_UNSUPPORTED;
    if (T == 0) return BEAM_OK;
    if (!x || !expert_offsets || !row_token || !w_gate_up || !w_down || !y) return BEAM_ERR_INVALID_ARG;
    if ((w_dtype == BEAM_FP8_E4M3 || w_dtype == BEAM_MXFP4) && (!x_scale || !s_gate_up || !s_down))
        return BEAM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y))
        return BEAM_ERR_INVALID_ARG;
    if (w_dtype == BEAM_FP8_E4M3 && (!aligned16(s_gate_up) || !aligned16(s_down)))
        return BEAM_ERR_INVALID_ARG;
    const beam::WKind wk = wkind(w_dtype);
    need = beam::experts_ws_bytes(T, cfg->topk, cfg->n_experts, cfg->hidden, cfg->d_ff, wk);
    a.T = T;
    a.K = cfg->topk;
    a.E = cfg->n_experts;
    a.H = cfg->hidden;
    a.F = cfg->d_ff;
    a.w = wk;
    a.x = x;
    a.xscale = x_scale;
    a.offsets = expert_offsets;
    a.row_token = row_token;
    a.wgu = w_gate_up;
    a.sgu = s_gate_up;
    a.wd = w_down;
    a.sd = s_down;
    a.y = y;
    a.y_bf16 = y_dtype == BEAM_BF16;
    return BEAM_OK;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` belongs to, looked up
// once per device with that device current.
hipError_t static_scratch(hipStream_t stream, void** out) {
    int cur = 0;
    hipError_t err = hipGetDevice(&cur);
    if (err != hipSuccess) return err;
    int dev = cur;
    if (stream) {
        hipDevice_t d = 0;
        err = hipStreamGetDevice(stream, &d);
        if (err != hipSuccess) return err;
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (err = hipSetDevice(dev)) != hipSuccess) return err;
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (err == hipSuccess) err = e2;
        }
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* beam_moe_status_string(beam_status s) {
    switch (s) {
        case BEAM_OK: return "ok";
        case BEAM_ERR_INVALID_ARG: return "invalid argument";
        case BEAM_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case BEAM_ERR_WORKSPACE: return "workspace missing or too small";
        case BEAM_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

size_t beam_moe_workspace_bytes(const beam_moe_cfg* cfg, int32_t T, beam_dtype w_dtype) {
    if (check_cfg(cfg) != BEAM_OK || T < 0 || T > kMaxT || !valid_dtype(w_dtype)) return 0;
    if (T == 0) return 256;
    size_t b = route_ws(cfg, T);
    const size_t pb = beam::permute_ws_bytes(T, cfg->topk, cfg->n_experts);
    const size_t eb = beam::experts_ws_bytes(T, cfg->topk, cfg->n_experts, cfg->hidden, cfg->d_ff,
                                             wkind(w_dtype));
    if (pb > b) b = pb;
    if (eb > b) b = eb;
    return b;
}

beam_status beam_moe_route(const beam_moe_cfg* cfg, int32_t T, const void* x, beam_dtype x_dtype,
                           const float* w_router, const float* bias, int32_t* topk_ids,
                           float* topk_w, float* logits_out, void* ws, size_t ws_bytes,
                           void* stream) {
    beam_status st = check_cfg(cfg);
    if (st != BEAM_OK) return st;
    if (T < 0 || T > kMaxT) return BEAM_ERR_INVALID_ARG;
    if (x_dtype != BEAM_BF16 && x_dtype != BEAM_F32) return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!x || !w_router || !bias || !topk_ids || !topk_w) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router) || (logits_out && !aligned16(logits_out)))
        return BEAM_ERR_INVALID_ARG;
    if (!ws || ws_bytes < route_ws(cfg, T) || !aligned16(ws)) return BEAM_ERR_WORKSPACE;
    beam::RouteArgs a{};
    a.T = T;
    a.H = cfg->hidden;
    a.E = cfg->n_experts;
    a.G = cfg->n_groups;
    a.kg = cfg->topk_groups;
    a.K = cfg->topk;
    a.topn = cfg->group_topn;
    a.scale = cfg->routed_scale;
    a.x = x;
    a.x_bf16 = x_dtype == BEAM_BF16;
    a.w = w_router;
    a.bias = bias;
    a.logits_out = logits_out;
    a.partials = static_cast<float*>(ws);
    a.ids = topk_ids;
    a.wts = topk_w;
    return beam::launch_route(a, static_cast<hipStream_t>(stream)) == hipSuccess ? BEAM_OK
                                                                                  : BEAM_ERR_HIP;
}

beam_status beam_moe_permute(const beam_moe_cfg* cfg, int32_t T, const int32_t* topk_ids,
                             int32_t* expert_offsets, int32_t* row_token, int32_t* pair_row,
                             const void* x, beam_dtype x_dtype, uint8_t* x_q, float* x_scale,
                             void* ws, size_t ws_bytes, void* stream) {
    beam_status st = check_cfg(cfg);
    if (st != BEAM_OK) return st;
    if (T < 0 || T > kMaxT) return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!topk_ids || !expert_offsets || !row_token || !pair_row) return BEAM_ERR_INVALID_ARG;
    if (x_q) {
        if (!x || !x_scale || x_dtype != BEAM_BF16) return BEAM_ERR_INVALID_ARG;
        if (!aligned16(x) || !aligned16(x_q)) return BEAM_ERR_INVALID_ARG;
    }
    const size_t need = beam::permute_ws_bytes(T, cfg->topk, cfg->n_experts);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return BEAM_ERR_WORKSPACE;
    beam::PermuteArgs a{};
    a.T = T;
    a.K = cfg->topk;
    a.E = cfg->n_experts;
    a.H = cfg->hidden;
    a.ids = topk_ids;
    a.offsets = expert_offsets;
    a.row_token = row_token;
    a.pair_row = pair_row;
    a.x = static_cast<const uint16_t*>(x);
    a.xq = x_q;
    a.xscale = x_scale;
    a.ws = ws;
    return beam::launch_permute(a, static_cast<hipStream_t>(stream)) == hipSuccess ? BEAM_OK
                                                                                    : BEAM_ERR_HIP;
}

beam_status beam_moe_experts(const beam_moe_cfg* cfg, int32_t T, beam_dtype w_dtype, const void* x,
                             beam_dtype x_dtype, const void* x_scale, const int32_t* expert_offsets,
                             const int32_t* row_token, const void* w_gate_up, const void* s_gate_up,
                             const void* w_down, const void* s_down, void* y, beam_dtype y_dtype,
                             void* ws, size_t ws_bytes, void* stream) {
    beam::ExpertsArgs a{};
    size_t need = 0;
    const beam_status st = experts_prepare(cfg, T, w_dtype, x, x_dtype, x_scale, expert_offsets, row_token,
                                           w_gate_up, s_gate_up, w_down, s_down, y, y_dtype, a, need);
    if (st != BEAM_OK || T == 0) return st;
    if (!ws || ws_bytes < need || !aligned16(ws)) return BEAM_ERR_WORKSPACE;
    a.ws = ws;
    return beam::launch_experts(a, static_cast<hipStream_t>(stream)) == hipSuccess ? BEAM_OK
                                                                                    : BEAM_ERR_HIP;
}

beam_status beam_moe_experts_static(const beam_moe_cfg* cfg, int32_t T, beam_dtype w_dtype,
                                    const void* x, beam_dtype x_dtype, const void* x_scale,
                                    const int32_t* expert_offsets, const int32_t* row_token,
                                    const void* w_gate_up, const void* s_gate_up, const void* w_down,
                                    const void* s_down, void* y, beam_dtype y_dtype, void* stream) {
    beam::ExpertsArgs a{};
    size_t need = 0;
    const beam_status st = experts_prepare(cfg, T, w_dtype, x, x_dtype, x_scale, expert_offsets, row_token,
                                           w_gate_up, s_gate_up, w_down, s_down, y, y_dtype, a, need);
    if (st != BEAM_OK || T == 0) return st;
    if (need > BEAM_MOE_STATIC_SCRATCH_BYTES) return BEAM_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* scr = nullptr;
    if (static_scratch(s, &scr) != hipSuccess) return BEAM_ERR_HIP;
    a.ws = scr;
    return beam::launch_experts(a, s) == hipSuccess ? BEAM_OK : BEAM_ERR_HIP;
}

beam_status beam_moe_pack_weights(const beam_moe_cfg* cfg, int32_t n_experts, beam_dtype w_dtype,
                                  const void* w_gate_up, const void* w_down, void* packed_gate_up,
                                  void* packed_down, void* stream) {
    // packing only depends on the matrix shapes (hidden, d_ff)
    if (!cfg || cfg->hidden <= 0 || cfg->d_ff <= 0) return BEAM_ERR_INVALID_ARG;
    if (cfg->hidden % 256 != 0 || cfg->hidden > 8192 || cfg->d_ff % 128 != 0 || cfg->d_ff > kMaxDenseFF)
        return BEAM_ERR_UNSUPPORTED;
    if (n_experts < 0 || !valid_dtype(w_dtype)) return BEAM_ERR_INVALID_ARG;
    if (w_dtype == BEAM_FP8_E4M3 && (cfg->hidden % 256 != 0 || cfg->d_ff % 256 != 0))
        return BEAM_ERR_UNSUPPORTED;
    if (w_dtype == BEAM_MXFP4 && !mx_shape_ok(cfg)) return BEAM_ERR_UNSUPPORTED;
    if (n_experts == 0) return BEAM_OK;
    if (!w_gate_up || !w_down || !packed_gate_up || !packed_down) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(packed_gate_up) || !aligned16(packed_down))
        return BEAM_ERR_INVALID_ARG;
    // bytes per 2 elements
    const size_t es2 = w_dtype == BEAM_F32 ? 8 : (w_dtype == BEAM_BF16 ? 4 : (w_dtype == BEAM_FP8_E4M3 ? 2 : 1));
    const size_t H = cfg->hidden, F = cfg->d_ff, E = (size_t)n_experts;
    const size_t gu_bytes = E * 2 * F * H * es2 / 2, d_bytes = E * H * F * es2 / 2;
    auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
        const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
        return x < y + nb && y < x + na;
    };
    if (overlap(w_gate_up, gu_bytes, packed_gate_up, gu_bytes) || overlap(w_down, d_bytes, packed_down, d_bytes) ||
        overlap(packed_gate_up, gu_bytes, packed_down, d_bytes))
        return BEAM_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    if (w_dtype == BEAM_F32) {   // the fp32 path reads plain row-major weights
        err = hipMemcpyAsync(packed_gate_up, w_gate_up, gu_bytes, hipMemcpyDeviceToDevice, s);
        if (err == hipSuccess)
            err = hipMemcpyAsync(packed_down, w_down, d_bytes, hipMemcpyDeviceToDevice, s);
    } else {
        err = beam::launch_pack(w_gate_up, packed_gate_up, E * 2 * F, (int)(H * es2 / 2), s);
        if (err == hipSuccess) err = beam::launch_pack(w_down, packed_down, E * H, (int)(F * es2 / 2), s);
    }
    return err == hipSuccess ? BEAM_OK : BEAM_ERR_HIP;
}

beam_status beam_moe_quantize_fp8(const beam_moe_cfg* cfg, int32_t T, const void* x, beam_dtype x_dtype,
                                  uint8_t* x_q, float* x_scale, void* stream) {
    beam_status st = check_cfg(cfg);
    if (st != BEAM_OK) return st;
    if (T < 0 || T > kMaxT) return BEAM_ERR_INVALID_ARG;
    if (x_dtype != BEAM_BF16) return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!x || !x_q || !x_scale) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(x_q)) return BEAM_ERR_INVALID_ARG;
    return beam::launch_quantize_x_e4m3(static_cast<const uint16_t*>(x), T, cfg->hidden, x_q, x_scale,
                                        static_cast<hipStream_t>(stream)) == hipSuccess
               ? BEAM_OK
               : BEAM_ERR_HIP;
}

beam_status beam_moe_quantize_mx(const beam_moe_cfg* cfg, int32_t T, const void* x, beam_dtype x_dtype,
                                 uint8_t* x_q, uint8_t* x_scale, void* stream) {
    beam_status st = check_cfg(cfg);
    if (st != BEAM_OK) return st;
    if (T < 0 || T > kMaxT) return BEAM_ERR_INVALID_ARG;
    if (x_dtype != BEAM_BF16 && x_dtype != BEAM_F32) return BEAM_ERR_INVALID_ARG;
    if (cfg->hidden % 512 != 0) return BEAM_ERR_UNSUPPORTED;
    if (T == 0) return BEAM_OK;
    if (!x || !x_q || !x_scale) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(x_q) & 3u) != 0) return BEAM_ERR_INVALID_ARG;
    return beam::launch_quantize_mx(x, x_dtype == BEAM_BF16, T, cfg->hidden, nullptr, x_q, x_scale,
                                    static_cast<hipStream_t>(stream)) == hipSuccess
               ? BEAM_OK
               : BEAM_ERR_HIP;
}

beam_status beam_moe_combine_norm(const beam_moe_cfg* cfg, int32_t T, const void* y,
                                  beam_dtype y_dtype, const int32_t* pair_row, const float* topk_w,
                                  void* h, void* x_next, beam_dtype act_dtype, const void* gamma_post,
                                  const void* gamma_pre, int32_t n, float* moe_out, void* stream) {
    beam_status st = check_cfg(cfg);
    if (st != BEAM_OK) return st;
    if (T < 0 || T > kMaxT || n < 1) return BEAM_ERR_INVALID_ARG;
    if ((y_dtype != BEAM_F32 && y_dtype != BEAM_BF16) || (act_dtype != BEAM_F32 && act_dtype != BEAM_BF16))
        return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!y || !pair_row || !topk_w || !h || !x_next || !gamma_post || !gamma_pre)
        return BEAM_ERR_INVALID_ARG;
    if (h == x_next) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(y) || !aligned16(h) || !aligned16(x_next) || !aligned16(gamma_post) ||
        !aligned16(gamma_pre) || (moe_out && !aligned16(moe_out)))
        return BEAM_ERR_INVALID_ARG;
    beam::CombineArgs a{};
    a.T = T;
    a.K = cfg->topk;
    a.H = cfg->hidden;
    a.y = y;
    a.y_bf16 = y_dtype == BEAM_BF16;
    a.pair_row = pair_row;
    a.w = topk_w;
    a.h = h;
    a.x_next = x_next;
    a.act_bf16 = act_dtype == BEAM_BF16;
    a.gpost = gamma_post;
    a.gpre = gamma_pre;
    a.c_res = (float)sqrt((double)(n - 1) / (double)n);
    a.c_new = (float)(1.0 / sqrt((double)n));
    a.eps = cfg->rms_eps;
    a.moe_out = moe_out;
    return beam::launch_combine_norm(a, static_cast<hipStream_t>(stream)) == hipSuccess ? BEAM_OK
                                                                                         : BEAM_ERR_HIP;
}

size_t beam_moe_dense_workspace_bytes(const beam_moe_cfg* cfg, int32_t T, int32_t d_ff) {
    if (!cfg || cfg->hidden <= 0 || cfg->hidden % 256 != 0 || cfg->hidden > 8192) return 0;
    if (T < 0 || T > kMaxT || d_ff <= 0 || d_ff % 128 != 0 || d_ff > kMaxDenseFF) return 0;
    if (T == 0) return 256;
    return dense_ws_bytes(T, cfg->hidden, d_ff);
}

beam_status beam_moe_dense_mlp(const beam_moe_cfg* cfg, int32_t T, int32_t d_ff, const void* x,
                               beam_dtype x_dtype, const void* w_gate_up, const void* w_down, float* y,
                               void* ws, size_t ws_bytes, void* stream) {
    if (!cfg || cfg->hidden <= 0 || d_ff <= 0 || T < 0 || T > kMaxT) return BEAM_ERR_INVALID_ARG;
    if (cfg->hidden % 256 != 0 || cfg->hidden > 8192 || d_ff % 128 != 0 || d_ff > kMaxDenseFF)
        return BEAM_ERR_UNSUPPORTED;
    if (x_dtype != BEAM_BF16) return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!x || !w_gate_up || !w_down || !y) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(y))
        return BEAM_ERR_INVALID_ARG;
    const int H = cfg->hidden;
    if (!ws || ws_bytes < dense_ws_bytes(T, H, d_ff) || !aligned16(ws)) return BEAM_ERR_WORKSPACE;
    const int S = dense_ksplit(T, H, d_ff), S1 = dense_ksplit1(T, H, d_ff);
    uint8_t* base = static_cast<uint8_t*>(ws);
    int32_t* offsets = reinterpret_cast<int32_t*>(base);
    int32_t* row_token = reinterpret_cast<int32_t*>(base + 256);
    uint8_t* ews = base + 256 + align256((size_t)T * sizeof(int32_t));
    uint8_t* after = ews + beam::experts_ws_bytes(T, 1, 1, H, d_ff, beam::W_BF16);
    float* parts = S > 1 ? reinterpret_cast<float*>(after) : y;
    if (S > 1) after += align256((size_t)S * T * H * sizeof(float));
    float* g1_parts = S1 > 1 ? reinterpret_cast<float*>(after) : nullptr;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the identity routing (one expert holding tokens 0..T-1 in order); the
    // direct kernels of small batches take it without reading it
    const bool identity = beam::experts_direct_path(T);
    if (!identity && beam::launch_dense_rows(T, offsets, row_token, st) != hipSuccess) return BEAM_ERR_HIP;
    beam::ExpertsArgs a{};
    a.identity_rows = identity;
    a.T = T;
    a.K = 1;
    a.E = 1;
    a.H = H;
    a.F = d_ff;
    a.w = beam::W_BF16;
    a.x = x;
    a.offsets = offsets;
    a.row_token = row_token;
    a.wgu = w_gate_up;
    a.wd = w_down;
    a.y = parts;
    a.y_bf16 = false;
    a.ws = ews;
    a.ksplit = S;
    a.y_slice_stride = (size_t)T * H;
    a.ksplit1 = S1;
    a.g1_parts = g1_parts;
    if (beam::launch_experts(a, st) != hipSuccess) return BEAM_ERR_HIP;
    if (S > 1 && beam::launch_sum_slices(parts, S, (size_t)T * H, y, st) != hipSuccess) return BEAM_ERR_HIP;
    return BEAM_OK;
}

beam_status beam_moe_permute_shard(const beam_moe_cfg* cfg, int32_t T, int32_t expert_begin, int32_t n_local,
                                   const int32_t* topk_ids, int32_t* expert_offsets, int32_t* row_token,
                                   int32_t* pair_row, void* ws, size_t ws_bytes, void* stream) {
    beam_status st = check_cfg(cfg);
    if (st != BEAM_OK) return st;
    if (T < 0 || T > kMaxT) return BEAM_ERR_INVALID_ARG;
    if (n_local <= 0 || expert_begin < 0 || expert_begin + n_local > cfg->n_experts) return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!topk_ids || !expert_offsets || !row_token || !pair_row) return BEAM_ERR_INVALID_ARG;
    const size_t need = beam::permute_ws_bytes(T, cfg->topk, n_local);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return BEAM_ERR_WORKSPACE;
    beam::PermuteArgs a{};
    a.T = T;
    a.K = cfg->topk;
    a.E = n_local;
    a.e_base = expert_begin;
    a.H = cfg->hidden;
    a.ids = topk_ids;
    a.offsets = expert_offsets;
    a.row_token = row_token;
    a.pair_row = pair_row;
    a.ws = ws;
    return beam::launch_permute(a, static_cast<hipStream_t>(stream)) == hipSuccess ? BEAM_OK : BEAM_ERR_HIP;
}

beam_status beam_moe_combine_partial(const beam_moe_cfg* cfg, int32_t T, const void* y, beam_dtype y_dtype,
                                     const int32_t* pair_row, const float* topk_w, float* m_out, void* stream) {
    beam_status st = check_cfg(cfg);
    if (st != BEAM_OK) return st;
    if (T < 0 || T > kMaxT) return BEAM_ERR_INVALID_ARG;
    if (y_dtype != BEAM_F32 && y_dtype != BEAM_BF16) return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!y || !pair_row || !topk_w || !m_out) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(y) || !aligned16(m_out)) return BEAM_ERR_INVALID_ARG;
    beam::CombineArgs a{};
    a.T = T;
    a.K = cfg->topk;
    a.H = cfg->hidden;
    a.y = y;
    a.y_bf16 = y_dtype == BEAM_BF16;
    a.pair_row = pair_row;
    a.w = topk_w;
    a.moe_out = m_out;
    a.partial_only = true;
    return beam::launch_combine_norm(a, static_cast<hipStream_t>(stream)) == hipSuccess ? BEAM_OK
                                                                                         : BEAM_ERR_HIP;
}

beam_status beam_moe_norm_boundary(const beam_moe_cfg* cfg, int32_t T, const void* m, beam_dtype m_dtype,
                                   void* h, void* x_next, beam_dtype act_dtype, const void* gamma_post,
                                   const void* gamma_pre, int32_t n, void* stream) {
    if (!cfg || cfg->hidden <= 0 || cfg->hidden % 256 != 0 || cfg->hidden > 8192) return BEAM_ERR_INVALID_ARG;
    if (!(cfg->rms_eps >= 0.f) || !isfinite(cfg->rms_eps)) return BEAM_ERR_INVALID_ARG;
    if (T < 0 || T > kMaxT || n < 1) return BEAM_ERR_INVALID_ARG;
    if ((m_dtype != BEAM_F32 && m_dtype != BEAM_BF16) || (act_dtype != BEAM_F32 && act_dtype != BEAM_BF16))
        return BEAM_ERR_INVALID_ARG;
    if (T == 0) return BEAM_OK;
    if (!m || !h || !x_next || !gamma_post || !gamma_pre || h == x_next) return BEAM_ERR_INVALID_ARG;
    if (!aligned16(m) || !aligned16(h) || !aligned16(x_next) || !aligned16(gamma_post) || !aligned16(gamma_pre))
        return BEAM_ERR_INVALID_ARG;
    beam::CombineArgs a{};
    a.T = T;
    a.K = 1;
    a.H = cfg->hidden;
    a.y = m;
    a.y_bf16 = m_dtype == BEAM_BF16;
    a.pair_row = nullptr;   // row t of m, weight 1
    a.w = nullptr;
    a.h = h;
    a.x_next = x_next;
    a.act_bf16 = act_dtype == BEAM_BF16;
    a.gpost = gamma_post;
    a.gpre = gamma_pre;
    a.c_res = (float)sqrt((double)(n - 1) / (double)n);
    a.c_new = (float)(1.0 / sqrt((double)n));
    a.eps = cfg->rms_eps;
    a.moe_out = nullptr;
    return beam::launch_combine_norm(a, static_cast<hipStream_t>(stream)) == hipSuccess ? BEAM_OK
                                                                                         : BEAM_ERR_HIP;
}

}  // extern "C"
