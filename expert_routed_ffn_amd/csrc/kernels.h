// Internal launch interface between the C ABI (beam_moe.hip) and the kernel
// files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace beam {

struct RouteArgs {
    int T, H, E, G, kg, K, topn;
    float scale;
    const void* x;
    bool x_bf16;
    const float* w;
    const float* bias;
    float* logits_out;  // [T,E] or null
    float* partials;    // workspace, route_partials_bytes(T, H, E)
    int32_t* ids;
    float* wts;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
int route_epl(int E);
size_t route_partials_bytes(int T, int H, int E);

struct PermuteArgs {
    int T, K, E, H;
    int e_base;             // ids are taken relative to it; ids outside [e_base, e_base + E) are dropped
    const int32_t* ids;
    int32_t* offsets;
    int32_t* row_token;
    int32_t* pair_row;
    const uint16_t* x;  // bf16, only with xq
    uint8_t* xq;
    float* xscale;
    void* ws;
};
size_t permute_ws_bytes(int T, int K, int E);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t st);
// dynamic per-token e4m3 quantisation of bf16 rows x [T,H]
hipError_t launch_quantize_x_e4m3(const uint16_t* x, int T, int H, uint8_t* xq, float* xscale, hipStream_t st);

enum WKind { W_F32 = 0, W_BF16 = 1, W_FP8 = 2, W_MXFP4 = 3 };

// most experts per layer (the item builder gives each expert one thread)
constexpr int kMaxExperts = 256;

struct ExpertsArgs {
    int T, K, E, H, F;
    WKind w;
    const void* x;          // F32 / BF16 activations, e4m3 codes or packed E2M1 codes
    const void* xscale;     // FP8: fp32 per token; MXFP4: E8M0 per 32-block
    const int32_t* offsets;
    const int32_t* row_token;
    const void* wgu;
    const void* sgu;        // FP8: fp32 per row; MXFP4: E8M0 per 32-block
    const void* wd;
    const void* sd;
    void* y;
    bool y_bf16;
    void* ws;
    // split of the down projection's K over gridDim.y slices (direct kernel
    // only); slice s writes its partial sums to y + s * y_slice_stride
    int ksplit = 1;
    size_t y_slice_stride = 0;
    // split of the gate/up projection's K (bf16, direct kernel only): slice s
    // writes the raw gate and up sums of row r to g1_parts[s][r][0:2F]
    // (fp32), and a fixed-order sum over the slices applies SwiGLU
    int ksplit1 = 1;
    float* g1_parts = nullptr;
    // one expert whose rows are the T tokens in order (a dense MLP): on the
    // direct path (T <= 16) offsets and row_token are then not read
    bool identity_rows = false;
};
// whether launch_experts takes the direct path (T <= 16 tokens)
bool experts_direct_path(int T);
size_t experts_ws_bytes(int T, int K, int E, int H, int F, WKind w);
hipError_t launch_experts(const ExpertsArgs& a, hipStream_t st);

// y[i] = sum over s of parts[s * n + i], s = 0..S-1 in order
hipError_t launch_sum_slices(const float* parts, int S, size_t n, float* y, hipStream_t st);
// offsets = {0, T}, row_token = 0..T-1 (the dense MLP as one expert over all rows)
hipError_t launch_dense_rows(int T, int32_t* offsets, int32_t* row_token, hipStream_t st);

// Reorders `rows` rows of `kb` bytes (rows % 16 == 0, kb % 256 == 0) into
// the packed tile layout of the expert GEMM.
hipError_t launch_pack(const void* src, void* dst, size_t rows, int kb, hipStream_t st);

// MXFP4 quantisation of `rows` rows of K values (bf16 or fp32), K % 512 == 0:
// packed E2M1 codes [rows, K/2] and E8M0 codes [rows, K/32].  With
// `row_count` non-null only rows below *row_count are done.
hipError_t launch_quantize_mx(const void* x, bool bf16, int rows, int K, const int32_t* row_count,
                              uint8_t* q, uint8_t* s, hipStream_t st);

struct CombineArgs {
    int T, K, H;
    const void* y;
    bool y_bf16;
    const int32_t* pair_row;
    const float* w;
    void* h;
    void* x_next;
    bool act_bf16;
    const void* gpost;
    const void* gpre;
    float c_res, c_new, eps;
    float* moe_out;
    bool partial_only;      // write m to moe_out and stop (no norm boundary)
};
hipError_t launch_combine_norm(const CombineArgs& a, hipStream_t st);

}  // namespace beam
