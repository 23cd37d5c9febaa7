// Weighted combine of the K expert outputs fused with the sandwich-norm
// boundary: post-RMSNorm, depth-scaled residual, next pre-RMSNorm.
// (TokenSpeed x Reflection Beam blog, "MNNVL all-reduce and SandwichNorm
//  fusion"; vLLM Beam summary, kernel changes 1 and 3 and the MoE and
//  residual section: h <- sqrt((n-1)/n) h + x/sqrt(n), fp32 math with the
//  bf16 rounding points of the reference.)
//
// One 256-thread workgroup per token; thread i owns elements i, i+256, ...
// of the hidden row, so every global access is a coalesced row segment.
#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int kMaxIt = 32;   // H <= 32 * 256
constexpr int kMaxK = 32;

template <bool BF> BEAM_DEV float ld_act(const void* p, size_t i) {
    if constexpr (BF) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
    else return static_cast<const float*>(p)[i];
}
template <bool BF> BEAM_DEV float rnd_act(float v) {
    if constexpr (BF) return bf16_to_f32(f32_to_bf16(v));
    else return v;
}
template <bool BF> BEAM_DEV void st_act(void* p, size_t i, float v) {
    if constexpr (BF) static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    else static_cast<float*>(p)[i] = v;
}

template <bool YBF, bool ABF>
__global__ __launch_bounds__(256) void beam_combine_norm(CombineArgs a) {
    __shared__ int rows_s[kMaxK];
    __shared__ float w_s[kMaxK];
    __shared__ float red[4];
    const int t = blockIdx.x, tid = threadIdx.x;
    const int H = a.H, K = a.K;
    const int TK = a.T * K;
    if (tid < K) {
        rows_s[tid] = a.pair_row[(size_t)t * K + tid];
        w_s[tid] = a.w[(size_t)t * K + tid];
    }
    __syncthreads();

    float m[kMaxIt];
#pragma unroll
    for (int it = 0; it < kMaxIt; ++it) m[it] = 0.f;
    for (int k = 0; k < K; ++k) {
        const int r = rows_s[k];
        if ((unsigned)r >= (unsigned)TK) continue;   // never read outside y
        const float wk = w_s[k];
        const size_t base = (size_t)r * H;
#pragma unroll
        for (int it = 0; it < kMaxIt; ++it) {
            const int i = it * 256 + tid;
            if (i < H) m[it] = fmaf(wk, ld_act<YBF>(a.y, base + i), m[it]);
        }
    }

    // post-norm
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < kMaxIt; ++it)
        if (it * 256 + tid < H) ss = fmaf(m[it], m[it], ss);
    ss = block_sum<4>(ss, red);
    const float rinv = 1.0f / sqrtf(ss / (float)H + a.eps);

    // residual update (h' overwrites m)
    const size_t rowo = (size_t)t * H;
    float ss2 = 0.f;
#pragma unroll
    for (int it = 0; it < kMaxIt; ++it) {
        const int i = it * 256 + tid;
        if (i < H) {
            if (a.moe_out) a.moe_out[rowo + i] = m[it];
            const float p = rnd_act<ABF>(m[it] * rinv * ld_act<ABF>(a.gpost, i));
            const float hn = rnd_act<ABF>(a.c_res * ld_act<ABF>(a.h, rowo + i) + a.c_new * p);
            m[it] = hn;
            ss2 = fmaf(hn, hn, ss2);
        }
    }
    ss2 = block_sum<4>(ss2, red);
    const float rinv2 = 1.0f / sqrtf(ss2 / (float)H + a.eps);
#pragma unroll
    for (int it = 0; it < kMaxIt; ++it) {
        const int i = it * 256 + tid;
        if (i < H) {
            st_act<ABF>(a.h, rowo + i, m[it]);
            st_act<ABF>(a.x_next, rowo + i, m[it] * rinv2 * ld_act<ABF>(a.gpre, i));
        }
    }
}

hipError_t launch_combine_norm(const CombineArgs& a, hipStream_t st) {
    dim3 grid(a.T), block(256);
    if (a.y_bf16) {
        if (a.act_bf16) hipLaunchKernelGGL((beam_combine_norm<true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((beam_combine_norm<true, false>), grid, block, 0, st, a);
    } else {
        if (a.act_bf16) hipLaunchKernelGGL((beam_combine_norm<false, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((beam_combine_norm<false, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace beam
