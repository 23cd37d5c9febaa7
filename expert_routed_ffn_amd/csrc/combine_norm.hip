// Weighted combine of the K expert outputs fused with the sandwich-norm
// boundary: post-RMSNorm, depth-scaled residual, next pre-RMSNorm.
// (TokenSpeed x Reflection Beam blog, "MNNVL all-reduce and SandwichNorm
//  fusion"; vLLM Beam summary, kernel changes 1 and 3 and the MoE and
//  residual section: h <- sqrt((n-1)/n) h + x/sqrt(n), fp32 math with the
//  bf16 rounding points of the reference.)
//
// One 256-thread workgroup per token; thread i owns the 4-element chunks
// i, i+256, ... of the hidden row, so every global access is a coalesced
// row segment, and the K expert rows of a token are read with all their
// loads in flight together.
#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int kMaxIt = 8;    // chunks of 4 per thread: H <= 8 * 1024
constexpr int kSmallT = 256; // up to this many tokens the grid is too small to hide latency

// 4 consecutive elements as loaded (two bf16 pairs or four fp32), then
// widened to fp32 in a separate step: a widening next to its load would make
// the load's wait come right after it, so keeping the raw bits lets a
// thread have all its loads in flight before the first one is used.  NT: a
// streaming (non-temporal) load, for data this kernel reads once (the
// expert rows y, the token's h), which should not push the reused gammas
// out of the caches.
template <bool BF> struct Raw4;
template <> struct Raw4<true> { uint2 v; };
template <> struct Raw4<false> { float4 v; };
template <bool BF, bool NT = false> BEAM_DEV Raw4<BF> ldr4(const void* p, size_t i) {
    Raw4<BF> r;
    if constexpr (BF) {
        typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
        const u32x2v* q = reinterpret_cast<const u32x2v*>(static_cast<const uint16_t*>(p) + i);
        const u32x2v u = NT ? __builtin_nontemporal_load(q) : *q;
        r.v = make_uint2(u.x, u.y);
    } else {
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        const f32x4v* q = reinterpret_cast<const f32x4v*>(static_cast<const float*>(p) + i);
        const f32x4v v = NT ? __builtin_nontemporal_load(q) : *q;
        r.v = make_float4(v.x, v.y, v.z, v.w);
    }
    return r;
}
template <bool BF> BEAM_DEV Raw4<BF> zero4() {
    Raw4<BF> r;
    if constexpr (BF) r.v = make_uint2(0u, 0u);
    else r.v = make_float4(0.f, 0.f, 0.f, 0.f);
    return r;
}
BEAM_DEV float4 wid4(Raw4<false> r) { return r.v; }
BEAM_DEV float4 wid4(Raw4<true> r) {
    return make_float4(__uint_as_float(r.v.x << 16), __uint_as_float(r.v.x & 0xFFFF0000u),
                       __uint_as_float(r.v.y << 16), __uint_as_float(r.v.y & 0xFFFF0000u));
}
template <bool BF> BEAM_DEV float rnd_act(float v) {
    if constexpr (BF) return bf16_to_f32(f32_to_bf16(v));
    else return v;
}
template <bool BF> BEAM_DEV void st4(void* p, size_t i, float4 v) {
    if constexpr (BF) {
        const uint32_t a = pack_bf16x2(v.x, v.y);
        const uint32_t b = pack_bf16x2(v.z, v.w);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = make_uint2(a, b);
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = v;
    }
}

BEAM_DEV float4 fma4(float w, float4 y, float4 m) {
    return make_float4(fmaf(w, y.x, m.x), fmaf(w, y.y, m.y), fmaf(w, y.z, m.z), fmaf(w, y.w, m.w));
}

// One workgroup per token; thread i owns the 4-element chunks i, i+256, ...
// RG expert rows have their loads issued together.  With few tokens (a
// grid of T workgroups cannot hide memory latency) RG covers all K rows and
// h and both gammas are loaded up front, so the kernel makes two round
// trips to memory instead of five; with many tokens one row at a time
// leaves registers for the most resident waves (measured on MI355X at
// 16384 tokens with bf16 y: 569 us with 4 rows at a time, 405 us with one).
// Every group of loads (a row's chunks, the residual's h and gamma chunks,
// the pre-norm gamma chunks) is issued whole before any of it is used.
template <bool YBF, bool ABF, int NIT, int RG>
__global__ __launch_bounds__(256) void beam_combine_norm(CombineArgs a) {
    __shared__ float red[4];
    const int t = blockIdx.x, tid = threadIdx.x;
    const int H = a.H, K = a.K;
    const int TK = a.T * K;
    // without pair_row the input row is the token's own row with weight 1
    // (norm boundary on a given m: a dense layer's MLP output or the sum of
    // expert-parallel partials)
    const int32_t* prow = a.pair_row ? a.pair_row + (size_t)t * K : nullptr;
    const float* wrow = a.w ? a.w + (size_t)t * K : nullptr;

    const size_t rowo = (size_t)t * H;
    constexpr bool kEager = RG >= 8;
    Raw4<ABF> hv[NIT], gpo[NIT], gpr[NIT];
    auto load_res = [&](Raw4<ABF>* hh, Raw4<ABF>* gg) {   // residual operands: h and the post-norm gamma
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int i = (it * 256 + tid) * 4;
            hh[it] = i < H ? ldr4<ABF, true>(a.h, rowo + i) : zero4<ABF>();
            gg[it] = i < H ? ldr4<ABF>(a.gpost, i) : zero4<ABF>();
        }
    };
    auto load_pre = [&](Raw4<ABF>* gg) {                  // the pre-norm gamma
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int i = (it * 256 + tid) * 4;
            gg[it] = i < H ? ldr4<ABF>(a.gpre, i) : zero4<ABF>();
        }
    };
    if constexpr (kEager) {
        if (!a.partial_only) {
            load_res(hv, gpo);
            load_pre(gpr);
        }
    }
    float4 m[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) m[it] = make_float4(0.f, 0.f, 0.f, 0.f);
    // K expert rows, RG at a time: indices and weights first, then every
    // row load of the group in flight together; dropped pairs (pair_row -1)
    // and anything outside y are skipped
    for (int k0 = 0; k0 < K; k0 += RG) {
        int rr[RG];
        float wk[RG];
#pragma unroll
        for (int j = 0; j < RG; ++j) {
            const int k = k0 + j;
            const int r = k < K ? (prow ? prow[k] : t) : -1;
            rr[j] = ((unsigned)r < (unsigned)TK) ? r : -1;   // never read outside y
            wk[j] = k < K ? (wrow ? wrow[k] : 1.0f) : 0.f;
        }
        Raw4<YBF> yv[RG][NIT];
#pragma unroll
        for (int j = 0; j < RG; ++j)
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                const int i = (it * 256 + tid) * 4;
                yv[j][it] = (rr[j] >= 0 && i < H) ? ldr4<YBF, true>(a.y, (size_t)rr[j] * H + i) : zero4<YBF>();
            }
#pragma unroll
        for (int j = 0; j < RG; ++j)
#pragma unroll
            for (int it = 0; it < NIT; ++it) m[it] = fma4(wk[j], wid4(yv[j][it]), m[it]);
    }

    if (a.partial_only) {   // one expert-parallel shard's share of m: no norm
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int i = (it * 256 + tid) * 4;
            if (i < H) *reinterpret_cast<float4*>(a.moe_out + rowo + i) = m[it];
        }
        return;
    }
    if constexpr (!kEager) load_res(hv, gpo);   // in flight during the post-norm reduction

    // post-norm
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it)
        if ((it * 256 + tid) * 4 < H)
            ss += (m[it].x * m[it].x + m[it].y * m[it].y) + (m[it].z * m[it].z + m[it].w * m[it].w);
    ss = block_sum<4>(ss, red);
    const float rinv = 1.0f / sqrtf(ss / (float)H + a.eps);

    // residual update; h' replaces m
    float ss2 = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = (it * 256 + tid) * 4;
        if (i < H) {
            if (a.moe_out) *reinterpret_cast<float4*>(a.moe_out + rowo + i) = m[it];
            const float4 g = wid4(gpo[it]);
            const float4 h = wid4(hv[it]);
            float4 hn;
            hn.x = rnd_act<ABF>(a.c_res * h.x + a.c_new * rnd_act<ABF>(m[it].x * rinv * g.x));
            hn.y = rnd_act<ABF>(a.c_res * h.y + a.c_new * rnd_act<ABF>(m[it].y * rinv * g.y));
            hn.z = rnd_act<ABF>(a.c_res * h.z + a.c_new * rnd_act<ABF>(m[it].z * rinv * g.z));
            hn.w = rnd_act<ABF>(a.c_res * h.w + a.c_new * rnd_act<ABF>(m[it].w * rinv * g.w));
            m[it] = hn;
            ss2 += (hn.x * hn.x + hn.y * hn.y) + (hn.z * hn.z + hn.w * hn.w);
        }
    }
    if constexpr (!kEager) load_pre(gpr);   // in flight during the pre-norm reduction
    ss2 = block_sum<4>(ss2, red);
    const float rinv2 = 1.0f / sqrtf(ss2 / (float)H + a.eps);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = (it * 256 + tid) * 4;
        if (i < H) {
            st4<ABF>(a.h, rowo + i, m[it]);
            const float4 g = wid4(gpr[it]);
            st4<ABF>(a.x_next, rowo + i,
                     make_float4(m[it].x * rinv2 * g.x, m[it].y * rinv2 * g.y, m[it].z * rinv2 * g.z,
                                 m[it].w * rinv2 * g.w));
        }
    }
}

template <int NIT, int RG>
static void launch_rg(const CombineArgs& a, hipStream_t st) {
    dim3 grid(a.T), block(256);
    if (a.y_bf16) {
        if (a.act_bf16) hipLaunchKernelGGL((beam_combine_norm<true, true, NIT, RG>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((beam_combine_norm<true, false, NIT, RG>), grid, block, 0, st, a);
    } else {
        if (a.act_bf16) hipLaunchKernelGGL((beam_combine_norm<false, true, NIT, RG>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((beam_combine_norm<false, false, NIT, RG>), grid, block, 0, st, a);
    }
}

template <int NIT>
static void launch_nit(const CombineArgs& a, hipStream_t st) {
    if (a.T <= kSmallT) launch_rg<NIT, 8>(a, st);
    else launch_rg<NIT, 1>(a, st);
}

hipError_t launch_combine_norm(const CombineArgs& a, hipStream_t st) {
    switch ((a.H + 1023) / 1024) {   // 4-element chunks per thread
        case 1: launch_nit<1>(a, st); break;
        case 2: launch_nit<2>(a, st); break;
        case 3: launch_nit<3>(a, st); break;
        case 4: launch_nit<4>(a, st); break;
        case 5: launch_nit<5>(a, st); break;
        case 6: launch_nit<6>(a, st); break;
        case 7: launch_nit<7>(a, st); break;
        default: launch_nit<kMaxIt>(a, st); break;
    }
    return hipGetLastError();
}

}  // namespace beam
