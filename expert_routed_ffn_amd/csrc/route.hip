// Router: FP32 logits (bf16 or fp32 activations x fp32 weights, fp32
// accumulation), then sigmoid + correction bias + group-limited top-k +
// renormalised weights in one wave per token.
// (TokenSpeed x Reflection Beam blog, "Fused FP32 routing" and
//  "Architecture"; vLLM Beam summary, MoE section.)
#include "common.h"
#include "kernels.h"

namespace beam {

template <typename XT> BEAM_DEV float ld_x(const XT* p);
template <> BEAM_DEV float ld_x<float>(const float* p) { return *p; }
template <> BEAM_DEV float ld_x<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// 4 consecutive activations as fp32 (bf16 widened exactly)
template <typename XT> BEAM_DEV float4 ld_x4(const XT* p);
template <> BEAM_DEV float4 ld_x4<float>(const float* p) { return *reinterpret_cast<const float4*>(p); }
template <> BEAM_DEV float4 ld_x4<uint16_t>(const uint16_t* p) {
    uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
}

// ---------------------------------------------------------------------------
// Small-batch logits (T <= kSmallT): workgroup (e, s) streams slice s of
// expert e's router row once and forms the partial dot products of all
// tokens with it (the pages' <=16-token GEMV design, re-tiled for
// 256-thread workgroups and split over K so that each thread has little
// serial work); the selection kernel adds the slices in slice order.
// Each thread covers NIT chunks of 4 values of the slice.  The loads of a
// batch of tokens are all issued before the first multiply-add, so the
// activations cost one memory round trip per batch rather than one per
// (token, chunk).
// ---------------------------------------------------------------------------
constexpr int kSmallT = 16;

template <typename XT> struct XRaw;                      // 4 activations as loaded
template <> struct XRaw<uint16_t> { uint2 v; };
template <> struct XRaw<float> { float4 v; };
template <typename XT> BEAM_DEV XRaw<XT> ld_xraw(const XT* p) {
    XRaw<XT> r;
    if constexpr (sizeof(XT) == 2) r.v = *reinterpret_cast<const uint2*>(p);
    else r.v = *reinterpret_cast<const float4*>(p);
    return r;
}
BEAM_DEV float4 widen(XRaw<float> r) { return r.v; }
BEAM_DEV float4 widen(XRaw<uint16_t> r) {
    return make_float4(__uint_as_float(r.v.x << 16), __uint_as_float(r.v.x & 0xFFFF0000u),
                       __uint_as_float(r.v.y << 16), __uint_as_float(r.v.y & 0xFFFF0000u));
}

template <typename XT, int NIT, int TB>
__global__ __launch_bounds__(256) void beam_router_logits_small(
    const XT* __restrict__ x, const float* __restrict__ w, float* __restrict__ logits,
    int T, int H, int E, int kslice) {
    // tokens whose loads are in flight together: TB (8 when T <= 8, else
    // 16), at most about 64 registers of raw activations per thread.  Past
    // T a batch re-reads token T-1 (a load under a token condition would
    // be waited for before the next one is issued).
    constexpr int kCap = 64 / (NIT * (int)sizeof(XT));
    constexpr int kBatch = TB < kCap ? TB : kCap;
    __shared__ float red[4][kSmallT];
    const int e = blockIdx.x;
    const int k0 = blockIdx.y * kslice, k1 = k0 + kslice;
    const float* wr = w + (size_t)e * H;
    logits += (size_t)blockIdx.y * T * E;
    float4 wv[NIT];
    bool ok[NIT];
    int kk[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int k = k0 + (it * 256 + threadIdx.x) * 4;
        ok[it] = k < k1;
        kk[it] = ok[it] ? k : k0;   // chunks past the slice read its first chunk and are not used
        wv[it] = *reinterpret_cast<const float4*>(wr + kk[it]);
    }
    __builtin_amdgcn_sched_barrier(0);   // the weight loads go out first
    float acc[kSmallT];
#pragma unroll
    for (int t0 = 0; t0 < kSmallT; t0 += kBatch) {
        if (t0 >= T) break;
        XRaw<XT> xr[kBatch][NIT];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int t = t0 + j < T ? t0 + j : T - 1;
#pragma unroll
            for (int it = 0; it < NIT; ++it) xr[j][it] = ld_xraw<XT>(x + (size_t)t * H + kk[it]);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            float a = 0.f;
#pragma unroll
            for (int it = 0; it < NIT; ++it) {
                if (ok[it]) {
                    const float4 xv = widen(xr[j][it]);
                    a = fmaf(xv.x, wv[it].x, a);
                    a = fmaf(xv.y, wv[it].y, a);
                    a = fmaf(xv.z, wv[it].z, a);
                    a = fmaf(xv.w, wv[it].w, a);
                }
            }
            acc[t0 + j] = a;
        }
    }
    const int lane = threadIdx.x & 63, wq = threadIdx.x >> 6;
#pragma unroll
    for (int t = 0; t < kSmallT; ++t) {
        if (t < T) {
            const float s = wave_sum(acc[t]);
            if (lane == 0) red[wq][t] = s;
        }
    }
    __syncthreads();
    if (threadIdx.x < T) {
        const int t = threadIdx.x;
        logits[(size_t)t * E + e] = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
    }
}

// ---------------------------------------------------------------------------
// Batched logits: C[T,E] = X[T,H] W[E,H]^T as an fp32 VALU GEMM.  Tile
// 64 tokens x 64 experts per 256-thread workgroup, 4x4 outputs per thread,
// K staged through LDS in chunks of 32 (k-major so each thread reads its
// four tokens / four experts with one 16-byte LDS read).
// ---------------------------------------------------------------------------
constexpr int kLT = 64, kLE = 64, kLK = 32;

template <typename XT>
__global__ __launch_bounds__(256) void beam_router_logits_tiled(
    const XT* __restrict__ x, const float* __restrict__ w, float* __restrict__ logits,
    int T, int H, int E) {
    __shared__ float xs[kLK][kLT + 4];
    __shared__ float ws[kLK][kLE + 4];
    const int t0 = blockIdx.x * kLT, e0 = blockIdx.y * kLE;
    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
    // loader mapping: each thread loads 8 consecutive k of one row
    const int lr = tid >> 2, lk = (tid & 3) * 8;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int k0 = 0; k0 < H; k0 += kLK) {
        {
            const int t = t0 + lr;
            float v[8];
            if (t < T) {
                const float4 a = ld_x4<XT>(x + (size_t)t * H + k0 + lk);
                const float4 b = ld_x4<XT>(x + (size_t)t * H + k0 + lk + 4);
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) xs[lk + i][lr] = v[i];
            const int e = e0 + lr;
            if (e < E) {
                const float4 a = *reinterpret_cast<const float4*>(w + (size_t)e * H + k0 + lk);
                const float4 b = *reinterpret_cast<const float4*>(w + (size_t)e * H + k0 + lk + 4);
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) ws[lk + i][lr] = v[i];
        }
        __syncthreads();
#pragma unroll 8
        for (int k = 0; k < kLK; ++k) {
            const float4 a = *reinterpret_cast<const float4*>(&xs[k][ty * 4]);
            const float4 b = *reinterpret_cast<const float4*>(&ws[k][tx * 4]);
            const float av[4] = {a.x, a.y, a.z, a.w};
            const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tx * 4 + j;
            if (e < E) logits[(size_t)t * E + e] = acc[i][j];
        }
    }
}

// ---------------------------------------------------------------------------
// Batched logits on matrix cores.  The fp32 router weights are split on the
// fly into three bf16 planes, W = hi + mid + lo, each plane holding the next
// 8 significant bits (the split is exact: every residual is representable),
// so every product x*hi, x*mid, x*lo of a bf16 activation is exact in fp32
// and the bf16 MFMA accumulates them in fp32 -- the pages' exact three-way
// bf16 decomposition of the FP32 router for large batches.
// Workgroup tile: 128 tokens x ME experts over 4*ME threads; each wave owns
// 16 experts and all eight 16-token blocks, so every split weight fragment
// feeds eight MFMAs.  ME = 128 (512 threads, 80 KB of LDS) from 1024 tokens
// halves the weight-tile re-reads; below, ME = 64 keeps twice as many
// workgroups for the small grids.  K is split over gridDim.z slices (deterministic
// partial sums, added in slice order by the selection kernel) so small
// batches still fill the chip.  Operands are staged through LDS (rows
// padded to 80 bytes: conflict-free 16-byte fragment reads), double-buffered
// in steps of 32 along K.
// ---------------------------------------------------------------------------
constexpr int kMT = 128, kME = 64, kMK = 32;   // kME: the expert tile's granularity
constexpr int kMEWideT = 1024;                  // tokens from which the expert tile is 2 * kME

BEAM_DEV void split3_bf16(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const uint32_t u = __float_as_uint(v);
    const uint32_t h = u & 0xFFFF0000u;                 // top 8 significant bits
    const float r1 = v - __uint_as_float(h);            // exact
    const uint32_t m = __float_as_uint(r1) & 0xFFFF0000u;
    const float r2 = r1 - __uint_as_float(m);           // exact, <= 8 significant bits
    hi = h >> 16;
    mid = m >> 16;
    lo = __float_as_uint(r2) >> 16;
}

template <int ME>
__global__ __launch_bounds__(4 * ME) void beam_router_logits_mfma(
    const uint16_t* __restrict__ x, const float* __restrict__ w, float* __restrict__ part,
    int T, int H, int E, int kchunk) {
    __shared__ uint4 xs[2][kMT][5];
    __shared__ uint4 wsh[2][3][ME][5];
    const int t0 = blockIdx.x * kMT, e0 = blockIdx.y * ME, sl = blockIdx.z;
    const int kbeg = sl * kchunk, nk = kchunk / kMK;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    // loader role: rows lr + ME * j of the token tile and row lr of the
    // expert tile, 8-element chunk lc
    constexpr int XJ = kMT / ME;
    const int lr = tid >> 2, lc = tid & 3;
    bool tv[XJ];
    const uint16_t* xp[XJ];
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
        tv[j] = t0 + ME * j + lr < T;
        xp[j] = x + (size_t)(tv[j] ? t0 + ME * j + lr : 0) * H + kbeg + 8 * lc;
    }
    const float* wp = w + (size_t)(e0 + lr) * H + kbeg + 8 * lc;
    uint4 xr[XJ];
    float4 w0, w1;
    auto gload = [&](int kk) {
#pragma unroll
        for (int j = 0; j < XJ; ++j)
            xr[j] = tv[j] ? *reinterpret_cast<const uint4*>(xp[j] + kk) : make_uint4(0, 0, 0, 0);
        w0 = *reinterpret_cast<const float4*>(wp + kk);
        w1 = *reinterpret_cast<const float4*>(wp + kk + 4);
    };
    auto swrite = [&](int buf) {
#pragma unroll
        for (int j = 0; j < XJ; ++j) xs[buf][ME * j + lr][lc] = xr[j];
        const float v[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        uint32_t hp[4], mp[4], lp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t h0, m0, l0, h1, m1, l1;
            split3_bf16(v[2 * j], h0, m0, l0);
            split3_bf16(v[2 * j + 1], h1, m1, l1);
            hp[j] = h0 | (h1 << 16);
            mp[j] = m0 | (m1 << 16);
            lp[j] = l0 | (l1 << 16);
        }
        wsh[buf][0][lr][lc] = make_uint4(hp[0], hp[1], hp[2], hp[3]);
        wsh[buf][1][lr][lc] = make_uint4(mp[0], mp[1], mp[2], mp[3]);
        wsh[buf][2][lr][lc] = make_uint4(lp[0], lp[1], lp[2], lp[3]);
    };

    f32x4 acc[kMT / 16];
#pragma unroll
    for (int nb = 0; nb < kMT / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    gload(0);
    swrite(0);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
        const int cur = it & 1;
        const bool more = it + 1 < nk;
        if (more) gload((it + 1) * kMK);
        bf16x8 a[3];
#pragma unroll
        for (int pl = 0; pl < 3; ++pl) a[pl] = __builtin_bit_cast(bf16x8, wsh[cur][pl][wave * 16 + r][g]);
#pragma unroll
        for (int nb = 0; nb < kMT / 16; ++nb) {
            const bf16x8 b = __builtin_bit_cast(bf16x8, xs[cur][nb * 16 + r][g]);
            // small terms first
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2], b, acc[nb], 0, 0, 0);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1], b, acc[nb], 0, 0, 0);
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b, acc[nb], 0, 0, 0);
        }
        if (more) swrite(cur ^ 1);
        __syncthreads();
    }
    // lane holds D[4g+i][r] = expert e0 + 16*wave + 4g + i, token t0 + 16*nb + r
    float* out = part + (size_t)sl * T * E;
#pragma unroll
    for (int nb = 0; nb < kMT / 16; ++nb) {
        const int t = t0 + nb * 16 + r;
        if (t < T)
            *reinterpret_cast<float4*>(out + (size_t)t * E + e0 + wave * 16 + 4 * g) =
                make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
    }
}

// ---------------------------------------------------------------------------
// Selection: one wave per token.  Lane l holds experts [l*EPL, l*EPL+EPL);
// a group of E/G experts spans LPG = E/G/EPL consecutive lanes.
//   s = sigmoid(logit), b = s + bias (fp32)
//   group score = sum of the `topn` largest b of the group (butterfly merge
//   of sorted top-n lists inside the group's lanes)
//   keep the `kg` best groups (ties: lower group)
//   K rounds of a wave-wide arg-max over 64-bit keys (ordered(b) << 32 |
//   ~expert) pick the experts in descending b, ties to the lower expert
//   w_k = scale * s_k / sum_j s_j
// ---------------------------------------------------------------------------
constexpr int kMaxTopn = 4;

// 64-bit value of the lane given by the DPP control CTRL (a permutation
// inside each row of 16 lanes; every lane is active)
template <int CTRL> BEAM_DEV uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}
BEAM_DEV uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
BEAM_DEV uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
// Maximum over the wave, the same in every lane: within each row of 16
// lanes by four DPP exchanges (swap neighbours, swap pairs, mirror halves
// of 8, mirror the row), then the four row maxima read as scalars.  No LDS
// round trips, unlike a butterfly of lane shuffles.
BEAM_DEV uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<0xB1>(v));    // quad_perm [1,0,3,2]
    v = max_u64(v, dpp_u64<0x4E>(v));    // quad_perm [2,3,0,1]
    v = max_u64(v, dpp_u64<0x141>(v));   // row_half_mirror
    v = max_u64(v, dpp_u64<0x140>(v));   // row_mirror
    return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)),
                   max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

template <int EPL>
__global__ __launch_bounds__(256) void beam_route_select(
    const float* __restrict__ part, int nsplit, float* __restrict__ logits_out,
    const float* __restrict__ bias, int32_t* __restrict__ ids_out, float* __restrict__ w_out,
    int T, int E, int G, int kg, int K, int topn, int lpg, float scale) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;   // whole wave exits together
    const size_t TE = (size_t)T * E;

    // logits = partial sums over the K slices, added in slice order; the
    // loads of four slices of all EPL experts are issued together, so the
    // partials cost one memory round trip per four slices, not one per
    // (slice, expert)
    constexpr int kSl = 4;
    const size_t at0 = (size_t)t * E + lane * EPL;
    float z[EPL], bi[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        z[i] = 0.f;
        bi[i] = lane * EPL + i < E ? bias[lane * EPL + i] : 0.f;
    }
    for (int sl0 = 0; sl0 < nsplit; sl0 += kSl) {
        float q[kSl][EPL];
#pragma unroll
        for (int j = 0; j < kSl; ++j)
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                q[j][i] = (sl0 + j < nsplit && lane * EPL + i < E) ? part[(size_t)(sl0 + j) * TE + at0 + i] : 0.f;
#pragma unroll
        for (int j = 0; j < kSl; ++j)
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (sl0 + j < nsplit) z[i] = sl0 + j == 0 ? q[j][i] : z[i] + q[j][i];
    }
    float s[EPL], b[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        if (e < E) {
            if (logits_out && logits_out != part) logits_out[at0 + i] = z[i];
            s[i] = 1.0f / (1.0f + expf(-z[i]));
            b[i] = s[i] + bi[i];
        } else {
            s[i] = 0.f;
            b[i] = -INFINITY;
        }
    }

    // --- group score: top-n of the group's biased scores
    float top[kMaxTopn];
#pragma unroll
    for (int j = 0; j < kMaxTopn; ++j) top[j] = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {          // insertion into a descending list
        float v = b[i];
#pragma unroll
        for (int j = 0; j < kMaxTopn; ++j) {
            const float hi = fmaxf(top[j], v), lo = fminf(top[j], v);
            top[j] = hi;
            v = lo;
        }
    }
    for (int o = 1; o < lpg; o <<= 1) {      // merge with the partner lane's list
        // both lists descend: max(a_j, b_{n-1-j}) is the top-n multiset
        // (bitonic), then a half-cleaner network sorts it again
        float c[kMaxTopn];
#pragma unroll
        for (int j = 0; j < kMaxTopn; ++j)
            c[j] = fmaxf(top[j], __shfl_xor(top[kMaxTopn - 1 - j], o, kWave));
#pragma unroll
        for (int d = kMaxTopn / 2; d > 0; d >>= 1)
#pragma unroll
            for (int j = 0; j < kMaxTopn; ++j)
                if ((j & d) == 0) {
                    const float hi = fmaxf(c[j], c[j + d]), lo = fminf(c[j], c[j + d]);
                    c[j] = hi;
                    c[j + d] = lo;
                }
#pragma unroll
        for (int j = 0; j < kMaxTopn; ++j) top[j] = c[j];
    }
    float gs = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopn; ++j)
        if (j < topn) gs += top[j];

    // --- keep the kg best groups
    const int my_group = lane / lpg;
    int rank = 0;
    for (int g = 0; g < G; ++g) {
        const float o = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gs), g * lpg));
        rank += (o > gs) || (o == gs && g < my_group);
    }
    const bool group_kept = (my_group < G) && (rank < kg);

    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        key[i] = (group_kept && e < E)
                     ? ((uint64_t)ordered_bits(b[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)
                     : 0ull;
    }

    // --- K rounds of wave arg-max
    float my_s = 0.f, ssum = 0.f;
    int my_id = 0;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_u64(best);
        const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
        const int owner = e / EPL, slot = e - owner * EPL;
        float se = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (i == slot) se = s[i];
        se = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(se), owner));
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == slot) key[i] = 0ull;
        }
        ssum += se;
        if (lane == k) { my_s = se; my_id = e; }
    }
    if (lane < K) {
        ids_out[(size_t)t * K + lane] = my_id;
        w_out[(size_t)t * K + lane] = scale * my_s / ssum;
    }
}

int route_epl(int E) { return E <= 64 ? 1 : (E <= 128 ? 2 : 4); }


// Expert tile of the matrix-core router for T tokens.
static int route_me(int T, int E) { return (T >= kMEWideT && E % (2 * kME) == 0) ? 2 * kME : kME; }

// K slices of the matrix-core router for T tokens: enough workgroups to
// fill the chip (about 640 with the 64-expert tile, three per CU; 256 with
// the 128-expert tile, whose 80 KB of LDS leave one or two per CU), each
// slice a multiple of 32 that divides H, at least 256.
int route_splits(int T, int H, int E) {
    if (T <= 0 || E % kME != 0) return 1;   // only the matrix-core router splits K
    const int me = route_me(T, E);
    const int tiles = ((T + kMT - 1) / kMT) * (E / me);
    const int target = me == kME ? 640 : 256;
    int want = (target + tiles - 1) / tiles;
    const int steps = H / kMK;
    if (want > H / 256) want = H / 256;
    for (int sl = want; sl > 1; --sl)
        if (steps % sl == 0) return sl;
    return 1;
}

bool route_uses_mfma(int T, int E, bool x_bf16) { return T > kSmallT && x_bf16 && E % kME == 0; }

// K slices of the small-batch router: four for wide rows (slices of at
// least 1024 values, a multiple of 4 each), else one
static int small_splits(int H) { return (H >= 4096 && H % 16 == 0) ? 4 : 1; }

static int route_nsplit(int T, int H, int E, bool x_bf16) {
    if (T <= kSmallT) return small_splits(H);
    return route_uses_mfma(T, E, x_bf16) ? route_splits(T, H, E) : 1;
}

size_t route_partials_bytes(int T, int H, int E) {
    const int s = std::max(route_nsplit(T, H, E, true), route_nsplit(T, H, E, false));
    return (size_t)s * T * E * sizeof(float);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
    const int T = a.T, H = a.H, E = a.E;
    // partial logits: the caller's logits_out when there is a single slice,
    // else the workspace
    const int nsplit = route_nsplit(T, H, E, a.x_bf16);
    float* part = (nsplit == 1 && a.logits_out) ? a.logits_out : a.partials;
    if (T <= kSmallT) {
        const dim3 grid(E, nsplit);
        const int ks = H / nsplit;   // <= 4096 (small_splits), a multiple of 4
        const int nit = (ks + 1023) / 1024;
        auto go = [&](auto nitc, auto tbc) {
            constexpr int NIT = decltype(nitc)::value, TB = decltype(tbc)::value;
            if (a.x_bf16)
                hipLaunchKernelGGL((beam_router_logits_small<uint16_t, NIT, TB>), grid, dim3(256), 0, st,
                                   (const uint16_t*)a.x, a.w, part, T, H, E, ks);
            else
                hipLaunchKernelGGL((beam_router_logits_small<float, NIT, TB>), grid, dim3(256), 0, st,
                                   (const float*)a.x, a.w, part, T, H, E, ks);
        };
        auto go_nit = [&](auto tbc) {
            if (nit <= 1) go(std::integral_constant<int, 1>{}, tbc);
            else if (nit <= 2) go(std::integral_constant<int, 2>{}, tbc);
            else go(std::integral_constant<int, 4>{}, tbc);
        };
        if (T <= 8) go_nit(std::integral_constant<int, 8>{});
        else go_nit(std::integral_constant<int, kSmallT>{});
    } else if (route_uses_mfma(T, E, a.x_bf16)) {
        const int me = route_me(T, E);
        dim3 grid((T + kMT - 1) / kMT, E / me, nsplit);
        if (me == kME)
            hipLaunchKernelGGL(beam_router_logits_mfma<kME>, grid, dim3(4 * kME), 0, st, (const uint16_t*)a.x, a.w,
                               part, T, H, E, H / nsplit);
        else
            hipLaunchKernelGGL(beam_router_logits_mfma<2 * kME>, grid, dim3(8 * kME), 0, st, (const uint16_t*)a.x,
                               a.w, part, T, H, E, H / nsplit);
    } else {
        dim3 grid((T + kLT - 1) / kLT, (E + kLE - 1) / kLE);
        if (a.x_bf16)
            hipLaunchKernelGGL(beam_router_logits_tiled<uint16_t>, grid, dim3(256), 0, st,
                               (const uint16_t*)a.x, a.w, part, T, H, E);
        else
            hipLaunchKernelGGL(beam_router_logits_tiled<float>, grid, dim3(256), 0, st,
                               (const float*)a.x, a.w, part, T, H, E);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int epl = route_epl(E);
    const int lpg = (E / a.G) / epl;
    dim3 grid((T + 3) / 4);
    switch (epl) {
        case 1:
            hipLaunchKernelGGL(beam_route_select<1>, grid, dim3(256), 0, st, part, nsplit, a.logits_out,
                               a.bias, a.ids, a.wts, T, E, a.G, a.kg, a.K, a.topn, lpg, a.scale);
            break;
        case 2:
            hipLaunchKernelGGL(beam_route_select<2>, grid, dim3(256), 0, st, part, nsplit, a.logits_out,
                               a.bias, a.ids, a.wts, T, E, a.G, a.kg, a.K, a.topn, lpg, a.scale);
            break;
        default:
            hipLaunchKernelGGL(beam_route_select<4>, grid, dim3(256), 0, st, part, nsplit, a.logits_out,
                               a.bias, a.ids, a.wts, T, E, a.G, a.kg, a.K, a.topn, lpg, a.scale);
            break;
    }
    return hipGetLastError();
}

}  // namespace beam
