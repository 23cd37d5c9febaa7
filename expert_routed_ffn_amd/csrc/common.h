// Device helpers shared by the Beam MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define BEAM_DEV __device__ __forceinline__

namespace beam {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bf16 bits

BEAM_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// round-to-nearest-even fp32 -> bf16; NaN stays a (quiet) NaN
// fp32 -> bf16, round to nearest even (NaN stays NaN): the gfx950
// conversion instruction
BEAM_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }

// two values, lo in the low half (one conversion instruction)
BEAM_DEV uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2v __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v{lo, hi}), bf16x2v));
}

// ---------------------------------------------------------------- e4m3 bits

// OCP E4M3FN encode: round to nearest even, saturate to +-448, NaN -> 0x7F.
BEAM_DEV uint32_t f32_to_e4m3(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return sign | 0x7Fu;          // NaN
    if (a >= 0x43E00000u) return sign | 0x7Eu;         // |f| >= 448 (incl. inf)
    if (a < 0x3C800000u) {                             // |f| < 2^-6: step 2^-9
        float s = __uint_as_float(a) * 512.0f;         // exact, < 8
        return sign | uint32_t(rintf(s));              // 8 -> 0x08 = 2^-6
    }
    uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;   // keep 3 mantissa bits, RNE
    return sign | (r - (120u << 3));                   // rebias exponent 127 -> 7
}

// Four values to OCP E4M3FN codes (byte j = value j), bit for bit as
// f32_to_e4m3: gfx950's conversion instruction rounds to nearest even and
// agrees with that formula for every fp32 input below 464 in magnitude (a
// check over all 2^32 inputs on MI355X); larger values are clamped to
// +-448 first (the saturated code 0x7E), and a NaN keeps its sign bit
// (0x7F / 0xFF), which the instruction does not.
BEAM_DEV uint32_t e4m3x4(float a, float b, float c, float d) {
    const float v[4] = {a, b, c, d};
    float w[4];
    bool any_nan = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w[j] = fminf(fmaxf(v[j], -448.0f), 448.0f);
        any_nan |= v[j] != v[j];
    }
    uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(w[0], w[1], 0, false);
    r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(w[2], w[3], (int)r, true);
    if (any_nan) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (v[j] != v[j])
                r = (r & ~(0xFFu << (8 * j))) | ((((__float_as_uint(v[j]) >> 24) & 0x80u) | 0x7Fu) << (8 * j));
    }
    return r;
}

// ---------------------------------------------------------------- reductions

BEAM_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

BEAM_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Block-wide sum; `red` is __shared__ float[blockDim/64]; every thread gets the sum.
template <int NWAVES>
BEAM_DEV float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) s += red[i];
    __syncthreads();
    return s;
}

template <int NWAVES>
BEAM_DEV float block_max(float v, float* red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = red[0];
#pragma unroll
    for (int i = 1; i < NWAVES; ++i) s = fmaxf(s, red[i]);
    __syncthreads();
    return s;
}

// order-preserving map of an fp32 onto uint32 (larger float -> larger uint)
BEAM_DEV uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// g * sigmoid(g), with the hardware reciprocal (1 ulp) in place of a
// correctly rounded division
BEAM_DEV float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

}  // namespace beam

namespace beam {

// Dynamic per-row e4m3 quantisation of `n` values (n % 4 == 0) by one
// wave, with no barriers:
//   scale = amax / 448 (correctly rounded fp32; 1 for an all-zero row),
//   code  = e4m3(v / scale) with a correctly rounded fp32 division.
// Lane l holds the 4-element chunks l, l + 64, ...; NIT >= n / 256 chunks
// per lane.  `load_raw(i)` loads chunk i as stored and `widen` turns it into
// fp32; all NIT loads are issued before the first is widened (lanes past n
// re-read chunk 0 and drop it), so a lane's loads cost one memory round
// trip.  The row maximum is exact whatever the reduction order.
template <int NIT, typename LoadRaw, typename Widen>
BEAM_DEV void quantize_row_e4m3_wave(LoadRaw load_raw, Widen widen, int n, uint8_t* __restrict__ q,
                                     float* scale_out) {
    const int lane = threadIdx.x & 63;
    decltype(load_raw(0)) raw[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = (it * 64 + lane) * 4;
        raw[it] = load_raw(i < n ? i : 0);
    }
    float v[NIT][4];
    float amax = 0.f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = (it * 64 + lane) * 4;
        const float4 f = widen(raw[it]);
        v[it][0] = f.x; v[it][1] = f.y; v[it][2] = f.z; v[it][3] = f.w;
        if (i < n) {
#pragma unroll
            for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(v[it][j]));
        }
    }
    amax = wave_max(amax);
    const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = (it * 64 + lane) * 4;
        if (i < n) {
            *reinterpret_cast<uint32_t*>(q + i) = e4m3x4(__fdiv_rn(v[it][0], s), __fdiv_rn(v[it][1], s),
                                                         __fdiv_rn(v[it][2], s), __fdiv_rn(v[it][3], s));
        }
    }
    if (lane == 0) *scale_out = s;
}

// Exclusive prefix sum of v over a 256-thread block.  Returns the exclusive
// value; *total gets the block total.  `tmp` is __shared__ int[4].
BEAM_DEV int block_exclusive_scan(int v, int* tmp, int* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
    }
    if (lane == 63) tmp[w] = incl;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        before += (i < w) ? tmp[i] : 0;
        tot += tmp[i];
    }
    __syncthreads();
    *total = tot;
    return before + incl - v;
}

}  // namespace beam
