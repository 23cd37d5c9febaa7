// Run-time MXFP4 quantisation (OCP Microscaling Formats v1.0): per block of
// 32 consecutive elements of a row, shared exponent e = floor(log2(amax)) - 2
// (kept in [-127, 127]), elements = nearest E2M1 value of v / 2^e with ties
// to even, saturating at 6.  Used for the layer input of the 4-bit experts
// and for their SwiGLU output before the down projection.  (TokenSpeed x
// Reflection Beam blog, "TensorRT-LLM NVFP4 MoE": 4-bit kernels quantise
// their inputs at run time.)
#include "common.h"
#include "kernels.h"

namespace beam {

// E2M1 code (0..15) of v * 2^-e; the scaling is exact (power of two).
// The kernel below encodes with gfx950's v_cvt_scalef32_pk_fp4_f32 given
// the scale 2^e, which gives these codes for every fp32 input, NaN
// included (a check over all 2^32 inputs at e = -127, -3, 0, 5 and 127 on
// MI355X); this is the definition it matches.
BEAM_DEV uint32_t e2m1_code(float v, int e) {
    const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
    float y = fminf(ldexpf(fabsf(v), -e), 6.0f);    // NaN -> 6 (fminf)
    uint32_t c;
    if (y < 2.0f) {                                 // grid step 0.5: codes 0..4
        c = (uint32_t)rintf(y * 2.0f);              // rintf: nearest, ties to even
    } else if (y < 4.0f) {                          // step 1: 2 -> 4, 3 -> 5, 4 -> 6
        c = (uint32_t)rintf(y) + 2u;
    } else {                                        // step 2: 4 -> 6, 6 -> 7
        c = (uint32_t)rintf(y * 0.5f) + 4u;
    }
    return sign | c;
}

// One thread per 8 consecutive elements; the 4 threads of a 32-block are
// neighbouring lanes of one wave.
template <bool BF>
__global__ __launch_bounds__(256) void beam_quantize_mx_rows(const void* __restrict__ x, int K,
                                                             const int32_t* __restrict__ row_count,
                                                             uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
    const size_t row = blockIdx.y;
    if (row_count && (int)row >= *row_count) return;
    const int i = (blockIdx.x * 256 + threadIdx.x) * 8;     // first element of this thread
    if (i >= K) return;                                      // K % 512 == 0: whole waves exit together
    float v[8];
    if constexpr (BF) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + row * K + i);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + row * K + i);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + row * K + i + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    int e = -127;
    if (amax > 0.f) {
        int ex;
        (void)frexpf(amax, &ex);                             // amax = m * 2^ex, m in [0.5, 1)
        e = min(max(ex - 3, -127), 127);
    }
    // element j -> nibble j: elements 2b, 2b + 1 -> low, high nibble of byte b
    const float scale = ldexpf(1.0f, e);   // exact for e in [-127, 127]
    uint32_t packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], scale, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[2], v[3], scale, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[4], v[5], scale, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[6], v[7], scale, 3);
    *reinterpret_cast<uint32_t*>(q + row * (K / 2) + i / 2) = packed;
    if ((threadIdx.x & 3) == 0) s[row * (K / 32) + i / 32] = (uint8_t)(e + 127);
}

hipError_t launch_quantize_mx(const void* x, bool bf16, int rows, int K, const int32_t* row_count,
                              uint8_t* q, uint8_t* s, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    dim3 grid((K / 8 + 255) / 256, rows);
    if (bf16)
        hipLaunchKernelGGL(beam_quantize_mx_rows<true>, grid, dim3(256), 0, st, x, K, row_count, q, s);
    else
        hipLaunchKernelGGL(beam_quantize_mx_rows<false>, grid, dim3(256), 0, st, x, K, row_count, q, s);
    return hipGetLastError();
}

}  // namespace beam
