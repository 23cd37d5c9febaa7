// Permutation: stable expert-major grouping of the T*K (token, slot) pairs
// via an LDS histogram, an exclusive prefix sum and an order-preserving
// scatter; plus the optional dynamic per-token e4m3 quantisation of x.
// (vLLM Beam summary, kernel list: the routing kernels of the MoE path;
//  TokenSpeed blog, "TensorRT-LLM NVFP4 MoE": input quantisation is
//  independent of the routes; Gaudi cookbook, "What was built": dynamic
//  per-token FP8 activations.)
#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int kPermThreads = 256;
constexpr int kPermFused = 4096;   // pairs up to which one workgroup does the whole permutation
// pairs per workgroup in the multi-block path: the scatter of a chunk is
// serial over its 256-pair steps, so small chunks spread it over many
// workgroups (128 at 131072 pairs); the scan reads the chunks' histograms
// 32 at a time, so their number costs it little
constexpr int kPermChunk = 1024;
constexpr int kMaxE = 256;

// Stable scatter of pairs [begin, end) given per-expert cursors in LDS
// (cursor[e] = first free permuted row of expert e for this range).  Pairs
// are taken 256 at a time; inside a wave the rank among equal experts comes
// from ballots over the expert id bits, and the four waves of a chunk
// claim their rows one after another so the order of p is kept.
BEAM_DEV void stable_scatter(const int32_t* __restrict__ ids, int e_base, int begin, int end, int K,
                             int E, int ebits, int* cursor, int32_t* __restrict__ row_token,
                             int32_t* __restrict__ pair_row) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = begin; base < end; base += kPermThreads) {
        const int p = base + threadIdx.x;
        bool valid = p < end;
        int e = valid ? ids[p] - e_base : 0;
        if (valid && (unsigned)e >= (unsigned)E) {   // out-of-range ids are dropped
            pair_row[p] = -1;
            valid = false;
            e = 0;
        }
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < ebits; ++bit) {
            const bool b = (e >> bit) & 1;
            const uint64_t bal = __ballot(valid && b);
            peers &= b ? bal : ~bal;
        }
        const int rank = __popcll(peers & lt_mask);
        const int cnt = __popcll(peers);
        for (int ww = 0; ww < kPermThreads / 64; ++ww) {
            if (w == ww && valid) {
                const int r = cursor[e] + rank;
                row_token[r] = p / K;
                pair_row[p] = r;
                if (rank == cnt - 1) cursor[e] = r + 1;
            }
            __syncthreads();
        }
    }
}

// Whole permutation in one workgroup (T*K <= kPermFused).
__global__ __launch_bounds__(kPermThreads) void beam_permute_fused(
    const int32_t* __restrict__ ids, int e_base, int TK, int K, int E, int ebits,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token, int32_t* __restrict__ pair_row) {
    __shared__ int hist[kMaxE];
    __shared__ int cursor[kMaxE];
    __shared__ int tmp[4];
    const int tid = threadIdx.x;
    if (tid < E) hist[tid] = 0;
    __syncthreads();
    for (int p = tid; p < TK; p += kPermThreads) {
        const int e = ids[p] - e_base;
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    int total;
    const int excl = block_exclusive_scan(tid < E ? hist[tid] : 0, tmp, &total);
    if (tid < E) {
        offsets[tid] = excl;
        cursor[tid] = excl;
    }
    if (tid == 0) offsets[E] = total;
    __syncthreads();
    stable_scatter(ids, e_base, 0, TK, K, E, ebits, cursor, row_token, pair_row);
}

// Multi-block path, step 1: per-chunk histograms bh[b][e].
__global__ __launch_bounds__(kPermThreads) void beam_permute_hist(
    const int32_t* __restrict__ ids, int e_base, int TK, int E, int chunk, int32_t* __restrict__ bh) {
    __shared__ int hist[kMaxE];
    const int tid = threadIdx.x;
    if (tid < E) hist[tid] = 0;
    __syncthreads();
    const int begin = blockIdx.x * chunk;
    const int end = min(begin + chunk, TK);
    for (int p = begin + tid; p < end; p += kPermThreads) {
        const int e = ids[p] - e_base;
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    if (tid < E) bh[(size_t)blockIdx.x * E + tid] = hist[tid];
}

// Step 2 (one workgroup): expert offsets and each chunk's first row per expert.
__global__ __launch_bounds__(kPermThreads) void beam_permute_scan(
    const int32_t* __restrict__ bh, int nb, int TK, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ bbase) {
    __shared__ int tmp[4];
    const int e = threadIdx.x;
    // the chunks' counts of expert e, kScanBatch loads in flight at a time
    // (indices past the last chunk re-read it and count zero)
    constexpr int kScanBatch = 32;
    const int ec = e < E ? e : 0;
    auto load_batch = [&](int b0, int (&v)[kScanBatch]) {
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) v[j] = bh[(size_t)min(b0 + j, nb - 1) * E + ec];
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) v[j] = b0 + j < nb ? v[j] : 0;
    };
    int tot = 0;
    for (int b0 = 0; b0 < nb; b0 += kScanBatch) {
        int v[kScanBatch];
        load_batch(b0, v);
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) tot += v[j];
    }
    int total;
    const int excl = block_exclusive_scan(e < E ? tot : 0, tmp, &total);
    if (e < E) offsets[e] = excl;
    int run = excl;
    for (int b0 = 0; b0 < nb; b0 += kScanBatch) {
        int v[kScanBatch];
        load_batch(b0, v);
#pragma unroll
        for (int j = 0; j < kScanBatch; ++j) {
            if (e < E && b0 + j < nb) bbase[(size_t)(b0 + j) * E + e] = run;
            run += v[j];
        }
    }
    if (e == 0) offsets[E] = total;
}

// Step 3: stable scatter of each chunk from its per-expert base rows.
__global__ __launch_bounds__(kPermThreads) void beam_permute_scatter(
    const int32_t* __restrict__ ids, int e_base, int TK, int K, int E, int ebits, int chunk,
    const int32_t* __restrict__ bbase, int32_t* __restrict__ row_token,
    int32_t* __restrict__ pair_row) {
    __shared__ int cursor[kMaxE];
    const int tid = threadIdx.x;
    if (tid < E) cursor[tid] = bbase[(size_t)blockIdx.x * E + tid];
    __syncthreads();
    const int begin = blockIdx.x * chunk;
    const int end = min(begin + chunk, TK);
    stable_scatter(ids, e_base, begin, end, K, E, ebits, cursor, row_token, pair_row);
}

// Dynamic per-token e4m3 quantisation of x: one wave per token row, four
// rows per workgroup.
template <int NIT>
__global__ __launch_bounds__(256) void beam_quantize_x_e4m3(
    const uint16_t* __restrict__ x, int T, int H, uint8_t* __restrict__ xq, float* __restrict__ xscale) {
    const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (size_t)T) return;   // whole wave exits together
    const uint16_t* xr = x + row * H;
    auto load_raw = [&](int i) { return *reinterpret_cast<const uint2*>(xr + i); };   // 4 bf16
    auto widen = [](uint2 u) {
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                           __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
    };
    quantize_row_e4m3_wave<NIT>(load_raw, widen, H, xq + row * H, xscale + row);
}

static int n_chunks(int TK) { return TK <= kPermFused ? 1 : (TK + kPermChunk - 1) / kPermChunk; }

size_t permute_ws_bytes(int T, int K, int E) {
    const int nb = n_chunks(T * K);
    return nb <= 1 ? 0 : 2 * (size_t)nb * E * sizeof(int32_t);
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t st) {
    const int TK = a.T * a.K;
    int ebits = 0;
    while ((1 << ebits) < a.E) ++ebits;
    const int nb = n_chunks(TK);
    if (nb <= 1) {
        hipLaunchKernelGGL(beam_permute_fused, dim3(1), dim3(kPermThreads), 0, st, a.ids, a.e_base, TK, a.K,
                           a.E, ebits, a.offsets, a.row_token, a.pair_row);
    } else {
        int32_t* bh = static_cast<int32_t*>(a.ws);
        int32_t* bb = bh + (size_t)nb * a.E;
        const int chunk = kPermChunk;
        hipLaunchKernelGGL(beam_permute_hist, dim3(nb), dim3(kPermThreads), 0, st, a.ids, a.e_base, TK, a.E,
                           chunk, bh);
        hipLaunchKernelGGL(beam_permute_scan, dim3(1), dim3(kPermThreads), 0, st, bh, nb, TK, a.E,
                           a.offsets, bb);
        hipLaunchKernelGGL(beam_permute_scatter, dim3(nb), dim3(kPermThreads), 0, st, a.ids, a.e_base, TK, a.K,
                           a.E, ebits, chunk, bb, a.row_token, a.pair_row);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.xq == nullptr) return err;
    return launch_quantize_x_e4m3(a.x, a.T, a.H, a.xq, a.xscale, st);
}

hipError_t launch_quantize_x_e4m3(const uint16_t* x, int T, int H, uint8_t* xq, float* xscale, hipStream_t st) {
    const dim3 grid((T + 3) / 4);   // H <= 8192: at most 32 chunks of 4 per lane
    if (H <= 2048)
        hipLaunchKernelGGL(beam_quantize_x_e4m3<8>, grid, dim3(256), 0, st, x, T, H, xq, xscale);
    else if (H <= 4096)
        hipLaunchKernelGGL(beam_quantize_x_e4m3<16>, grid, dim3(256), 0, st, x, T, H, xq, xscale);
    else if (H <= 5120)   // the Beam hidden size
        hipLaunchKernelGGL(beam_quantize_x_e4m3<20>, grid, dim3(256), 0, st, x, T, H, xq, xscale);
    else
        hipLaunchKernelGGL(beam_quantize_x_e4m3<32>, grid, dim3(256), 0, st, x, T, H, xq, xscale);
    return hipGetLastError();
}

}  // namespace beam
