// Grouped SwiGLU experts: GEMM1 (gate and up projections with SwiGLU fused
// into the epilogue) and GEMM2 (down projection) over the expert-grouped
// rows, bf16, fp8-e4m3 or MXFP4 on MFMA, plus a plain fp32 path for small
// shapes.
// (TokenSpeed x Reflection Beam blog, "TensorRT-LLM NVFP4 MoE": both expert
//  GEMMs with SwiGLU fused into the first; "NVFP4 and FP8 checkpoints":
//  4-bit weights; Gaudi cookbook, "What was built" and "EP vs TP quality":
//  per-channel FP8 weights, dynamic per-token activations, down-projection
//  input quantised per token over all d_ff.)
//
// Work decomposition.  A work item is (expert e, up to MC consecutive
// permuted rows of e), taken from the expert offsets on the device, so the
// host never reads routing results (the direct kernels find their item in
// the offsets; the others read a list a one-block kernel builds).  A
// 256-thread workgroup takes one item and one N-tile of weight rows; each
// of its 4 waves owns two 16-row MFMA tiles of weights (four on the wide
// path) -- GEMM1: gate rows and the matching up rows, so SwiGLU happens in
// registers; GEMM2: output rows -- and the item's rows in blocks of 16.  Weights stream from HBM
// straight into MFMA A-operand registers, each weight byte read once per
// item, from the packed layout (pack.hip): every weight load instruction of
// a wave reads 1 KiB of contiguous whole cache lines, non-temporally.
// Activation rows (few, L2-resident) are the B operand; lane (r, g) reads
// bytes [64 s + 16 g, +16) of its row for piece s, the same k bytes the
// packed A fragment holds.  bf16: MFMA step s uses piece s.  fp8: MFMA step
// t uses pieces 2t and 2t+1 (32 bytes = the lane's 32 k values).
#include <type_traits>

#include <atomic>

#include "common.h"
#include "kernels.h"

namespace beam {

constexpr int kKIterBytes = 256;    // bytes of one row consumed per K iteration

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

BEAM_DEV uint4 ld16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// streamed-once weights: non-temporal 16-byte load
BEAM_DEV uint4 ld16_nt(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- items

__global__ __launch_bounds__(256) void beam_build_items(const int32_t* __restrict__ offsets, int E,
                                                        int MC, int4* __restrict__ items,
                                                        int* __restrict__ n_items,
                                                        int* __restrict__ first_item,
                                                        int* __restrict__ unit_ctr) {
    __shared__ int tmp[4];
    const int e = threadIdx.x;
    const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int nch = (cnt + MC - 1) / MC;
    int total;
    const int first = block_exclusive_scan(nch, tmp, &total);
    // .w = (index of the item within its expert << 16) | items of the expert;
    // an expert with more than one item has its weights read by several
    // workgroups, which should then keep them cacheable
    for (int c = 0; c < nch; ++c)
        items[first + c] = make_int4(e, offsets[e] + c * MC, min(MC, cnt - c * MC), (c << 16) | nch);
    if (e < E) first_item[e] = first;
    if (e < 16) unit_ctr[e] = 0;   // the wide kernels' per-XCD unit counters
    if (e == 0) {
        *n_items = total;
        first_item[E] = total;
    }
}

// ---------------------------------------------------------------- MFMA

typedef int i32x4v __attribute__((ext_vector_type(4)));

// bytes of one row of k values
template <int KIND> BEAM_DEV constexpr int row_bytes(int k) {
    return KIND == W_BF16 ? 2 * k : (KIND == W_MXFP4 ? k / 2 : k);
}

// One 256-byte K iteration of MXFP4 operands (512 E2M1 values of the row):
// piece s is one K = 128 MFMA in which lane (r, g) holds the 32 values of
// block 4 s + g of the iteration, i.e. bytes [64 s + 16 g, +16) -- the same
// bytes on the weight (A) and the activation (B) side.  sa / sb hold the
// 16 E8M0 codes of the iteration's blocks for the lane's weight row /
// activation row; block 4 s + g is byte g of word s.
BEAM_DEV void mfma_kiter_mx(const uint4 (&a)[4], const uint4 (&b)[4], const uint4& sa, const uint4& sb,
                            f32x4& acc) {
    const int sh = 8 * ((threadIdx.x & 63) >> 4);
    const uint32_t wa[4] = {sa.x, sa.y, sa.z, sa.w};
    const uint32_t wb[4] = {sb.x, sb.y, sb.z, sb.w};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const i32x8 av = {(int)a[s].x, (int)a[s].y, (int)a[s].z, (int)a[s].w, 0, 0, 0, 0};
        const i32x8 bv = {(int)b[s].x, (int)b[s].y, (int)b[s].z, (int)b[s].w, 0, 0, 0, 0};
        // formats 4/4 = E2M1 x E2M1 (the low 4 dwords of each operand);
        // per-lane E8M0 scales from byte 0 of the shifted words
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, 0, (int)((wa[s] >> sh) & 0xFF),
                                                               0, (int)((wb[s] >> sh) & 0xFF));
    }
}

template <int KIND>
BEAM_DEV void mfma_kiter(const uint4 (&a)[4], const uint4 (&b)[4], f32x4& acc) {
    if constexpr (KIND == W_BF16) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[s]),
                                                          __builtin_bit_cast(bf16x8, b[s]), acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const i32x8 av = __builtin_shufflevector(__builtin_bit_cast(i32x4v, a[2 * s]),
                                                     __builtin_bit_cast(i32x4v, a[2 * s + 1]),
                                                     0, 1, 2, 3, 4, 5, 6, 7);
            const i32x8 bv = __builtin_shufflevector(__builtin_bit_cast(i32x4v, b[2 * s]),
                                                     __builtin_bit_cast(i32x4v, b[2 * s + 1]),
                                                     0, 1, 2, 3, 4, 5, 6, 7);
            // formats 0/0 = e4m3 x e4m3; block scales 127 = 2^0 (unscaled)
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
        }
    }
}

struct GemmParams {
    const int4* items;
    const int* n_items;
    int n_tiles;
    const uint8_t* act;        // G1: x rows (bf16 or e4m3), gathered by token; G2: a rows
    const int32_t* row_token;  // G1 only
    const float* act_scale;    // fp8: G1 per token, G2 per row
    const uint8_t* W;          // expert weight stacks
    const float* wscale;       // fp8: per output row
    const uint8_t* mx_act;     // MXFP4: E8M0 codes of the activation rows [rows, K/32]
    const uint8_t* mx_w;       // MXFP4: E8M0 codes of the weight rows [E, rows, K/32]
    int ksplit;                // direct kernel: K slices (gridDim.y); GEMM1 then
                               // stores raw gate/up sums, fp32 [row][2F] per slice
    size_t out_slice;          // elements between the fp32 outputs of two slices
    int H, F;
    void* out;
    bool out_bf16;             // G2 only
    // wide path: per expert (E + 1 entries) the index of its first item and
    // its first row; the experts' units are taken in that order
    const int* first_item;
    const int32_t* offsets;
    int E;
    int* unit_ctr;             // wide path: 8 unit counters, one per XCD, zero at launch
    int identity_rows;         // direct path: > 0 = one expert whose rows are tokens 0..identity_rows-1
};

template <int V> struct IC { static constexpr int value = V; };

// GEMM1 epilogue of 4 a-columns [f, f+4) of one row: lane holds the gate
// and up accumulators of weight rows f + i (fp8: scaled back to real units).
// sx, sg, su: the fp8 scales of the token and of the gate / up rows (unused
// for the other kinds).
template <int KIND>
BEAM_DEV void store_swiglu_s(const GemmParams& p, int f, size_t row, float sx, float4 sg, float4 su,
                             const f32x4& accg, const f32x4& accu) {
    float gv[4], uv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { gv[i] = accg[i]; uv[i] = accu[i]; }
    if constexpr (KIND == W_FP8) {
        gv[0] *= sx * sg.x; gv[1] *= sx * sg.y; gv[2] *= sx * sg.z; gv[3] *= sx * sg.w;
        uv[0] *= sx * su.x; uv[1] *= sx * su.y; uv[2] *= sx * su.z; uv[3] *= sx * su.w;
        float4 av;
        av.x = silu_f32(gv[0]) * uv[0];
        av.y = silu_f32(gv[1]) * uv[1];
        av.z = silu_f32(gv[2]) * uv[2];
        av.w = silu_f32(gv[3]) * uv[3];
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + row * p.F + f) = av;
    } else if constexpr (KIND == W_MXFP4) {   // the MX scales are inside the MFMA
        const float4 av = make_float4(silu_f32(gv[0]) * uv[0], silu_f32(gv[1]) * uv[1],
                                      silu_f32(gv[2]) * uv[2], silu_f32(gv[3]) * uv[3]);
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + row * p.F + f) = av;
    } else {
        float av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = silu_f32(gv[i]) * uv[i];
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + row * p.F + f) =
            make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
    }
}

template <int KIND>
BEAM_DEV void store_swiglu(const GemmParams& p, int e, int f, size_t row, int tok, const f32x4& accg,
                           const f32x4& accu) {
    float sx = 1.f;
    float4 sg = make_float4(1.f, 1.f, 1.f, 1.f), su = sg;
    if constexpr (KIND == W_FP8) {
        const int nrows_w = 2 * p.F;
        sx = p.act_scale[tok];
        sg = *reinterpret_cast<const float4*>(p.wscale + (size_t)e * nrows_w + f);
        su = *reinterpret_cast<const float4*>(p.wscale + (size_t)e * nrows_w + p.F + f);
    }
    store_swiglu_s<KIND>(p, f, row, sx, sg, su, accg, accu);
}

// GEMM2 epilogue of 4 output columns [o, o+4) of one row; sa, sw: the fp8
// scales of the row and of the weight rows (unused for the other kinds).
template <int KIND>
BEAM_DEV void store_out_s(const GemmParams& p, int o, size_t row, float sa, float4 sw, const f32x4& acc) {
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = acc[i];
    if constexpr (KIND == W_FP8) {
        v[0] *= sa * sw.x; v[1] *= sa * sw.y; v[2] *= sa * sw.z; v[3] *= sa * sw.w;
    }
    if (p.out_bf16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + row * p.H + o) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + row * p.H + o) =
            make_float4(v[0], v[1], v[2], v[3]);
    }
}

template <int KIND>
BEAM_DEV void store_out(const GemmParams& p, int e, int o, size_t row, const f32x4& acc) {
    float sa = 1.f;
    float4 sw = make_float4(1.f, 1.f, 1.f, 1.f);
    if constexpr (KIND == W_FP8) {
        sa = p.act_scale[row];
        sw = *reinterpret_cast<const float4*>(p.wscale + (size_t)e * p.H + o);
    }
    store_out_s<KIND>(p, o, row, sa, sw, acc);
}

// Epilogue for one 16-column block: lane holds D[4g+i][r] = weight row
// (a0/a1 + 4g + i) x item row `row`.  GEMM1 applies SwiGLU (and the fp8
// scales) and writes a; GEMM2 writes y.
template <int KIND, bool G1>
BEAM_DEV void store_block(const GemmParams& p, int e, int a0, int a1, size_t row, int tok,
                          const f32x4& acc0, const f32x4& acc1) {
    const int g = (threadIdx.x & 63) >> 4;
    if constexpr (G1) {
        store_swiglu<KIND>(p, e, a0 + 4 * g, row, tok, acc0, acc1);
    } else {
        store_out<KIND>(p, e, a0 + 4 * g, row, acc0);
        store_out<KIND>(p, e, a1 + 4 * g, row, acc1);
    }
}

// Weight rows of this wave: GEMM1 16 gate rows + the matching 16 up rows of
// N-tile `tile` (64 + 64 rows per workgroup); GEMM2 32 output rows (128 per
// workgroup).  Returns the packed-tile base pointers of the lane's pieces.
template <int KIND, bool G1>
BEAM_DEV void weight_rows(const GemmParams& p, int e, int tile, int& a0, int& a1, const uint8_t*& pa0,
                          const uint8_t*& pa1) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kbytes = row_bytes<KIND>(G1 ? p.H : p.F);
    const int nrows_w = G1 ? 2 * p.F : p.H;
    a0 = G1 ? tile * 64 + wave * 16 : tile * 128 + wave * 32;
    a1 = G1 ? p.F + a0 : a0 + 16;
    const uint8_t* We = p.W + (size_t)e * nrows_w * kbytes;
    // packed tiles: row block a/16 starts at (a/16)*16*kbytes; lane's piece at +lane*16
    pa0 = We + (size_t)(a0 >> 4) * 16 * kbytes + lane * 16;
    pa1 = We + (size_t)(a1 >> 4) * 16 * kbytes + lane * 16;
}

// ---- small items (<= 16 rows): B fragments straight from L2 into registers
template <int KIND, bool G1>
BEAM_DEV void gemm_item_direct(const GemmParams& p, int e, int row0, int rows, int tile) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int krow = row_bytes<KIND>(G1 ? p.H : p.F);
    // K slice of this workgroup (the whole row unless GEMM2 is split)
    const int kslice = krow / p.ksplit;
    const int kbeg = (int)blockIdx.y * kslice, kbytes = kbeg + kslice;
    int a0, a1;
    const uint8_t *pa0, *pa1;
    weight_rows<KIND, G1>(p, e, tile, a0, a1, pa0, pa1);

    const bool bval = r < rows;
    int tok;
    const uint8_t* pb;
    if constexpr (G1) {
        tok = bval ? (p.identity_rows ? row0 + r : p.row_token[row0 + r]) : 0;
        pb = p.act + (size_t)tok * krow + 16 * g;
    } else {
        tok = row0 + r;
        pb = p.act + (size_t)(bval ? row0 + r : row0) * krow + 16 * g;
    }

    // MXFP4: E8M0 rows of the lane's two weight rows and its activation row;
    // a 256-byte K iteration covers 16 blocks = 16 scale bytes
    const uint8_t *psa0 = nullptr, *psa1 = nullptr, *psb = nullptr;
    if constexpr (KIND == W_MXFP4) {
        const int kblk = (G1 ? p.H : p.F) / 32;
        const size_t wrow0 = (size_t)e * (G1 ? 2 * p.F : p.H);
        psa0 = p.mx_w + (wrow0 + a0 + r) * kblk;
        psa1 = p.mx_w + (wrow0 + a1 + r) * kblk;
        psb = p.mx_act + (size_t)(G1 ? tok : (bval ? row0 + r : row0)) * kblk;
    }

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    uint4 wa0[2][4], wa1[2][4], xb[2][4];
    uint4 sa0[2], sa1[2], sb[2];
    auto load = [&](int buf, int k) {
        // k: byte offset along the row, a multiple of 256 (one packed tile)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            wa0[buf][s] = ld16_nt(pa0 + (size_t)k * 16 + 1024 * s);
            wa1[buf][s] = ld16_nt(pa1 + (size_t)k * 16 + 1024 * s);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) xb[buf][s] = bval ? ld16(pb + k + 64 * s) : make_uint4(0, 0, 0, 0);
        if constexpr (KIND == W_MXFP4) {
            sa0[buf] = ld16(psa0 + k / 16);
            sa1[buf] = ld16(psa1 + k / 16);
            sb[buf] = ld16(psb + k / 16);
        }
    };
    auto compute = [&](int buf) {
        if constexpr (KIND == W_MXFP4) {
            mfma_kiter_mx(wa0[buf], xb[buf], sa0[buf], sb[buf], acc0);
            mfma_kiter_mx(wa1[buf], xb[buf], sa1[buf], sb[buf], acc1);
        } else {
            mfma_kiter<KIND>(wa0[buf], xb[buf], acc0);
            mfma_kiter<KIND>(wa1[buf], xb[buf], acc1);
        }
    };

    // every pass of the loop prefetches unconditionally; the last one or two
    // K iterations are peeled off after it
    const int nkit = (kbytes - kbeg) / kKIterBytes;
    load(0, kbeg);
    int j = 0;
    for (; j + 2 < nkit; j += 2) {
        load(1, kbeg + (j + 1) * kKIterBytes);
        compute(0);
        load(0, kbeg + (j + 2) * kKIterBytes);
        compute(1);
    }
    if (j + 1 < nkit) {
        load(1, kbeg + (j + 1) * kKIterBytes);
        compute(0);
        compute(1);
    } else {
        compute(0);
    }
    if (!bval) return;
    if (p.ksplit > 1) {   // partial sums of this K slice to its own fp32 output
        if constexpr (G1) {   // raw gate (row a0 + 4g + i) and up (a1 + 4g + i) sums
            float* o = static_cast<float*>(p.out) + blockIdx.y * p.out_slice + (size_t)(row0 + r) * 2 * p.F;
            *reinterpret_cast<float4*>(o + a0 + 4 * g) = make_float4(acc0[0], acc0[1], acc0[2], acc0[3]);
            *reinterpret_cast<float4*>(o + a1 + 4 * g) = make_float4(acc1[0], acc1[1], acc1[2], acc1[3]);
        } else {
            GemmParams q = p;
            q.out = static_cast<float*>(p.out) + blockIdx.y * p.out_slice;
            store_block<KIND, G1>(q, e, a0, a1, (size_t)row0 + r, tok, acc0, acc1);
        }
        return;
    }
    store_block<KIND, G1>(p, e, a0, a1, (size_t)row0 + r, tok, acc0, acc1);
}

// ---- large items (<= kLdsRows rows): the item's activation rows are staged
// once per workgroup in LDS (double-buffered, 256 bytes of K per stage) and
// shared by the 4 waves; weights keep streaming into registers.
constexpr int kLdsRows = 128;
constexpr int kWideRows = 128;   // rows of a work item on the wide path
// rows of a 4-bit work item on the LDS path: eight 16-row blocks of E2M1
// operands (each MFMA takes them zero-padded to eight registers) do not fit
// in the registers of one wave
constexpr int kLdsRowsMx = 64;
constexpr int kLook = 3;         // wide path: LDS fragment reads issued this many groups ahead

// LDS position of 16-byte chunk c of staged row rr: chunks are XOR-swizzled
// with the row's low 4 bits so the 16 rows read by one MFMA fragment load
// hit 16 different bank groups.
BEAM_DEV int lds_pos(int rr, int c) { return rr * 16 + (c ^ (rr & 15)); }

template <int KIND, bool G1, int NB, bool NT>
BEAM_DEV void gemm_item_lds(const GemmParams& p, int e, int row0, int rows, int tile,
                            uint4 (*bs)[kLdsRows * 16], uint4 (*bss)[kLdsRows]) {
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int kbytes = row_bytes<KIND>(G1 ? p.H : p.F);
    const int nk = kbytes / kKIterBytes;
    int a0, a1;
    const uint8_t *pa0, *pa1;
    weight_rows<KIND, G1>(p, e, tile, a0, a1, pa0, pa1);

    // loader role: thread t copies chunk c = t % 16 of rows t/16 + 16 i
    const int lc = threadIdx.x & 15, lr = threadIdx.x >> 4;
    const uint8_t* src[NB];
    bool sval[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int rr = lr + 16 * i;
        sval[i] = rr < rows;
        size_t srow = row0;
        if (sval[i]) srow = G1 ? (size_t)p.row_token[row0 + rr] : (size_t)(row0 + rr);
        else if (G1) srow = 0;
        src[i] = p.act + srow * kbytes + 16 * lc;
    }
    uint4 stage[NB];
    // MXFP4: the staged rows' E8M0 codes (16 per 256-byte K iteration) go to
    // LDS too, copied by the chunk-0 thread of each row; the lane's weight
    // rows' codes stream into registers with the weights
    const uint8_t* ssrc[NB];
    uint4 sstage[NB];
    const uint8_t *psa0 = nullptr, *psa1 = nullptr;
    uint4 sa0[2], sa1[2];
    if constexpr (KIND == W_MXFP4) {
        const int kblk = (G1 ? p.H : p.F) / 32;
#pragma unroll
        for (int i = 0; i < NB; ++i) ssrc[i] = p.mx_act + (size_t)((src[i] - p.act) / kbytes) * kblk;
        const size_t wrow0 = (size_t)e * (G1 ? 2 * p.F : p.H);
        psa0 = p.mx_w + (wrow0 + a0 + r) * kblk;
        psa1 = p.mx_w + (wrow0 + a1 + r) * kblk;
    }
    auto gload = [&](int k) {
#pragma unroll
        for (int i = 0; i < NB; ++i) stage[i] = sval[i] ? ld16(src[i] + k) : make_uint4(0, 0, 0, 0);
        if constexpr (KIND == W_MXFP4) {
#pragma unroll
            for (int i = 0; i < NB; ++i)
                sstage[i] = (sval[i] && lc == 0) ? ld16(ssrc[i] + k / 16) : make_uint4(0, 0, 0, 0);
        }
    };
    auto swrite = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NB; ++i) bs[buf][lds_pos(lr + 16 * i, lc)] = stage[i];
        if constexpr (KIND == W_MXFP4) {
            if (lc == 0) {
#pragma unroll
                for (int i = 0; i < NB; ++i) bss[buf][lr + 16 * i] = sstage[i];
            }
        }
    };

    f32x4 acc0[NB], acc1[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        acc0[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    uint4 wa0[2][4], wa1[2][4];
    auto aload = [&](int buf, int k) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if constexpr (NT) {
                wa0[buf][s] = ld16_nt(pa0 + (size_t)k * 16 + 1024 * s);
                wa1[buf][s] = ld16_nt(pa1 + (size_t)k * 16 + 1024 * s);
            } else {
                wa0[buf][s] = ld16(pa0 + (size_t)k * 16 + 1024 * s);
                wa1[buf][s] = ld16(pa1 + (size_t)k * 16 + 1024 * s);
            }
        }
        if constexpr (KIND == W_MXFP4) {
            sa0[buf] = ld16(psa0 + k / 16);
            sa1[buf] = ld16(psa1 + k / 16);
        }
    };
    // one K step on LDS buffer CUR; with PREF it prefetches step kit+1 into
    // the other buffer.  The loop body always prefetches and the last one or
    // two steps are peeled off after it: a prefetch under a run-time
    // condition would make the compiler's wait counts cover both paths, so
    // the first MFMAs of a step would wait for the loads just issued.
    auto step = [&](auto curc, auto prefc, int kit) {
        constexpr int CUR = decltype(curc)::value;
        constexpr bool more = decltype(prefc)::value != 0;
        if constexpr (more) {
            gload((kit + 1) * kKIterBytes);
            aload(CUR ^ 1, (kit + 1) * kKIterBytes);
            // keep the prefetch at the top of the step (the scheduler would
            // otherwise sink the activation loads next to their LDS stores)
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            uint4 xb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) xb[s] = bs[CUR][lds_pos(nb * 16 + r, 4 * s + g)];
            if constexpr (KIND == W_MXFP4) {
                const uint4 sb = bss[CUR][nb * 16 + r];
                mfma_kiter_mx(wa0[CUR], xb, sa0[CUR], sb, acc0[nb]);
                mfma_kiter_mx(wa1[CUR], xb, sa1[CUR], sb, acc1[nb]);
            } else {
                mfma_kiter<KIND>(wa0[CUR], xb, acc0[nb]);
                mfma_kiter<KIND>(wa1[CUR], xb, acc1[nb]);
            }
        }
        if constexpr (more) swrite(CUR ^ 1);
        __syncthreads();
    };

    gload(0);
    aload(0, 0);
    swrite(0);
    __syncthreads();
    int kit = 0;
    for (; kit + 2 < nk; kit += 2) {
        step(IC<0>{}, IC<1>{}, kit);
        step(IC<1>{}, IC<1>{}, kit + 1);
    }
    if (kit + 1 < nk) {   // two steps left
        step(IC<0>{}, IC<1>{}, kit);
        step(IC<1>{}, IC<0>{}, kit + 1);
    } else {              // one step left
        step(IC<0>{}, IC<0>{}, kit);
    }

    if constexpr (KIND == W_FP8) {
        // every scale the row blocks need is loaded before the first store
        // (a store between them would make each block wait for its own)
        float sa[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int c = nb * 16 + r < rows ? nb * 16 + r : 0;
            sa[nb] = G1 ? p.act_scale[p.row_token[row0 + c]] : p.act_scale[row0 + c];
        }
        const size_t wrow0 = (size_t)e * (G1 ? 2 * p.F : p.H);
        const float4 sw0 = *reinterpret_cast<const float4*>(p.wscale + wrow0 + a0 + 4 * g);
        const float4 sw1 = *reinterpret_cast<const float4*>(p.wscale + wrow0 + a1 + 4 * g);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int c = nb * 16 + r;
            if (c < rows) {
                if constexpr (G1) {   // a1 = F + a0: the up rows of the gate rows a0
                    store_swiglu_s<KIND>(p, a0 + 4 * g, (size_t)row0 + c, sa[nb], sw0, sw1, acc0[nb], acc1[nb]);
                } else {
                    store_out_s<KIND>(p, a0 + 4 * g, (size_t)row0 + c, sa[nb], sw0, acc0[nb]);
                    store_out_s<KIND>(p, a1 + 4 * g, (size_t)row0 + c, sa[nb], sw1, acc1[nb]);
                }
            }
        }
    } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const int c = nb * 16 + r;
            if (c < rows) {
                const int tok = G1 ? p.row_token[row0 + c] : row0 + c;
                store_block<KIND, G1>(p, e, a0, a1, (size_t)row0 + c, tok, acc0[nb], acc1[nb]);
            }
        }
    }
}

// Item i of the direct path: the i-th expert, in expert order, that has
// rows (at T <= 16 an expert has at most T rows, so each touched expert is
// one item).  Every wave finds it in the offsets on its own, lane l looking
// at experts 4l .. 4l+3 (E <= 256), with one round trip to memory and no
// item list.  Returns false past the last touched expert.
BEAM_DEV bool direct_item(const int32_t* __restrict__ off, int E, int i, int& e, int& row0, int& rows) {
    const int lane = threadIdx.x & 63;
    int o[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
        const int x = 4 * lane + j;
        o[j] = off[x <= E ? x : E];
    }
    bool f[4];
    int before = 0, mine = 0, total = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[j] = 4 * lane + j < E && o[j + 1] > o[j];
        const unsigned long long b = __ballot(f[j]);
        // touched experts 4m + j of the lanes m below this one
        before += __builtin_amdgcn_mbcnt_hi((unsigned)(b >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)b, 0));
        mine += f[j] ? 1 : 0;
        total += __popcll(b);
    }
    if (i >= total) return false;
    // experts below 4l + j, in order: those of the lanes below (before) and
    // this lane's set flags j' < j
    int jj = 0, seen = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (f[j] && before + seen == i) jj = j;
        seen += f[j] ? 1 : 0;
    }
    const unsigned long long owner = __ballot(before <= i && i < before + mine);
    const int L = __ffsll(owner) - 1;   // the one lane holding expert number i
    int lo = o[0], hi = o[1];
#pragma unroll
    for (int j = 1; j < 4; ++j) {
        lo = jj == j ? o[j] : lo;
        hi = jj == j ? o[j + 1] : hi;
    }
    e = __builtin_amdgcn_readlane(4 * lane + jj, L);
    row0 = __builtin_amdgcn_readlane(lo, L);
    rows = __builtin_amdgcn_readlane(hi, L) - row0;
    return true;
}

template <int KIND, bool G1>
__global__ __launch_bounds__(256) void beam_expert_gemm_direct(GemmParams p) {
    const int item = blockIdx.x / p.n_tiles;
    const int tile = blockIdx.x - item * p.n_tiles;
    int e = 0, row0 = 0, rows = p.identity_rows;
    if (p.identity_rows) {
        if (item > 0) return;
    } else if (!direct_item(p.offsets, p.E, item, e, row0, rows)) {
        return;
    }
    gemm_item_direct<KIND, G1>(p, e, row0, rows, tile);
}

template <int KIND, bool G1, bool NT>
BEAM_DEV void dispatch_lds(const GemmParams& p, int4 it, int tile, uint4 (*bs)[kLdsRows * 16],
                           uint4 (*bss)[kLdsRows]) {
    if (it.z <= 16)
        gemm_item_lds<KIND, G1, 1, NT>(p, it.x, it.y, it.z, tile, bs, bss);
    else if (it.z <= 32)
        gemm_item_lds<KIND, G1, 2, NT>(p, it.x, it.y, it.z, tile, bs, bss);
    else if (KIND == W_MXFP4 || it.z <= 64)   // 4-bit items hold at most kLdsRowsMx rows
        gemm_item_lds<KIND, G1, 4, NT>(p, it.x, it.y, it.z, tile, bs, bss);
    else if constexpr (KIND != W_MXFP4)
        gemm_item_lds<KIND, G1, 8, NT>(p, it.x, it.y, it.z, tile, bs, bss);
}

// bf16: two waves per SIMD, so the 4-wave workgroups of two items overlap
// one another's load latency (fits in 256 registers without spills); the
// fp8 variant needs more registers and keeps one.
template <int KIND, bool G1>
__global__ __launch_bounds__(256, KIND == W_BF16 ? 2 : 1) void beam_expert_gemm_lds(GemmParams p) {
    __shared__ uint4 bs[2][kLdsRows * 16];
    __shared__ uint4 bss[2][KIND == W_MXFP4 ? kLdsRows : 1];   // MXFP4 activation scales
    const int item = blockIdx.x / p.n_tiles;
    const int tile = blockIdx.x - item * p.n_tiles;
    if (item >= *p.n_items) return;
    const int4 it = p.items[item];
    auto bssp = reinterpret_cast<uint4 (*)[kLdsRows]>(&bss[0][0]);
    // weights read once (single-item expert): non-temporal; shared by the
    // expert's other items: plain loads that stay in L2
    if ((it.w & 0xFFFF) == 1) dispatch_lds<KIND, G1, true>(p, it, tile, bs, bssp);
    else dispatch_lds<KIND, G1, false>(p, it, tile, bs, bssp);
}

// ---- wide tiles for large items: each wave owns FOUR 16-row weight tiles
// (GEMM1: 32 gate rows and the 32 matching up rows; GEMM2: 64 output rows),
// so a workgroup covers 256 weight rows x up to 128 item rows and every
// activation fragment read from LDS feeds four MFMAs instead of two.  The
// 4 x NB accumulator tiles live in registers (AGPRs), one wave per SIMD.
template <int KIND, bool G1>
BEAM_DEV void wide_rows(const GemmParams& p, int e, int tile, int (&a)[4], const uint8_t* (&pa)[4]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kbytes = row_bytes<KIND>(G1 ? p.H : p.F);
    const int nrows_w = G1 ? 2 * p.F : p.H;
    if constexpr (G1) {
        const int f0 = tile * 128 + wave * 32;
        a[0] = f0; a[1] = f0 + 16; a[2] = p.F + f0; a[3] = p.F + f0 + 16;
    } else {
        const int o0 = tile * 256 + wave * 64;
        a[0] = o0; a[1] = o0 + 16; a[2] = o0 + 32; a[3] = o0 + 48;
    }
    const uint8_t* We = p.W + (size_t)e * nrows_w * kbytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) pa[j] = We + (size_t)(a[j] >> 4) * 16 * kbytes + lane * 16;
}

// 32 bytes at p and p + 1024 (two pieces of a packed tile, or of an LDS
// row) as the 8-register operand of the fp8 MFMA
BEAM_DEV i32x8 pair8(uint4 lo, uint4 hi) {
    return __builtin_shufflevector(__builtin_bit_cast(i32x4v, lo), __builtin_bit_cast(i32x4v, hi), 0, 1, 2, 3,
                                   4, 5, 6, 7);
}

// One work unit of the wide path: N-tile `tile` of item `row0, rows` of
// expert e, which has cnt items.
struct WideUnit {
    int e, row0, rows, tile, cnt;
};

// Unit j in expert-major, N-tile, item order from the per-expert tables
// (first item in tab[0, E], first row in tab[E + 1, 2E + 1]); ecur only
// moves forward, as a workgroup's units do.
BEAM_DEV WideUnit wide_unit(const int* tab, int E, int nt, int j, int& ecur) {
    while (__builtin_amdgcn_readfirstlane(tab[ecur + 1]) * nt <= j) ++ecur;
    const int e = ecur;
    const int fi = __builtin_amdgcn_readfirstlane(tab[e]);
    const int cnt = __builtin_amdgcn_readfirstlane(tab[e + 1]) - fi;
    const int local = j - fi * nt;
    const int tile = local / cnt, ii = local - tile * cnt;
    const int row0 = __builtin_amdgcn_readfirstlane(tab[E + 1 + e]) + ii * kWideRows;
    const int rows = min(kWideRows, __builtin_amdgcn_readfirstlane(tab[E + 2 + e]) - row0);
    return {e, row0, rows, tile, cnt};
}

// Activation rows of the loader role (thread t copies chunk t % 16 of item
// rows t/16 + 16 i): GEMM1 gathers token rows, GEMM2 reads the item's rows.
// Padding rows of a partial item load a real row (the item's first): an
// output row depends only on its own input row, and padding rows are never
// stored.
template <bool G1>
BEAM_DEV void wide_srow(const GemmParams& p, const WideUnit& u, int (&srow)[8]) {
    const int lr = threadIdx.x >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int rr = lr + 16 * i < u.rows ? lr + 16 * i : 0;
        srow[i] = G1 ? p.row_token[u.row0 + rr] : u.row0 + rr;
    }
}

// `ahead` runs once the first K iteration is staged: loads issued there
// wait behind no load of this unit, and their results (this unit's fp8
// scales wsv and asv) are wanted only at its end.  `tail` runs after the
// last MFMA is issued, before the epilogue.
template <int KIND, bool G1, int NB, bool NT, typename Ahead, typename Tail>
BEAM_DEV void gemm_item_wide(const GemmParams& p, int e, int row0, int rows, int tile, const int (&srow)[8],
                             const float& wsv, const float& asv, uint4 (*bs)[kWideRows * 16], uint4* ssc,
                             float* scl, Ahead&& ahead, Tail&& tail) {
    constexpr bool MX = KIND == W_MXFP4;
    constexpr int NS = (KIND == W_FP8) ? 2 : 4;   // MFMA steps per 256-byte K iteration
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int kbytes = row_bytes<KIND>(G1 ? p.H : p.F);
    const int nk = kbytes / kKIterBytes;
    int a[4];
    const uint8_t* pa[4];
    wide_rows<KIND, G1>(p, e, tile, a, pa);

    // loader role: thread t copies chunk c = t % 16 of rows t/16 + 16 i
    const int lc = threadIdx.x & 15, lr = threadIdx.x >> 4;
    int sr[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if constexpr (MX) {   // gathered here: fewer registers live across the call
            const int rr = lr + 16 * i < rows ? lr + 16 * i : 0;
            sr[i] = G1 ? p.row_token[row0 + rr] : row0 + rr;
        } else {
            sr[i] = srow[i];
        }
    }
    const uint8_t* act = p.act + 16 * lc;
    // MXFP4: the E8M0 codes of the item's activation rows for the whole K
    // go to LDS once (row rr's 16 codes of K iteration c at ssc[16 rr + c]);
    // each weight row's 16 codes per K iteration stream with its weights
    const int kblk = (G1 ? p.H : p.F) / 32;
    const uint8_t* psw[4] = {nullptr, nullptr, nullptr, nullptr};
    if constexpr (MX) {
        // two threads per item row, each copying every other 16-code chunk
        // of the row's whole K (nk <= 16: K <= 8192): one row-map load, then
        // up to eight independent loads, all issued before the first LDS
        // store (a store next to its load would wait for it before the
        // next load goes out)
        const int rr = threadIdx.x >> 1, c0 = threadIdx.x & 1;
        const int src = rr < rows ? rr : 0;
        const size_t srow_mx = G1 ? (size_t)p.row_token[row0 + src] : (size_t)(row0 + src);
        const uint8_t* pmx = p.mx_act + srow_mx * kblk;
        uint4 sv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = c0 + 2 * i;
            sv[i] = c < nk ? ld16(pmx + c * 16) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = c0 + 2 * i;
            if (c < nk) ssc[rr * 16 + c] = sv[i];
        }
        const size_t wrow0 = (size_t)e * (G1 ? 2 * p.F : p.H);
#pragma unroll
        for (int j = 0; j < 4; ++j) psw[j] = p.mx_w + (wrow0 + a[j] + r) * kblk;
    }
    uint4 stage[NB];
    auto gload = [&](int k) {
#pragma unroll
        for (int i = 0; i < NB; ++i) stage[i] = ld16(act + (size_t)sr[i] * kbytes + k);
    };
    auto swrite = [&](int buf) {
#pragma unroll
        for (int i = 0; i < NB; ++i) bs[buf][lds_pos(lr + 16 * i, lc)] = stage[i];
    };
    auto wload = [&](int j, int q, int k) -> uint4 {
        if constexpr (NT) return ld16_nt(pa[j] + (size_t)k * 16 + 1024 * q);
        else return ld16(pa[j] + (size_t)k * 16 + 1024 * q);
    };

    f32x4 acc[4][NB];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[j][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // One set of weight fragments, one register group per MFMA step; the
    // group of step st is reloaded for the next K iteration as soon as the
    // step's last MFMA has issued (one iteration of latency to hide).
    using WFrag = typename std::conditional<KIND == W_FP8, i32x8, uint4>::type;
    WFrag wa[4][NS];
    uint4 sw[4];   // MXFP4: the lane's weight rows' 16 E8M0 codes of the K iteration
    auto aload_step = [&](int st, int k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (KIND == W_FP8) wa[j][st] = pair8(wload(j, 2 * st, k), wload(j, 2 * st + 1, k));
            else wa[j][st] = wload(j, st, k);
        }
        if constexpr (MX) {   // after the iteration's last step: the next iteration's codes
            if (st == NS - 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) sw[j] = ld16(psw[j] + k / 16);
            }
        }
    };
    // B fragment q of a K iteration (q = st * NB + nb): the 16 rows of row
    // block nb for MFMA step st, from the staged LDS tile (MXFP4: with the
    // row's E8M0 word of the step)
    struct MxB {
        uint4 v;
        uint32_t s;
    };
    using BFrag = typename std::conditional<MX, MxB, WFrag>::type;
    auto bload = [&](const uint4* b, int q, int kit) -> BFrag {
        const int st = q / NB, nb = q % NB;
        if constexpr (MX)
            return MxB{b[lds_pos(nb * 16 + r, 4 * st + g)],
                       reinterpret_cast<const uint32_t*>(ssc)[((nb * 16 + r) * 16 + kit) * 4 + st]};
        else if constexpr (KIND == W_BF16)
            return b[lds_pos(nb * 16 + r, 4 * st + g)];
        else
            return pair8(b[lds_pos(nb * 16 + r, 4 * (2 * st) + g)], b[lds_pos(nb * 16 + r, 4 * (2 * st + 1) + g)]);
    };
    gload(0);
#pragma unroll
    for (int st = 0; st < NS; ++st) aload_step(st, 0);
    if constexpr (MX) {
#pragma unroll
        for (int j = 0; j < 4; ++j) sw[j] = ld16(psw[j]);
    }
    swrite(0);
    __syncthreads();
    ahead();
    // One straight-line body per LDS buffer, the pair unrolled in the loop
    // (no runtime buffer index).  The NS * NB fragment groups of an iteration run
    // as one sequence with the LDS reads kLook groups ahead of their MFMAs
    // (one wave per SIMD: nothing else hides the LDS latency), and the
    // weight registers of step st are reloaded right after the step's last
    // MFMA; with no branches in the body the scheduling barriers keep that
    // order.  The last iteration reloads its own K slice (in bounds, never
    // used).
    constexpr int NQ = NS * NB;
    constexpr int kReadsPerFrag = KIND == W_BF16 ? 1 : 2;   // LDS reads per B fragment
    // instruction classes of the scheduling-group hints
    constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;
    // fp8 fragments are twice as wide: two groups ahead leave the registers
    // for the four-iteration loop pass
    constexpr int kLookKind = KIND == W_FP8 ? 2 : kLook;
    constexpr int LOOK = kLookKind < NQ ? kLookKind : NQ;
    auto body = [&](auto curc, int kit) {
        constexpr int cur = decltype(curc)::value;
        const int knext = (kit + 1 < nk ? kit + 1 : kit) * kKIterBytes;
        gload(knext);
        const uint4* bcur = bs[cur];
        BFrag xq[LOOK];
#pragma unroll
        for (int d = 0; d < LOOK; ++d) xq[d] = bload(bcur, d, kit);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, LOOK * kReadsPerFrag, 0);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int st = q / NB, nb = q % NB;
            const BFrag xb = xq[q % LOOK];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (MX) {
                    // formats 4/4 = E2M1 x E2M1 (the low 4 dwords of each
                    // operand); lane (r, g) takes byte g of the step's words
                    const uint32_t wsw = st == 0 ? sw[j].x : st == 1 ? sw[j].y : st == 2 ? sw[j].z : sw[j].w;
                    const int sh = 8 * g;
                    const i32x8 av = {(int)wa[j][st].x, (int)wa[j][st].y, (int)wa[j][st].z, (int)wa[j][st].w,
                                      0, 0, 0, 0};
                    const i32x8 bv = {(int)xb.v.x, (int)xb.v.y, (int)xb.v.z, (int)xb.v.w, 0, 0, 0, 0};
                    acc[j][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        av, bv, acc[j][nb], 4, 4, 0, (int)((wsw >> sh) & 0xFF), 0, (int)((xb.s >> sh) & 0xFF));
                } else if constexpr (KIND == W_BF16)
                    acc[j][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, wa[j][st]), __builtin_bit_cast(bf16x8, xb), acc[j][nb], 0, 0, 0);
                else   // formats 0/0 = e4m3 x e4m3; block scales 127 = 2^0 (unscaled)
                    acc[j][nb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wa[j][st], xb, acc[j][nb],
                                                                                  0, 0, 0, 127, 0, 127);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
            if (q + LOOK < NQ) {
                xq[q % LOOK] = bload(bcur, q + LOOK, kit);
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReadsPerFrag, 0);
            }
            if (nb == NB - 1) {
                __builtin_amdgcn_sched_barrier(0);
                aload_step(st, knext);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        swrite(cur ^ 1);
        __syncthreads();
    };
    // eight iterations per loop pass: the register shuffle the compiler puts
    // at the loop head (about 0.6 moves per MFMA with a pair per pass) is
    // paid once per eight; then fours, pairs and a last one
    int kit = 0;
    for (; kit + 7 < nk; kit += 8) {
        body(IC<0>{}, kit);
        body(IC<1>{}, kit + 1);
        body(IC<0>{}, kit + 2);
        body(IC<1>{}, kit + 3);
        body(IC<0>{}, kit + 4);
        body(IC<1>{}, kit + 5);
        body(IC<0>{}, kit + 6);
        body(IC<1>{}, kit + 7);
    }
    for (; kit + 3 < nk; kit += 4) {
        body(IC<0>{}, kit);
        body(IC<1>{}, kit + 1);
        body(IC<0>{}, kit + 2);
        body(IC<1>{}, kit + 3);
    }
    for (; kit + 1 < nk; kit += 2) {
        body(IC<0>{}, kit);
        body(IC<1>{}, kit + 1);
    }
    if (kit < nk) body(IC<0>{}, kit);   // odd K-iteration count: the last one
    tail();

    // fp8: the scales of the tile's 256 weight rows and of the item's rows,
    // loaded before the K loop, go through LDS to the lanes that need them
    if constexpr (KIND == W_FP8) {
        scl[threadIdx.x] = wsv;
        if (lc < 8) scl[256 + lr + 16 * lc] = asv;
        __syncthreads();
    }
    // the lane's weight rows a[j] + 4 g as positions among the tile's 256
    const int wave = threadIdx.x >> 6;
    int lw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) lw[j] = G1 ? (j >= 2 ? 128 : 0) + 32 * wave + 16 * (j & 1) : 64 * wave + 16 * j;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int c = nb * 16 + r;
        if (c < rows) {
            const size_t row = (size_t)row0 + c;
            float sx = 1.f;
            float4 sw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) sw[j] = make_float4(1.f, 1.f, 1.f, 1.f);
            if constexpr (KIND == W_FP8) {
                sx = scl[256 + c];
#pragma unroll
                for (int j = 0; j < 4; ++j) sw[j] = *reinterpret_cast<const float4*>(scl + lw[j] + 4 * g);
            }
            if constexpr (G1) {
                store_swiglu_s<KIND>(p, a[0] + 4 * g, row, sx, sw[0], sw[2], acc[0][nb], acc[2][nb]);
                store_swiglu_s<KIND>(p, a[1] + 4 * g, row, sx, sw[1], sw[3], acc[1][nb], acc[3][nb]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) store_out_s<KIND>(p, a[j] + 4 * g, row, sx, sw[j], acc[j][nb]);
            }
        }
    }
}

template <int KIND, bool G1, bool NT, typename Ahead, typename Tail>
BEAM_DEV void dispatch_wide(const GemmParams& p, const WideUnit& u, const int (&srow)[8], const float& wsv,
                            const float& asv, uint4 (*bs)[kWideRows * 16], uint4* ssc, float* scl, Ahead&& ahead,
                            Tail&& tail) {
    if (u.rows <= 32)
        gemm_item_wide<KIND, G1, 2, NT>(p, u.e, u.row0, u.rows, u.tile, srow, wsv, asv, bs, ssc, scl, ahead, tail);
    else if (u.rows <= 64)
        gemm_item_wide<KIND, G1, 4, NT>(p, u.e, u.row0, u.rows, u.tile, srow, wsv, asv, bs, ssc, scl, ahead, tail);
    else
        gemm_item_wide<KIND, G1, 8, NT>(p, u.e, u.row0, u.rows, u.tile, srow, wsv, asv, bs, ssc, scl, ahead, tail);
}

// Persistent: one workgroup per CU.  Work units are ordered expert by
// expert, N-tile by N-tile, item by item, so the items of one expert that
// share an N-tile of weights are neighbours.  Workgroups go to the 8 XCDs
// round-robin (block b runs on XCD b % 8), so each XCD is given one
// contiguous range of units, which its workgroups take in order from a
// counter of their own: neighbours run together, share the XCD's L2, and
// each weight tile is fetched about once for all the items of its expert;
// a workgroup that draws short units draws more of them.  A unit's position
// is computed from two per-expert tables held in LDS (no memory round
// trip), and its fp8 epilogue scales are loaded behind its first K stage.
// Every unit is computed whole by one workgroup, so the result does not
// depend on which workgroup takes it.
template <int KIND, bool G1>
__global__ __launch_bounds__(256, 1) void beam_expert_gemm_wide(GemmParams p) {
    __shared__ uint4 bs[2][kWideRows * 16];
    // MXFP4: the activation rows' E8M0 codes for the whole K (16 per K iteration)
    __shared__ uint4 ssc[KIND == W_MXFP4 ? kWideRows * 16 : 1];
    // fp8: scales of the tile's 256 weight rows, then of the item's 128 rows
    __shared__ __align__(16) float scl[KIND == W_FP8 ? 384 : 4];
    __shared__ int tab[2 * (kMaxExperts + 1)];
    __shared__ int nxt[1];
    const int E = p.E, nt = p.n_tiles;
    if constexpr (KIND == W_MXFP4) {
        // no registers to spare for a unit loop: one unit per workgroup, and
        // the item gathers its own rows
        const int total = *p.n_items * nt;
        const int per_xcd = (total + 7) >> 3;
        const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
        if (slot >= per_xcd) return;
        const int j = xcd * per_xcd + slot;
        if (j >= total) return;
        const int4 any = p.items[j / nt];             // an item of the unit's expert
        const int cnt = any.w & 0xFFFF;
        const int first = j / nt - (any.w >> 16);     // the expert's first item
        const int local = j - first * nt;             // = tile * cnt + item within the expert
        const int tile = local / cnt;
        const int4 it = p.items[first + (local - tile * cnt)];
        const WideUnit u{it.x, it.y, it.z, tile, cnt};
        const int srow[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        const float one = 1.f;
        auto none = [] {};
        if (cnt == 1) dispatch_wide<KIND, G1, true>(p, u, srow, one, one, bs, ssc, scl, none, none);
        else dispatch_wide<KIND, G1, false>(p, u, srow, one, one, bs, ssc, scl, none, none);
        return;
    }
    for (int i = threadIdx.x; i <= E; i += 256) {
        tab[i] = p.first_item[i];
        tab[E + 1 + i] = p.offsets[i];
    }
    __syncthreads();
    const int total = __builtin_amdgcn_readfirstlane(tab[E]) * nt;
    const int per_xcd = (total + 7) >> 3;
    const int xcd = blockIdx.x & 7;
    const int base = xcd * per_xcd, end = min(total, base + per_xcd);
    // the XCD's units are handed out in order by its counter; a workgroup
    // asks for its next unit when its last MFMA of this one has issued, so
    // the answer comes back during the epilogue, and the units running on
    // the XCD stay neighbours
    int* ctr = p.unit_ctr + xcd;
    if (threadIdx.x == 0) nxt[0] = atomicAdd(ctr, 1);
    __syncthreads();
    int j = base + nxt[0];
    if (j >= end) return;
    const int lc = threadIdx.x & 15;
    int ecur = 0;
    WideUnit u = wide_unit(tab, E, nt, j, ecur);
    int srow[8];
    wide_srow<G1>(p, u, srow);
    for (;;) {
        int fut = 0;
        float wsv = 1.f, asv = 1.f;
        auto ahead = [&] {
            if constexpr (KIND == W_FP8) {
                const int t = threadIdx.x;
                const size_t wr = G1 ? (size_t)u.e * 2 * p.F + (t < 128 ? 0 : p.F) + u.tile * 128 + (t & 127)
                                     : (size_t)u.e * p.H + u.tile * 256 + t;
                wsv = p.wscale[wr];
                int sr = srow[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) sr = (lc & 7) == i ? srow[i] : sr;
                if (lc < 8) asv = p.act_scale[sr];
            }
        };
        auto tail = [&] {
            if (threadIdx.x == 0) fut = atomicAdd(ctr, 1);
        };
        // weights read once (single-item expert): non-temporal; shared by the
        // expert's other items: plain loads that stay in L2
        if (u.cnt == 1) dispatch_wide<KIND, G1, true>(p, u, srow, wsv, asv, bs, ssc, scl, ahead, tail);
        else dispatch_wide<KIND, G1, false>(p, u, srow, wsv, asv, bs, ssc, scl, ahead, tail);
        // nxt was last read before this unit's K loop, whose barriers every
        // wave has passed since
        if (threadIdx.x == 0) nxt[0] = fut;
        __syncthreads();
        j = base + nxt[0];
        if (j >= end) break;
        u = wide_unit(tab, E, nt, j, ecur);
        wide_srow<G1>(p, u, srow);
    }
}

// Per-row e4m3 re-quantisation of the fp32 SwiGLU output (fp8 path): one
// wave per row, four rows per workgroup.
template <int NIT>
__global__ __launch_bounds__(256) void beam_quantize_a_e4m3(const float* __restrict__ a,
                                                            const int32_t* __restrict__ offsets, int E,
                                                            int F, uint8_t* __restrict__ aq,
                                                            float* __restrict__ ascale) {
    const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (size_t)offsets[E]) return;   // whole wave exits together
    const float* ar = a + row * F;
    auto load_raw = [&](int i) { return *reinterpret_cast<const float4*>(ar + i); };
    auto widen = [](float4 f) { return f; };
    quantize_row_e4m3_wave<NIT>(load_raw, widen, F, aq + row * F, ascale + row);
}

// SwiGLU of K-split GEMM1 sums: a[r][f] = bf16(silu(sum_s g) * sum_s v), the
// slices added in order (deterministic); g = parts[s][r][f], v = parts[s][r][F + f].
__global__ __launch_bounds__(256) void beam_swiglu_slices(const float* __restrict__ parts, int S, int rows,
                                                          int F, uint16_t* __restrict__ a) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;   // element of a, F % 4 == 0
    if (i >= (size_t)rows * F) return;
    const size_t r = i / F, f = i - r * F;
    const size_t stride = (size_t)rows * 2 * F;
    const float* pg = parts + r * 2 * F + f;
    float4 gs = *reinterpret_cast<const float4*>(pg);
    float4 vs = *reinterpret_cast<const float4*>(pg + F);
    for (int s = 1; s < S; ++s) {
        const float4 gv = *reinterpret_cast<const float4*>(pg + s * stride);
        const float4 uv = *reinterpret_cast<const float4*>(pg + s * stride + F);
        gs.x += gv.x; gs.y += gv.y; gs.z += gv.z; gs.w += gv.w;
        vs.x += uv.x; vs.y += uv.y; vs.z += uv.z; vs.w += uv.w;
    }
    const uint32_t lo = pack_bf16x2(silu_f32(gs.x) * vs.x, silu_f32(gs.y) * vs.y);
    const uint32_t hi = pack_bf16x2(silu_f32(gs.z) * vs.z, silu_f32(gs.w) * vs.w);
    *reinterpret_cast<uint2*>(a + i) = make_uint2(lo, hi);
}

// ---------------------------------------------------------------- fp32 path
// One workgroup per permuted row; plain fp32 FMA dot products.

BEAM_DEV int expert_of_row(const int32_t* offsets, int E, int row) {
    int lo = 0, hi = E;   // largest e with offsets[e] <= row
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= row) lo = mid; else hi = mid;
    }
    return lo;
}

__global__ __launch_bounds__(256) void beam_expert_f32_gemm1(
    const float* __restrict__ x, const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_token,
    const float* __restrict__ wgu, int E, int H, int F, float* __restrict__ a) {
    const int row = blockIdx.x;
    if (row >= offsets[E]) return;
    const int e = expert_of_row(offsets, E, row);
    const float* xr = x + (size_t)row_token[row] * H;
    for (int j = threadIdx.x; j < F; j += blockDim.x) {
        const float* wg = wgu + ((size_t)e * 2 * F + j) * H;
        const float* wu = wgu + ((size_t)e * 2 * F + F + j) * H;
        float gs = 0.f, us = 0.f;
        for (int i = 0; i < H; ++i) {
            gs = fmaf(xr[i], wg[i], gs);
            us = fmaf(xr[i], wu[i], us);
        }
        a[(size_t)row * F + j] = (gs / (1.0f + expf(-gs))) * us;
    }
}

__global__ __launch_bounds__(256) void beam_expert_f32_gemm2(
    const float* __restrict__ a, const int32_t* __restrict__ offsets, const float* __restrict__ wd,
    int E, int H, int F, void* __restrict__ y, bool y_bf16) {
    const int row = blockIdx.x;
    if (row >= offsets[E]) return;
    const int e = expert_of_row(offsets, E, row);
    const float* ar = a + (size_t)row * F;
    for (int o = threadIdx.x; o < H; o += blockDim.x) {
        const float* w = wd + ((size_t)e * H + o) * F;
        float s = 0.f;
        for (int j = 0; j < F; ++j) s = fmaf(ar[j], w[j], s);
        if (y_bf16)
            static_cast<uint16_t*>(y)[(size_t)row * H + o] = f32_to_bf16(s);
        else
            static_cast<float*>(y)[(size_t)row * H + o] = s;
    }
}

// ---------------------------------------------------------------- host side

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Kernel choice by the mean rows per expert, T*K/E:
//   T <= 16:   one 16-row item per touched expert, weights straight into
//              registers (beam_expert_gemm_direct), so weights are read
//              exactly once;
//   < 256:     mostly one 128-row item per expert, so each weight byte is
//              streamed once: two 16-row weight tiles per wave, two waves
//              per SIMD for more bytes in flight (beam_expert_gemm_lds);
//   >= 256:    128-row items, several per expert, sharing each weight tile
//              through L2: four weight tiles per wave, XCD-grouped work
//              order, one persistent workgroup per CU
//              (beam_expert_gemm_wide).
enum GemmPath { PATH_DIRECT, PATH_LDS, PATH_WIDE };

bool experts_direct_path(int T) { return T <= 16; }

static GemmPath gemm_path(int T, int K, int E) {
    if (experts_direct_path(T)) return PATH_DIRECT;
    return (long long)T * K >= 256LL * E ? PATH_WIDE : PATH_LDS;
}

static int rows_per_item(int T, int K, int E, WKind w) {
    switch (gemm_path(T, K, E)) {
        case PATH_DIRECT: return 16;
        case PATH_LDS: return w == W_MXFP4 ? kLdsRowsMx : kLdsRows;
        default: return kWideRows;
    }
}

static size_t max_items(int T, int K, int E, WKind w) {
    const size_t TK = (size_t)T * K;
    return TK / rows_per_item(T, K, E, w) + (size_t)std::min<size_t>(E, TK);
}

struct ExpertsWs {
    int* n_items;
    int* unit_ctr;     // 16 counters: GEMM1's 8, then GEMM2's
    int* first_item;   // [E + 1]: first item of each expert, then the item count
    int4* items;
    void* a;        // bf16 [TK,F] (BF16) or fp32 [TK,F] (FP8, MXFP4, F32)
    uint8_t* aq;    // FP8: e4m3 [TK,F]; MXFP4: packed E2M1 [TK,F/2]
    float* ascale;  // FP8: [TK]
    uint8_t* amx;   // MXFP4: E8M0 [TK,F/32]
    size_t bytes;
};

static ExpertsWs carve(void* base, int T, int K, int E, int F, WKind w) {
    const size_t TK = (size_t)T * K;
    ExpertsWs s{};
    uint8_t* p = static_cast<uint8_t*>(base);
    size_t off = 0;
    s.n_items = reinterpret_cast<int*>(p + off);
    s.unit_ctr = s.n_items + 16;
    off += 256;
    s.first_item = reinterpret_cast<int*>(p + off);
    off += align256((size_t)(E + 1) * sizeof(int));
    s.items = reinterpret_cast<int4*>(p + off);
    off += align256(max_items(T, K, E, w) * sizeof(int4));
    s.a = p + off;
    off += align256(TK * F * (w == W_BF16 ? 2 : 4));
    if (w == W_FP8) {
        s.aq = p + off;
        off += align256(TK * F);
        s.ascale = reinterpret_cast<float*>(p + off);
        off += align256(TK * sizeof(float));
    }
    if (w == W_MXFP4) {
        s.aq = p + off;
        off += align256(TK * F / 2);
        s.amx = p + off;
        off += align256(TK * F / 32);
    }
    s.bytes = off;
    return s;
}

size_t experts_ws_bytes(int T, int K, int E, int H, int F, WKind w) {
    (void)H;
    return carve(nullptr, T, K, E, F, w).bytes;
}


// compute units of the current device (looked up once per device; calls
// from several host threads may look it up concurrently, harmlessly)
static int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int KIND, bool G1>
static void launch_gemm(GemmParams p, int n_items_max, GemmPath path, hipStream_t st) {
    const int H = p.H, F = p.F;
    if (path == PATH_WIDE) {
        p.n_tiles = G1 ? F / 128 : H / 256;
        // one workgroup per CU, the same number on each XCD (MXFP4: one
        // workgroup per unit)
        const int per_xcd = (n_items_max * p.n_tiles + 7) / 8;
        const int slots = KIND == W_MXFP4 ? per_xcd : std::max(1, std::min(per_xcd, device_cus() / 8));
        hipLaunchKernelGGL((beam_expert_gemm_wide<KIND, G1>), dim3(8 * slots), dim3(256), 0, st, p);
        return;
    }
    p.n_tiles = G1 ? F / 64 : H / 128;
    if (path == PATH_DIRECT)
        hipLaunchKernelGGL((beam_expert_gemm_direct<KIND, G1>), dim3(n_items_max * p.n_tiles, p.ksplit),
                           dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((beam_expert_gemm_lds<KIND, G1>), dim3(n_items_max * p.n_tiles), dim3(256), 0, st, p);
}

hipError_t launch_experts(const ExpertsArgs& a, hipStream_t st) {
    const int TK = a.T * a.K;
    ExpertsWs ws = carve(a.ws, a.T, a.K, a.E, a.F, a.w);
    if (a.w == W_F32) {
        hipLaunchKernelGGL(beam_expert_f32_gemm1, dim3(TK), dim3(256), 0, st, (const float*)a.x,
                           a.offsets, a.row_token, (const float*)a.wgu, a.E, a.H, a.F, (float*)ws.a);
        hipLaunchKernelGGL(beam_expert_f32_gemm2, dim3(TK), dim3(256), 0, st, (const float*)ws.a,
                           a.offsets, (const float*)a.wd, a.E, a.H, a.F, a.y, a.y_bf16);
        return hipGetLastError();
    }
    const int mc = rows_per_item(a.T, a.K, a.E, a.w);
    const int n_items_max = (int)max_items(a.T, a.K, a.E, a.w);
    const GemmPath path = gemm_path(a.T, a.K, a.E);
    // the direct kernels find their items in the offsets themselves
    if (path != PATH_DIRECT)
        hipLaunchKernelGGL(beam_build_items, dim3(1), dim3(256), 0, st, a.offsets, a.E, mc, ws.items,
                           ws.n_items, ws.first_item, ws.unit_ctr);

    GemmParams p{};
    p.items = ws.items;
    p.n_items = ws.n_items;
    p.first_item = ws.first_item;
    p.offsets = a.offsets;
    p.E = a.E;
    p.unit_ctr = ws.unit_ctr;
    p.identity_rows = (a.identity_rows && path == PATH_DIRECT) ? a.T : 0;
    p.H = a.H;
    p.F = a.F;
    p.ksplit = 1;

    // GEMM1 + SwiGLU
    p.act = static_cast<const uint8_t*>(a.x);
    p.row_token = a.row_token;
    p.act_scale = static_cast<const float*>(a.xscale);
    p.W = static_cast<const uint8_t*>(a.wgu);
    p.wscale = static_cast<const float*>(a.sgu);
    p.out = ws.a;
    p.out_bf16 = false;
    if (a.w == W_MXFP4) {
        p.act_scale = nullptr;
        p.wscale = nullptr;
        p.mx_act = static_cast<const uint8_t*>(a.xscale);
        p.mx_w = static_cast<const uint8_t*>(a.sgu);
        launch_gemm<W_MXFP4, true>(p, n_items_max, path, st);
    } else if (a.w == W_BF16) {
        if (path == PATH_DIRECT && a.ksplit1 > 1) {   // raw sums per K slice, then SwiGLU
            p.ksplit = a.ksplit1;
            p.out = a.g1_parts;
            p.out_slice = (size_t)TK * 2 * a.F;
            launch_gemm<W_BF16, true>(p, n_items_max, path, st);
            hipLaunchKernelGGL(beam_swiglu_slices, dim3((unsigned)(((size_t)TK * a.F / 4 + 255) / 256)), dim3(256),
                               0, st, a.g1_parts, a.ksplit1, TK, a.F, static_cast<uint16_t*>(ws.a));
            p.ksplit = 1;
        } else {
            launch_gemm<W_BF16, true>(p, n_items_max, path, st);
        }
    } else {
        launch_gemm<W_FP8, true>(p, n_items_max, path, st);
    }

    // GEMM2 (split over K on the direct kernel when the caller asks)
    if (path == PATH_DIRECT && a.ksplit > 1) {
        p.ksplit = a.ksplit;
        p.out_slice = a.y_slice_stride;
    }
    p.row_token = nullptr;
    p.unit_ctr = ws.unit_ctr + 8;
    p.W = static_cast<const uint8_t*>(a.wd);
    p.wscale = static_cast<const float*>(a.sd);
    p.out = a.y;
    p.out_bf16 = a.y_bf16;
    if (a.w == W_MXFP4) {
        // the fp32 SwiGLU output, quantised per 32-block of its row
        hipError_t err = launch_quantize_mx(ws.a, false, TK, a.F, a.offsets + a.E, ws.aq, ws.amx, st);
        if (err != hipSuccess) return err;
        p.act = ws.aq;
        p.wscale = nullptr;
        p.mx_act = ws.amx;
        p.mx_w = static_cast<const uint8_t*>(a.sd);
        launch_gemm<W_MXFP4, false>(p, n_items_max, path, st);
    } else if (a.w == W_FP8) {
        const dim3 qgrid((TK + 3) / 4);
        const float* af = static_cast<const float*>(ws.a);
        if (a.F <= 1024)
            hipLaunchKernelGGL(beam_quantize_a_e4m3<4>, qgrid, dim3(256), 0, st, af, a.offsets, a.E, a.F, ws.aq,
                               ws.ascale);
        else if (a.F <= 2048)
            hipLaunchKernelGGL(beam_quantize_a_e4m3<8>, qgrid, dim3(256), 0, st, af, a.offsets, a.E, a.F, ws.aq,
                               ws.ascale);
        else if (a.F <= 2560)   // the Beam d_ff
            hipLaunchKernelGGL(beam_quantize_a_e4m3<10>, qgrid, dim3(256), 0, st, af, a.offsets, a.E, a.F, ws.aq,
                               ws.ascale);
        else if (a.F <= 4096)
            hipLaunchKernelGGL(beam_quantize_a_e4m3<16>, qgrid, dim3(256), 0, st, af, a.offsets, a.E, a.F, ws.aq,
                               ws.ascale);
        else
            hipLaunchKernelGGL(beam_quantize_a_e4m3<32>, qgrid, dim3(256), 0, st, af, a.offsets, a.E, a.F, ws.aq,
                               ws.ascale);
        p.act = ws.aq;
        p.act_scale = ws.ascale;
        launch_gemm<W_FP8, false>(p, n_items_max, path, st);
    } else {
        p.act = static_cast<const uint8_t*>(ws.a);
        p.act_scale = nullptr;
        launch_gemm<W_BF16, false>(p, n_items_max, path, st);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- dense layer helpers

__global__ __launch_bounds__(256) void beam_sum_slices(const float* __restrict__ parts, int S, size_t n,
                                                       float* __restrict__ y) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;                              // n % 4 == 0
    float4 acc = *reinterpret_cast<const float4*>(parts + i);
    for (int s = 1; s < S; ++s) {                    // fixed order: deterministic
        const float4 v = *reinterpret_cast<const float4*>(parts + (size_t)s * n + i);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<float4*>(y + i) = acc;
}

__global__ __launch_bounds__(256) void beam_dense_rows(int T, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ row_token) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < T) row_token[i] = i;
    if (i == 0) {
        offsets[0] = 0;
        offsets[1] = T;
    }
}

hipError_t launch_sum_slices(const float* parts, int S, size_t n, float* y, hipStream_t st) {
    const size_t blocks = (n / 4 + 255) / 256;
    hipLaunchKernelGGL(beam_sum_slices, dim3((unsigned)blocks), dim3(256), 0, st, parts, S, n, y);
    return hipGetLastError();
}

hipError_t launch_dense_rows(int T, int32_t* offsets, int32_t* row_token, hipStream_t st) {
    hipLaunchKernelGGL(beam_dense_rows, dim3((T + 255) / 256), dim3(256), 0, st, T, offsets, row_token);
    return hipGetLastError();
}

}  // namespace beam
