/*
 * beam_moe.h -- C ABI of one Beam-style mixture-of-experts layer forward on
 * an AMD Instinct MI355X (gfx950).
 *
 * The layer (TokenSpeed x Reflection Beam blog, section "Architecture";
 * vLLM Beam summary, MoE and residual section):
 *   route        FP32 router projection, sigmoid scores + per-expert
 *                correction bias, group-limited top-k (4 of 8 groups, then
 *                8 experts), renormalised weights times the routed scale 2.5
 *   permute      stable expert-major grouping of the (token, slot) pairs,
 *                plus optional dynamic per-token e4m3 quantisation of x
 *   experts      grouped SwiGLU MLP per expert (GEMM1 + SwiGLU, GEMM2) in
 *                bf16, fp8-e4m3 (per-channel weight scales, per-token
 *                activation scales) or fp32
 *   combine_norm weighted combine of the K expert outputs, post-RMSNorm,
 *                depth-scaled residual h <- sqrt((n-1)/n) h + p / sqrt(n),
 *                next pre-RMSNorm
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major, densely packed,
 *     owned by the caller.  The library never allocates, frees, copies to
 *     the host or synchronises; every call only enqueues kernels on
 *     `stream` (a hipStream_t; NULL = the default stream) and returns.
 *   - `cfg` is a host pointer, read during the call only.
 *   - Arguments are validated before anything is enqueued: an invalid call
 *     returns a non-zero status and enqueues nothing.  T == 0 returns
 *     BEAM_OK and enqueues nothing.  A failed launch returns BEAM_ERR_HIP.
 *   - `ws` is a caller-owned device workspace of at least
 *     beam_moe_workspace_bytes(cfg, T, w_dtype) bytes.  One workspace may be
 *     shared by the calls of one layer on one stream; calls that overlap in
 *     time must not share one.
 *   - Calls on one stream are ordered; the library keeps no state between
 *     calls (other than each device's compute-unit count, looked up once),
 *     so calls on different streams or threads are independent.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum beam_status {
    BEAM_OK = 0,
    BEAM_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad dtype     */
    BEAM_ERR_UNSUPPORTED = 2,   /* shape the kernels are not built for        */
    BEAM_ERR_WORKSPACE = 3,     /* ws missing or smaller than required         */
    BEAM_ERR_HIP = 4            /* a kernel launch failed                      */
} beam_status;

typedef enum beam_dtype {
    BEAM_F32 = 0,
    BEAM_BF16 = 1,
    BEAM_FP8_E4M3 = 2,          /* OCP E4M3FN codes (uint8), max 448, no inf  */
    BEAM_MXFP4 = 3              /* OCP MXFP4: E2M1 codes packed two per byte  */
                                /* (element 2i in the low nibble of byte i),  */
                                /* with one E8M0 scale code (uint8, value     */
                                /* 2^(code-127)) per 32 consecutive elements  */
                                /* of a row, stored row-major [rows, K/32]    */
} beam_dtype;

/* Layer shape.  Beam: {5120, 256, 8, 4, 8, 2, 2560, 2.5f, 1e-6f}. */
typedef struct beam_moe_cfg {
    int32_t hidden;        /* H: multiple of 256 (512 for MXFP4), at most 8192 */
    int32_t n_experts;     /* E: at most 256                                  */
    int32_t n_groups;      /* G: E % G == 0; experts [g*E/G, (g+1)*E/G) form group g */
    int32_t topk_groups;   /* groups kept per token, 1..G                     */
    int32_t topk;          /* K experts per token, 1..min(32, topk_groups*E/G)*/
    int32_t group_topn;    /* biased scores summed per group score, 1..min(4, E/G) */
    int32_t d_ff;          /* F: multiple of 128 (256 fp8, 512 MXFP4 experts)  */
    float routed_scale;    /* routing weights sum to this (2.5)               */
    float rms_eps;         /* RMSNorm epsilon (1e-6)                           */
} beam_moe_cfg;

/*
 * beam_moe_route -- router projection, scores, group-limited top-k, weights.
 * (TokenSpeed blog, "Fused FP32 routing": bf16 activations times fp32 router
 *  weights with fp32 accumulation and logits, then sigmoid, bias,
 *  group top-k and the 2.5 scale folded into the weights.)
 *
 *   x          [T,H] activations, dtype x_dtype (BF16 or F32)
 *   w_router   [E,H] fp32; row e produces expert e's logit
 *   bias       [E]   fp32 correction bias (used for selection only)
 *   topk_ids   [T,K] int32 out: chosen experts, descending biased score
 *                    s+bias, ties to the lower expert index
 *   topk_w     [T,K] fp32 out: routed_scale * s_k / sum_j s_j over the K
 *                    chosen experts (s = sigmoid(logit), unbiased)
 *   logits_out [T,E] fp32 out, nullable: the router logits
 *   ws         required (partial logits), see beam_moe_workspace_bytes
 * Group score = sum of the group_topn largest biased scores of the group;
 * the topk_groups best groups are kept (ties: lower group index).
 * For T > 16 with bf16 x the logits run on matrix cores through the exact
 * three-way bf16 split of the fp32 router weights (TokenSpeed blog, "Fused
 * FP32 routing": Tensor Core path for large batches); products are exact
 * and accumulation is fp32 in every path.
 */
beam_status beam_moe_route(const beam_moe_cfg* cfg, int32_t T,
                           const void* x, beam_dtype x_dtype,
                           const float* w_router, const float* bias,
                           int32_t* topk_ids, float* topk_w, float* logits_out,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * beam_moe_permute -- group the T*K (token, slot) pairs by expert.
 * (vLLM Beam summary, kernel list: the MoE path's routing kernels that
 *  group tokens by expert; TokenSpeed blog, "TensorRT-LLM NVFP4 MoE": input
 *  quantisation does not depend on the routes.)
 *
 *   topk_ids        [T,K] int32 in (values in [0,E); pair p = t*K + k)
 *   expert_offsets  [E+1] int32 out: exclusive prefix sum of per-expert
 *                   pair counts (expert_offsets[E] = T*K when every id is valid)
 *   row_token       [T*K] int32 out: permuted row r -> token t
 *   pair_row        [T*K] int32 out: pair p -> permuted row r
 *   Within one expert, rows follow ascending p (stable, unique).
 *   x, x_dtype      [T,H] BF16 activations, read only when x_q != NULL
 *   x_q             [T,H] uint8 out, nullable: e4m3 codes of x / x_scale[t]
 *                   (round to nearest even, saturating at 448)
 *   x_scale         [T] fp32 out (required with x_q): amax(|x[t]|) / 448,
 *                   1 for an all-zero row
 * Ids outside [0,E) are a caller error; such pairs are dropped: they get no
 * row, pair_row[p] = -1 for them (beam_moe_combine_norm skips such entries)
 * and expert_offsets[E] counts only the valid pairs, so no access ever
 * leaves the buffers.
 *   ws              required when T*K > 4096 (per-chunk histograms), 16-byte
 *                   aligned; see beam_moe_workspace_bytes
 */
beam_status beam_moe_permute(const beam_moe_cfg* cfg, int32_t T,
                             const int32_t* topk_ids,
                             int32_t* expert_offsets, int32_t* row_token, int32_t* pair_row,
                             const void* x, beam_dtype x_dtype,
                             uint8_t* x_q, float* x_scale,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * beam_moe_quantize_fp8 -- dynamic per-token e4m3 quantisation of the layer
 * input for the FP8 experts, the same codes and scales beam_moe_permute
 * writes when given x_q.  (Gaudi cookbook, "What was built": dynamic
 * per-token activation scales; TokenSpeed blog, "TensorRT-LLM NVFP4 MoE":
 * the input quantisation does not depend on the routes, so it may run on a
 * second stream of the same priority alongside the router.)
 *
 *   x        [T,H] BF16
 *   x_q      [T,H] out: e4m3 codes, round to nearest even, saturating at
 *            +-448; 16-byte aligned
 *   x_scale  [T] out: amax/448 of the row in fp32 (1 for an all-zero row)
 * T = 0 is a no-op.  NaN elements do not enter the row maximum and get the
 * e4m3 NaN code; a row holding +-Inf gets an infinite scale, code 0 for its
 * finite elements and the NaN code for the infinite ones (no fault, no
 * hang).
 */
beam_status beam_moe_quantize_fp8(const beam_moe_cfg* cfg, int32_t T, const void* x, beam_dtype x_dtype,
                                  uint8_t* x_q, float* x_scale, void* stream);

/*
 * beam_moe_quantize_mx -- run-time MXFP4 quantisation of the layer input for
 * the 4-bit experts.  (TokenSpeed blog, "TensorRT-LLM NVFP4 MoE": the 4-bit
 * MoE quantises its input at run time, a step independent of the routes
 * that may run on a second stream alongside the router; OCP Microscaling
 * Formats (MX) v1.0: shared exponent floor(log2(amax)) - 2 per block of 32,
 * elements rounded to the nearest E2M1 value, ties to even, saturating.)
 *
 *   x        [T,H] BF16 or F32 (x_dtype)
 *   x_q      [T,H/2] out: E2M1 codes, element 2i in the low nibble of byte i
 *   x_scale  [T,H/32] out: E8M0 scale codes; block b covers elements
 *            [32b, 32b+32) of its row; an all-zero block gets code 0
 * Requires hidden % 512 == 0.  E2M1 has no NaN or infinity: NaN and +-Inf
 * elements are stored as +-6, and a block holding +-Inf gets some in-range
 * scale code (no fault, no hang; the token's routing weights still carry
 * the NaN of its router logits).
 */
beam_status beam_moe_quantize_mx(const beam_moe_cfg* cfg, int32_t T, const void* x, beam_dtype x_dtype,
                                 uint8_t* x_q, uint8_t* x_scale, void* stream);

/*
 * beam_moe_experts -- grouped SwiGLU expert MLP over the permuted rows.
 * (TokenSpeed blog, "TensorRT-LLM NVFP4 MoE": GEMM1 with SwiGLU fused,
 *  then GEMM2; Gaudi cookbook, "What was built" and "EP vs TP quality":
 *  per-channel FP8 weights, dynamic per-token activations, the
 *  down-projection input quantised per token over the whole d_ff.)
 *
 * For permuted row r (expert e, token t = row_token[r]):
 *   g = x[t] W_gu[e][0:F]^T,  v = x[t] W_gu[e][F:2F]^T,  a = silu(g) * v,
 *   y[r] = a W_down[e]^T
 *   w_dtype   F32: x F32, a kept fp32.   BF16: x BF16, a rounded to bf16.
 *             FP8_E4M3: x is the e4m3 codes x_q with per-token x_scale from
 *             beam_moe_permute; weights are e4m3 codes with per-output-row
 *             fp32 scales; a is re-quantised per row over all F columns
 *             (scale amax/448) before GEMM2.
 *             MXFP4: the 4-bit experts (TokenSpeed blog, "NVFP4 and FP8
 *             checkpoints": 4-bit E2M1 expert weights with block scales,
 *             re-encoded here as OCP MXFP4); x is x_q / x_scale from
 *             beam_moe_quantize_mx; the fp32 SwiGLU output a is quantised
 *             the same way (32-element blocks) before GEMM2; all products on
 *             the scaled FP4 x FP4 matrix cores, fp32 accumulation.
 *             Requires hidden and d_ff multiples of 512.
 *   x         [T,H] dtype per w_dtype (x_dtype must be F32, BF16, FP8_E4M3
 *             or MXFP4 to match; MXFP4: [T,H/2] bytes); x_scale: FP8 [T]
 *             fp32, MXFP4 [T,H/32] E8M0 codes, else unused
 *   expert_offsets [E+1], row_token [T*K] from beam_moe_permute
 *   w_gate_up [E,2F,H]: rows [0,F) gate, [F,2F) up; s_gate_up FP8 [E,2F]
 *             fp32, MXFP4 [E,2F,H/32] E8M0 codes
 *   w_down    [E,H,F]; s_down FP8 [E,H] fp32, MXFP4 [E,H,F/32] E8M0 codes
 *             Both weight stacks must be the output of beam_moe_pack_weights
 *             (same size, tiled layout); the scales stay row-major.
 *   y         [T*K,H] out, dtype y_dtype (F32 or BF16): unweighted expert
 *             outputs in permuted row order
 */
beam_status beam_moe_experts(const beam_moe_cfg* cfg, int32_t T, beam_dtype w_dtype,
                             const void* x, beam_dtype x_dtype, const void* x_scale,
                             const int32_t* expert_offsets, const int32_t* row_token,
                             const void* w_gate_up, const void* s_gate_up,
                             const void* w_down, const void* s_down,
                             void* y, beam_dtype y_dtype,
                             void* ws, size_t ws_bytes, void* stream);

/* Bytes of the per-GPU device array beam_moe_experts_static works in. */
#define BEAM_MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * beam_moe_experts_static -- beam_moe_experts without a caller workspace,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).
 *
 * Arguments, layouts and results are those of beam_moe_experts minus
 * ws / ws_bytes; it launches the same kernels.  Its workspace is a
 * file-scope device array of BEAM_MOE_STATIC_SCRATCH_BYTES (64 MiB) that
 * every GPU the library runs on holds until the process ends; the first
 * call on a device looks up that device's copy (no allocation by this
 * library, no host synchronisation).  Nothing in it has to start at zero:
 * each call writes every part of it that it reads.
 *   - Returns BEAM_ERR_UNSUPPORTED, enqueuing nothing, when the experts
 *     step needs more workspace than that (at the Beam shape: more than
 *     about 1,600 tokens with bf16 experts, about 540 with fp8 experts).
 *   - All calls on one GPU share the array: calls that overlap in time on
 *     one GPU (different streams, threads or graphs running concurrently)
 *     race and corrupt each other's results.  Calls ordered on one stream
 *     are safe.
 */
beam_status beam_moe_experts_static(const beam_moe_cfg* cfg, int32_t T, beam_dtype w_dtype,
                                    const void* x, beam_dtype x_dtype, const void* x_scale,
                                    const int32_t* expert_offsets, const int32_t* row_token,
                                    const void* w_gate_up, const void* s_gate_up,
                                    const void* w_down, const void* s_down,
                                    void* y, beam_dtype y_dtype, void* stream);

/*
 * beam_moe_combine_norm -- weighted combine + sandwich-norm boundary.
 * (TokenSpeed blog, "MNNVL all-reduce and SandwichNorm fusion": post-norm,
 *  depth-scaled residual and next pre-norm in one kernel; vLLM Beam
 *  summary, kernel change 3: the same kernel combines the top-8 expert
 *  outputs; MoE and residual section: h <- sqrt((n-1)/n) h + x / sqrt(n).)
 *
 * Per token t:
 *   m      = sum_k topk_w[t,k] * y[pair_row[t*K+k]]            (fp32)
 *   p      = round(m / sqrt(mean(m^2) + eps) * gamma_post)
 *   h'     = round(sqrt((n-1)/n) * h[t] + p / sqrt(n))          -> h[t] (in place)
 *   x_next = round(h' / sqrt(mean(h'^2) + eps) * gamma_pre)
 * where round() is to act_dtype (BF16, or F32 = no rounding beyond fp32).
 *   y [T*K,H] dtype y_dtype (F32|BF16); pair_row [T*K]; topk_w [T,K] fp32
 *   h, x_next [T,H] act_dtype; gamma_post, gamma_pre [H] act_dtype
 *   n        residual index >= 1 (n = 1 gives h' = p)
 *   moe_out  [T,H] fp32 out, nullable: m
 * h and x_next must not overlap.
 */
beam_status beam_moe_combine_norm(const beam_moe_cfg* cfg, int32_t T,
                                  const void* y, beam_dtype y_dtype,
                                  const int32_t* pair_row, const float* topk_w,
                                  void* h, void* x_next, beam_dtype act_dtype,
                                  const void* gamma_post, const void* gamma_pre,
                                  int32_t n, float* moe_out, void* stream);

/*
 * beam_moe_norm_boundary -- the sandwich-norm boundary on a given m: the
 * same post-RMSNorm, depth-scaled residual and next pre-RMSNorm as
 * beam_moe_combine_norm, with m supplied by the caller instead of combined
 * from expert rows.  For a dense layer's MLP output, and for the sum of the
 * expert-parallel shards' partial outputs after the all-reduce.
 * (TokenSpeed blog, "Architecture": a norm before and after every block;
 *  "Tensor parallelism and expert parallelism": under EP8 the
 *  normalisation runs separately from the all-reduce.)
 *   m      [T,H] F32 or BF16 (m_dtype); h, x_next, gammas, n as in
 *          beam_moe_combine_norm (h updated in place, must not alias x_next)
 */
beam_status beam_moe_norm_boundary(const beam_moe_cfg* cfg, int32_t T, const void* m, beam_dtype m_dtype,
                                   void* h, void* x_next, beam_dtype act_dtype,
                                   const void* gamma_post, const void* gamma_pre, int32_t n, void* stream);

/*
 * beam_moe_permute_shard -- beam_moe_permute restricted to one
 * expert-parallel shard: the pairs whose expert lies in
 * [expert_begin, expert_begin + n_local) are grouped by local expert
 * (id - expert_begin) in the same stable order; every other pair gets
 * pair_row[p] = -1.  (TokenSpeed blog, "Tensor parallelism and expert
 * parallelism": with EP8 each GPU holds 32 complete experts and processes
 * the tokens routed to them; Gaudi cookbook, "At a glance": EP 8, 32
 * experts per card -- exactly one routing group.)
 *   expert_offsets [n_local+1], row_token [T*K] (the first
 *   expert_offsets[n_local] entries used), pair_row [T*K]
 *   ws              required when T*K > 4096, 16-byte aligned; at most the
 *                   size beam_moe_workspace_bytes gives for the full layer
 * The shard's experts then run through beam_moe_experts with a cfg whose
 * n_experts is n_local and the shard's slices of the weight stacks.
 */
beam_status beam_moe_permute_shard(const beam_moe_cfg* cfg, int32_t T, int32_t expert_begin, int32_t n_local,
                                   const int32_t* topk_ids, int32_t* expert_offsets, int32_t* row_token,
                                   int32_t* pair_row, void* ws, size_t ws_bytes, void* stream);

/*
 * beam_moe_combine_partial -- one shard's share of the weighted combine:
 *   m_out[t] = sum over k with pair_row[t*K+k] >= 0 of topk_w[t,k] * y[pair_row[t*K+k]]
 * (fp32, no norm).  The shards' m_out summed over all shards (the
 * all-reduce) equal the layer's m.  (TokenSpeed blog, "Tensor parallelism
 * and expert parallelism": the all-reduce sums the MoE output, no
 * all-to-all.)
 *   y [T*K,H] F32|BF16, pair_row [T*K] from beam_moe_permute_shard,
 *   topk_w [T,K], m_out [T,H] fp32 out
 */
beam_status beam_moe_combine_partial(const beam_moe_cfg* cfg, int32_t T, const void* y, beam_dtype y_dtype,
                                     const int32_t* pair_row, const float* topk_w, float* m_out, void* stream);

/*
 * beam_moe_dense_mlp -- the SwiGLU MLP of a dense layer over all T tokens:
 *   y[t] = (silu(x[t] W_gu[0:d_ff]^T) * x[t] W_gu[d_ff:2 d_ff]^T) W_down^T
 * with the SwiGLU output rounded to bf16, fp32 accumulation, y fp32 (the
 * expert GEMMs with one "expert" holding every row).  (vLLM Beam summary,
 * MoE section: layers 0-2 use a dense SwiGLU MLP with d_ff 20480 instead of
 * the MoE; TokenSpeed blog, "Architecture": the first 3 layers are dense.)
 *   d_ff      multiple of 128, at most 32768 (cfg->d_ff is not used)
 *   x         [T,H] BF16
 *   w_gate_up [2 d_ff, H] bf16, w_down [H, d_ff] bf16, both packed by
 *             beam_moe_pack_weights (a cfg with this d_ff, n_experts 1)
 *   y         [T,H] fp32 out
 *   ws        beam_moe_dense_workspace_bytes(cfg, T, d_ff) bytes, 16-byte
 *             aligned; at T <= 16 both projections are split over K and
 *             the slices are summed in a fixed order (deterministic; the
 *             gate and up sums before SwiGLU is applied)
 */
beam_status beam_moe_dense_mlp(const beam_moe_cfg* cfg, int32_t T, int32_t d_ff, const void* x,
                               beam_dtype x_dtype, const void* w_gate_up, const void* w_down, float* y,
                               void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of beam_moe_dense_mlp for T tokens (0 for invalid input). */
size_t beam_moe_dense_workspace_bytes(const beam_moe_cfg* cfg, int32_t T, int32_t d_ff);

/*
 * beam_moe_pack_weights -- one-time re-layout of expert weight stacks into
 * the tiled order beam_moe_experts streams from (load time, not per layer
 * call).  Each expert matrix of R rows x KB bytes is cut into 16-row x
 * 256-byte tiles stored as [piece s][lane r+16g][16 bytes], lane (r, g)
 * holding bytes [64s+16g, +16) of row r; the tiles of a 16-row block follow
 * each other along the row.  Sizes are unchanged.  For F32 stacks the
 * packed layout is the plain row-major one (a copy).
 *
 *   n_experts       number of expert matrices in each stack (may be a
 *                   subset of cfg->n_experts, to pack expert by expert);
 *                   cfg->d_ff may be up to 32768 here (the dense layers)
 *   w_gate_up       [n_experts,2F,H] row-major in; w_down [n_experts,H,F]
 *                   (MXFP4: the packed E2M1 bytes, K/2 per row; the E8M0
 *                   scales are not re-laid out)
 *   packed_gate_up, packed_down: outputs of the same byte sizes; they must
 *                   not overlap the inputs or each other.
 * (Layout choice for MI355X HBM: every weight load instruction of the
 *  expert GEMM then reads whole 128-byte lines of one contiguous KiB.)
 */
beam_status beam_moe_pack_weights(const beam_moe_cfg* cfg, int32_t n_experts, beam_dtype w_dtype,
                                  const void* w_gate_up, const void* w_down,
                                  void* packed_gate_up, void* packed_down, void* stream);

/* Workspace bytes that route, permute and experts need for T tokens with
 * experts of w_dtype (the maximum over the three).  0 for invalid input. */
size_t beam_moe_workspace_bytes(const beam_moe_cfg* cfg, int32_t T, beam_dtype w_dtype);

/* Static, human-readable name of a status code. */
const char* beam_moe_status_string(beam_status status);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
