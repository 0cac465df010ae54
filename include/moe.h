/*
 * moe.h -- C ABI of one sparse Mixture-of-Experts FFN layer on AMD MI355X
 * (gfx950).  Built as routing_expert_ffn_amd/libmoe.so.
 *
 * The layer (cited by page title and section):
 *   router logits   l = x W_r^T (+ logit_bias)            "MoE架构揭秘：大模型参数激活率与专家路由机制解析", 3.1
 *   scoring         softmax over E logits                 same section
 *                   or sigmoid + selection-only bias      "15. DeepSeek：MLA、MoE 与 MTP", "V3 的 MoE：256 个专家怎样选 8 个"
 *                   or sqrt(softplus) + selection bias    same page, "V4：放弃潜向量，改用压缩注意力" (FFN paragraph)
 *   hash routing    experts fixed by a token-id table     same V4 paragraph (moe_route_hash, moe_forward_hash)
 *   group limit     groups of E/G experts scored by the sum of their two best
 *                   biased scores, topk_group groups kept  same DeepSeek section
 *   top-k + gates   renormalised softmax ("GPT-4 Has 1.8 Trillion Parameters.
 *                   It Uses 2% of Them Per Token", MoEBlock sketch in 4.1),
 *                   plain softmax (DeepSeek-V2, no renormalisation), or
 *                   unbiased sigmoid scores renormalised x routed_scaling_factor
 *   capacity        an expert takes at most C tokens; later tokens go to their
 *                   next-best allowed expert ("GPT-4 Has 1.8 Trillion ...", 2.2)
 *   experts         SwiGLU FFN y = W_down (silu(W_gate x) * W_up x), shared
 *                   experts always active and added unweighted
 *                   ("MoE on KnightLi的博客", activation functions; DeepSeek page,
 *                   "671B 和 37B 的参数账")
 *   combine         out = sum_j w_j * expert_{idx_j}(x) + sum_s shared_s(x)
 *   FP8 experts     E4M3 matrices, UE8M0 scales per 128 x 128 weight block and
 *                   per 1 x 128 activation tile   DeepSeek page, "FP8 训练是训练配方，不是架构"
 *
 * Conventions shared by every call
 *  - Every pointer argument that names a tensor is a DEVICE pointer on the
 *    current HIP device, owned by the caller, row-major and densely packed.
 *    The library allocates no device memory and keeps no device state.
 *  - "Input dtype" (moe_config.dtype) applies to x and every weight matrix:
 *    MOE_BF16 (bfloat16) or MOE_F32; MOE_FP8 layers take bf16 x and router
 *    weight and E4M3 expert matrices with block scales (moe_forward_fp8).
 *    Logits, gates and biases are fp32.
 *  - Matrices keep their reduction dimension contiguous: w_router [E,H],
 *    w_gate/w_up [E+S,I,H], w_down [E+S,H,I]; routed experts 0..E-1 first,
 *    shared experts E..E+S-1 after them.
 *  - Row space of the experts: routed rows 0..T*k-1 ordered by (expert asc,
 *    token asc), shared expert s of token t at row T*k + s*T + t.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and never synchronises the host.
 *  - Workspace: `ws` is a device buffer of at least moe_workspace_size() bytes,
 *    256-byte aligned, owned by the caller, not used concurrently by two calls.
 *  - Errors: arguments are validated before anything is enqueued; on failure
 *    the call returns a negative moe_status, enqueues nothing and records a
 *    message for moe_last_error().  A failed kernel launch returns
 *    MOE_ERR_HIP.  Faults inside kernels surface asynchronously (at the
 *    caller's next synchronisation).  T == 0 is a successful no-op.
 *  - Size limit of the expert FFN (moe_forward*, moe_expert_ffn*): for bf16
 *    and FP8 layers x must hold fewer than 2^31 bytes (T * H * 2 for bf16,
 *    T * H E4M3 codes for FP8), else MOE_ERR_UNSUPPORTED: the gate/up GEMM
 *    gathers token rows through one 32-bit buffer resource.  Split larger
 *    batches.
 *  - Routing is reproducible bit for bit: selection works on fp32 values with
 *    ties broken by the lower index, and sigmoid selection scores use the fp32
 *    sigmoid built from correctly rounded operations that moe_route documents.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* bad pointer, size or configuration            */
  MOE_ERR_UNSUPPORTED = -2, /* valid layer this build does not run          */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  MOE_ERR_HIP = -4          /* a HIP runtime call failed                    */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1, MOE_SCORE_SQRTSOFTPLUS = 2 } moe_scoring;
/* MOE_FP8: x and the router weight are bf16; the expert matrices are E4M3
 * codes with one UE8M0 scale per 128 x 128 block (moe_forward_fp8,
 * moe_expert_ffn_fp8). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8 = 2 } moe_dtype;

/* Layer description: the fields the DeepSeek page reads from a checkpoint's
 * config (n_routed_experts, n_shared_experts, num_experts_per_tok, n_group,
 * topk_group, moe_intermediate_size, routed_scaling_factor, scoring
 * function) plus the capacity factor of the capacity passage and the
 * drop_tokens switch of the GPT-4 page's serving configuration. */
typedef struct moe_config {
  int32_t hidden_size;           /* H; bf16 needs H % 256 == 0, f32 H % 32 == 0 */
  int32_t n_routed_experts;      /* E, 1..512                                     */
  int32_t n_shared_experts;      /* S, 0..64, each shaped like a routed expert   */
  int32_t top_k;                 /* k, 1..min(E, 32)                              */
  int32_t n_group;               /* G >= 1, E % G == 0, E/G >= 2 when G > 1      */
  int32_t topk_group;            /* 1..G, top_k <= topk_group * E / G            */
  int32_t moe_intermediate_size; /* I; bf16 needs I % 128 == 0, f32 I % 32 == 0 */
  int32_t scoring;               /* moe_scoring                                   */
  int32_t norm_topk_prob;        /* 1: gates renormalised over the selection     */
  float routed_scaling_factor;   /* multiplies every routed gate (2.5 for V3)    */
  double capacity_factor;        /* <= 0: unlimited; else C = ceil(((cf*T)*k)/E)
                                    evaluated in IEEE double, left to right      */
  int32_t dtype;                 /* moe_dtype of x and every weight (MOE_FP8: see
                                    moe_dtype)                                    */
  int32_t out_dtype;             /* moe_dtype of `out`                            */
  int32_t drop_tokens;           /* with a capacity: 1 = drop the overflow, 0 =
                                    re-route it to the next-best allowed expert */
} moe_config;

/* Bytes of workspace every call below needs for this layer and T tokens
 * (the largest need of any call; one buffer serves them all).
 * Returns MOE_ERR_INVALID_ARG for an invalid configuration or T < 0. */
moe_status moe_workspace_size(const moe_config* cfg, int64_t T, size_t* bytes);

/* Router: logits, scoring, group-limited top-k, gates, optional capacity.
 *   x            [T,H] input dtype (unused when logits_in is given)
 *   w_router     [E,H] input dtype (unused when logits_in is given)
 *   logit_bias   [E] fp32 added to every logit, or NULL
 *   sel_bias     [E] fp32 selection-only bias (sigmoid and sqrt(softplus)
 *                scoring), or NULL
 *   logits_in    [T,E] fp32 logits to route instead of computing them, or NULL
 *   logits_out   [T,E] fp32 computed logits (bias included), or NULL
 *   topk_idx     [T,k] int32 out: chosen experts in rank order, -1 = empty slot
 *   topk_w       [T,k] fp32 out: gates (0 for an empty slot)
 *   expert_counts[E] int32 out: tokens per expert, or NULL
 * Selection score: softmax scoring ranks the fp32 logits; sigmoid scoring
 * ranks c_e = fl32(sigmoid32(l_e) + sel_bias_e) and sqrt(softplus) scoring
 * c_e = fl32(sqrtsoftplus32(l_e) + sel_bias_e), where sigmoid32 clamps l to
 * [-80,80] and evaluates 1/(1+e) (l >= 0, e = exp32(-l)) or e/(1+e) (l < 0,
 * e = exp32(l)); exp32(z) = ldexp(p(r), n), n = rint(fl32(z*0x1.715476p+0)),
 * r = fma(-n, 0x1.7f7d1cp-20, fma(-n, 0x1.62e4p-1, z)), p = Horner with fma of
 * the fp32 coefficients {1, 1, 0x1p-1, 0x1.555556p-3, 0x1.555556p-5,
 * 0x1.111112p-7, 0x1.6c16c2p-10, 0x1.a01a02p-13}; sqrtsoftplus32(l) =
 * sqrt(fl32(max(l,0) + log1p32(exp32(-min(|l|,80))))) with the correctly
 * rounded square root, log1p32(u) = fl32(fl32(z+z) * q), z = u/fl32(2+u),
 * q = Horner with fma in w = fl32(z*z) of the fp32 coefficients {1,
 * 0x1.555556p-2, 0x1.99999ap-3, 0x1.24924ap-3, 0x1.c71c72p-4, 0x1.745d18p-4,
 * 0x1.3b13b2p-4, 0x1.111112p-4} (1/(2j+1)).  Gates of sigmoid and
 * sqrt(softplus) scoring use the unbiased score.  Group score = fl32(best +
 * second best) of a group's c.  Ties rank the lower index first.
 * Capacity: tokens in index order each take their best-ranked allowed experts
 * with fewer than C tokens so far; C = ceil(((cf*T)*k)/E) in double.  With
 * drop_tokens (the serving configuration of "GPT-4 Has 1.8 Trillion
 * Parameters ...", section 4.2) each token keeps its top-k and their gates,
 * and in token order an assignment whose expert already holds C tokens is
 * dropped (index -1, gate 0) instead of going to another expert.
 * Workspace: required (MOE_ERR_WORKSPACE otherwise) with a capacity limit and
 * for bf16 layers that compute their logits; fp32 layers and logits_in
 * routing without a capacity limit may pass ws = NULL. */
moe_status moe_route(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                     const float* logit_bias, const float* sel_bias, const float* logits_in,
                     float* logits_out, int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                     void* ws, size_t ws_bytes, void* stream);

/* Hash routing ("15. DeepSeek：MLA、MoE 与 MTP", section "V4：放弃潜向量，改用压缩注意力",
 * FFN paragraph: in its first layers a fixed table keyed by the token id picks
 * the experts and the router only weights them).  Arguments as moe_route,
 * plus
 *   token_ids    [T] int32 device: id of every token
 *   tid2eid      [vocab,k] int32 device: experts of every id, in slot order
 *                (NULL allowed only when vocab == 0)
 *   vocab        rows of tid2eid, >= 0
 * Slot j of token t takes e = tid2eid[token_ids[t], j]; a token id outside
 * [0, vocab) takes no expert; an entry outside [0, E) or equal to an earlier
 * entry of its row leaves its slot empty (-1, gate 0).  The gates are those
 * of cfg's scoring over the chosen experts (the logits are still computed;
 * sel_bias does not apply).  A capacity limit needs drop_tokens = 1 (there
 * is no next-best expert to re-route to; MOE_ERR_INVALID_ARG otherwise).
 * Workspace: required for bf16 layers that compute their logits. */
moe_status moe_route_hash(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                          const float* logit_bias, const float* logits_in, float* logits_out, const int32_t* token_ids,
                          const int32_t* tid2eid, int64_t vocab, int32_t* topk_idx, float* topk_w,
                          int32_t* expert_counts, void* ws, size_t ws_bytes, void* stream);

/* Dispatch: expert histogram and stable permutation of (token, slot) pairs
 * ("MoE架构揭秘：大模型参数激活率与专家路由机制解析", section 4.1: the tokens of
 * each expert are gathered together rather than masked per expert; "GPT-4 Has
 * 1.8 Trillion Parameters. It Uses 2% of Them Per Token", section 4.2: the
 * router's output is packed with the token ids into one routing batch that a
 * single kernel dispatches to the experts).
 *   topk_idx       [T,k] int32, each row distinct experts in [0,E) or -1
 *   expert_counts  [E]   int32 out
 *   expert_offsets [E+1] int32 out: exclusive prefix sum of the counts
 *   row_token      [T*k + S*T] int32 out: token of every row (-1 = unused row)
 *   slot_row       [T,k] int32 out: row of (t, j), -1 for an empty slot
 * Rows of one expert are in ascending token order.  Out-of-range indices are
 * the caller's contract violation: they are counted nowhere (undefined rows).
 * T == 0: expert_counts and expert_offsets are set to zero (no rows). */
moe_status moe_permute(const moe_config* cfg, int64_t T, const int32_t* topk_idx, int32_t* expert_counts,
                       int32_t* expert_offsets, int32_t* row_token, int32_t* slot_row, void* ws,
                       size_t ws_bytes, void* stream);

/* Experts: for every routed row r (expert e, token t = row_token[r]) and every
 * shared row, y_rows[r] = W_down[e] (silu(W_gate[e] x_t) * W_up[e] x_t).
 *   x              [T,H] input dtype
 *   w_gate, w_up   [E+S,I,H] input dtype;  w_down [E+S,H,I] input dtype
 *   expert_offsets [E+1], row_token [T*k+S*T] as written by moe_permute
 *   y_rows         [T*k+S*T, H] fp32 out; unused routed rows are left untouched
 * bf16 layers accumulate in fp32 on the matrix cores and round the SwiGLU
 * activation h to bf16 (the input of the down projection); expert outputs
 * stay fp32 so the combine adds unrounded values. */
moe_status moe_expert_ffn(const moe_config* cfg, int64_t T, const void* x, const void* w_gate,
                          const void* w_up, const void* w_down, const int32_t* expert_offsets,
                          const int32_t* row_token, void* y_rows, void* ws, size_t ws_bytes, void* stream);

/* Combine ("15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家怎样选
 * 8 个", last line of its router code block: the layer output is the
 * gate-weighted sum of the chosen experts' outputs plus the shared expert's):
 * out[t] = sum_j topk_w[t,j] * y_rows[slot_row[t,j]] (empty slots
 * skipped) + sum_s y_rows[T*k + s*T + t], accumulated in fp32 in that order.
 *   y_rows [T*k+S*T, H] fp32; slot_row, topk_w [T,k]; out [T,H] out_dtype */
moe_status moe_combine(const moe_config* cfg, int64_t T, const void* y_rows, const int32_t* slot_row,
                       const float* topk_w, void* out, void* stream);

/* The whole layer in one call: route, permute, experts and combine (the
 * layer of "15. DeepSeek：MLA、MoE 与 MTP", section "V3 的 MoE：256 个专家怎样选
 * 8 个", router code block from the logits to its last line, with the softmax
 * routing of "MoE架构揭秘：大模型参数激活率与专家路由机制解析", section 3.1, and the
 * capacity of "GPT-4 Has 1.8 Trillion Parameters ...", section 2.2, as
 * configured).
 * out [T,H] in cfg->out_dtype.  topk_idx, topk_w, expert_counts and
 * logits_out are optional outputs (NULL = keep them in the workspace). */
moe_status moe_forward(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                       const float* logit_bias, const float* sel_bias, const void* w_gate, const void* w_up,
                       const void* w_down, void* out, int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                       float* logits_out, void* ws, size_t ws_bytes, void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Every argument but ws and ws_bytes as moe_forward;
 * the caller still passes every input and output.  The workspace is a static
 * device array of the library, 64 MiB per GPU, held until the process ends
 * (enough for the DeepSeek-V3-shaped layer up to about 200 tokens): a layer
 * and batch whose moe_workspace_size exceeds 64 MiB are rejected with
 * MOE_ERR_WORKSPACE before anything is enqueued.  No device memory is
 * allocated or freed.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents (nothing in it is assumed zero): calls that
 * may overlap on one GPU (two host threads, or two streams without an order
 * between them) race and must be serialised by the caller.  Not for MOE_FP8
 * layers (MOE_ERR_INVALID_ARG). */
moe_status moe_forward_noalloc(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                               const float* logit_bias, const float* sel_bias, const void* w_gate, const void* w_up,
                               const void* w_down, void* out, int32_t* topk_idx, float* topk_w,
                               int32_t* expert_counts, float* logits_out, void* stream);

/* moe_forward with hash routing (moe_route_hash's selection): token_ids,
 * tid2eid and vocab as there, every other argument as moe_forward. */
moe_status moe_forward_hash(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                            const float* logit_bias, const int32_t* token_ids, const int32_t* tid2eid, int64_t vocab,
                            const void* w_gate, const void* w_up, const void* w_down, void* out, int32_t* topk_idx,
                            float* topk_w, int32_t* expert_counts, float* logits_out, void* ws, size_t ws_bytes,
                            void* stream);

/* FP8 experts ("15. DeepSeek：MLA、MoE 与 MTP", section "FP8 训练是训练配方，不是架构":
 * E4M3 inputs of the matrix products, one scale per 1 x 128 activation tile
 * and per 128 x 128 weight block, UE8M0 scales as in V3.1).  cfg->dtype must
 * be MOE_FP8.
 *   x            [T,H] bf16;  w_router [E,H] bf16
 *   w_gate, w_up [E+S,I,H] E4M3 codes (1 byte: sign, 4 exponent bits with
 *                bias 7, 3 mantissa bits; subnormals; 0x7F/0xFF are NaN)
 *   s_gate, s_up [E+S,I/128,H/128] UE8M0 bytes b: the block's scale is
 *                2^(b-127) (b = 255 is not allowed)
 *   w_down       [E+S,H,I] E4M3 codes;  s_down [E+S,H/128,I/128] UE8M0
 * Element (r,c) of an expert matrix is code(r,c) * 2^(b(r/128,c/128) - 127).
 * x and the SwiGLU output h are quantised per row and 128-wide tile as
 * moe_quantize_fp8 describes (h from its fp32 value); the products run on the
 * matrix cores with the scales applied per 128-wide K block and fp32
 * accumulation.  Everything else (routing, capacity, combine, outputs,
 * workspace) as moe_forward / moe_expert_ffn. */
moe_status moe_forward_fp8(const moe_config* cfg, int64_t T, const void* x, const void* w_router,
                           const float* logit_bias, const float* sel_bias, const uint8_t* w_gate, const uint8_t* s_gate,
                           const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                           void* out, int32_t* topk_idx, float* topk_w, int32_t* expert_counts, float* logits_out,
                           void* ws, size_t ws_bytes, void* stream);
moe_status moe_expert_ffn_fp8(const moe_config* cfg, int64_t T, const void* x, const uint8_t* w_gate,
                              const uint8_t* s_gate, const uint8_t* w_up, const uint8_t* s_up, const uint8_t* w_down,
                              const uint8_t* s_down, const int32_t* expert_offsets, const int32_t* row_token,
                              void* y_rows, void* ws, size_t ws_bytes, void* stream);
/* 1 x 128 tile quantisation of bf16 rows to E4M3 (the activation format of
 * the FP8 experts).
 *   in      [rows,K] bf16 device, 16-byte aligned; K a positive multiple of 128
 *   codes   [rows,K] E4M3 out, 8-byte aligned
 *   scales  [rows, scale_stride] UE8M0 out; tile j of row r at r*scale_stride + j
 * A tile's scale is 2^p for the smallest p >= -127 with amax/2^p <= 448
 * (p = -127 when amax is zero or subnormal); each code is value/2^p rounded
 * to the nearest E4M3 value, ties to the even mantissa, sign kept (also on
 * zero).  Bytes of scales past K/128 in a row are left untouched. */
moe_status moe_quantize_fp8(int64_t rows, int32_t K, const void* in, uint8_t* codes, uint8_t* scales,
                            int32_t scale_stride, void* stream);

/* One step of auxiliary-loss-free load balancing ("15. DeepSeek：MLA、MoE 与
 * MTP", section "V3 的 MoE：256 个专家怎样选 8 个", the bias paragraph) and the
 * load telemetry of its monitoring paragraph (plus the expert-call entropy of
 * "GPT-4稀疏激活原理：2%参数调用背后的MoE工程实践", section 4.4).
 *   expert_counts [E] int32, e.g. from moe_route / moe_forward (N = their sum)
 *   sel_bias      [E] fp32, updated in place, or NULL (telemetry only): an
 *                 expert with n_e > N/E gets fl32(b - gamma), one with
 *                 n_e < N/E gets fl32(b + gamma), one at the mean keeps b
 *                 (the test is exact: n_e * E against N); N == 0: no change
 *   gamma         the step, >= 0 (the page uses 0.001)
 *   share         [E] fp32 out, n_e / N (0 when N == 0), or NULL
 *   stats         [4] fp32 out, or NULL: entropy of the shares in nats
 *                 (0 ln 0 = 0), largest share, experts above the mean,
 *                 experts below the mean
 * Only cfg's expert count is used.  Deterministic (fixed-order reductions). */
moe_status moe_balance_update(const moe_config* cfg, const int32_t* expert_counts, float* sel_bias, float gamma,
                              float* share, float* stats, void* stream);

/* Attainable-rate probes: the library's own kernels measuring what the part
 * delivers, so that the layer's rates can be quoted against the sustained
 * rates of the same chip at its power limit as well as against the nominal
 * peaks.  Each enqueues one kernel on `stream` (timed by the caller) and
 * writes blocks * 256 floats to the device array `sink` (values without
 * meaning, written so nothing is optimised away).
 * moe_probe_mfma_bf16: `blocks` workgroups of four wavefronts, each wavefront
 *   issuing `iters` rounds of eight independent v_mfma_f32_32x32x16_bf16 on
 *   pseudo-random register operands: vary = 1 takes four A and four B
 *   fragments in turn (inputs change between instructions, as in a GEMM),
 *   vary = 0 one fixed pair; *flops (host) gets the FLOPs the launch
 *   performs (blocks * iters * 4 * 8 * 32768).
 * moe_probe_mfma_fp8: the same with v_mfma_scale_f32_32x32x64_f8f6f4 (the
 *   FP8 expert GEMMs' instruction) on pseudo-random E4M3 operands with unit
 *   block scales; *flops = blocks * iters * 4 * 8 * 131072.
 * moe_probe_read: reads the `bytes` (a positive multiple of 16) of the
 *   16-byte aligned device buffer `buf` once, in 16-byte pieces with eight in
 *   flight per lane, over `blocks` workgroups of 256 threads; mode 0: plain
 *   loads, 1: non-temporal loads, 2: global->LDS copies (the form the expert
 *   GEMMs stream their operands in), 3: global->LDS copies with the
 *   non-temporal policy. */
moe_status moe_probe_mfma_bf16(int32_t vary, int32_t blocks, int64_t iters, float* sink, double* flops,
                               void* stream);
moe_status moe_probe_mfma_fp8(int32_t vary, int32_t blocks, int64_t iters, float* sink, double* flops,
                              void* stream);
moe_status moe_probe_read(int32_t mode, int32_t blocks, const void* buf, size_t bytes, float* sink, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

/* Optional per-kernel timing.  moe_timing_enable(n) makes the library bracket
 * each of its next n kernel launches with hipEventRecord on the launch stream
 * (n <= 0 disables).  moe_timing_read waits for those events and returns, per
 * kernel id (< n_kernels), the summed duration in milliseconds and the launch
 * count; then clears the record.  moe_kernel_name(id) names kernel id (NULL
 * past the last).  Not thread-safe: time from one thread. */
moe_status moe_timing_enable(int32_t max_launches);
moe_status moe_timing_read(double* ms, int64_t* launches, int32_t n_kernels);
const char* moe_kernel_name(int32_t id);
/* Bracket only the launches of kernel `kernel_id` (-1: every kernel, the
 * default): two events per timed launch perturb the stream less than two per
 * kernel of the layer (MOE_ERR_INVALID_ARG for an unknown id). */
moe_status moe_timing_only(int32_t kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
