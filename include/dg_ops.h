/*
 * libdg op-level entry points: each runs exactly the kernels the context
 * calls of dg.h use for one step of the pipeline, on caller-provided buffers,
 * so that every step can be checked and timed on its own.  Same conventions
 * as dg.h (device pointers unless marked (host), caller-owned memory,
 * asynchronous on the given hipStream_t `stream`, host-side validation before
 * any launch, no allocation, no abort).  `workspace` must hold the bytes the
 * matching *_workspace_bytes function returns.
 */
#ifndef DG_OPS_H
#define DG_OPS_H

#include "dg.h"

#ifdef __cplusplus
extern "C" {
#endif

/* RMSNorm of fp32 rows into bf16: out = bf16(x / sqrt(mean(x^2) + eps) * g)
 * (pre-norm blocks of the decoder; layer internals are not on the pages).
 * x [rows, H] fp32, g [H] fp32, out [rows, H] bf16. */
dg_status dg_op_rmsnorm(const float* x, int32_t rows, int32_t hidden,
                        const float* g, float eps, void* out, void* stream);

/* Dense projection y = x W^T with bf16 operands and fp32 accumulation
 * (Q/K/V, output projection and router logits of every layer).
 * x [M, K] bf16, w [N, K] bf16 in the packed layout (dg.h), K a multiple
 * of 64.
 * mode 0: out [M, N] bf16 = y;  1: out [M, N] fp32 = y;
 * mode 2: out [M, N] fp32 += y (residual add). */
dg_status dg_op_linear(const void* x, int32_t m, int32_t k, const void* w,
                       int32_t n, int32_t mode, void* out, void* stream);

/* The W8A8 projection (proj_dtype DG_FP8_E4M3; write-up Table 3 and
 * Figure 11 captions, FP8 serving): y[r, n] = s_r x w_scale[n] x
 * sum_k q_r[k] q_n[k], with x's rows [M, K] bf16 quantised to E4M3 codes
 * q_r and scales s_r as dg_op_quantize_rows does and w8 [N, K] E4M3 codes
 * (packed, DG_FP8_E4M3) with per-row scales w_scale [N]; modes as
 * dg_op_linear.  K a multiple of 128 up to 4096 (else DG_ERR_SHAPE); the
 * FP8 MFMA from 1024 rows.  workspace of dg_op_linear_e4m3_workspace_bytes
 * (m, k), device memory, 256-byte aligned. */
dg_status dg_op_linear_e4m3(const void* x, int32_t m, int32_t k, const void* w8,
                            const float* w_scale, int32_t n, int32_t mode,
                            void* out, void* workspace, size_t workspace_bytes,
                            void* stream);
size_t dg_op_linear_e4m3_workspace_bytes(int32_t m, int32_t k);

/* Canvas attention of one layer (write-up Figure 4 stage 2: bidirectional
 * over the canvas plus attention to the cached context; model card "Model
 * Overview").  For canvas b, query head h, position i:
 *   o = sum_j softmax_j(q . k_j / sqrt(D)) v_j
 * over the prefix_len[b] cached keys of slot req[b], the canvas keys of the
 * canvases before b in the batch with the same req (several canvases of
 * one request, contiguous in block order: model card "block-autoregressive
 * multi-canvas sampling"), and the canvas_len keys of canvas b (with
 * causal != 0 only its keys j <= i), KV head h / (Hq / Hkv).
 * DG_ERR_INVALID_ARG if equal req entries are not contiguous.
 * qkv [n*canvas_len, (Hq + 2 Hkv) D] bf16 (Q, K, V of the canvas rows as
 * written by the Q/K/V projection); k_cache / v_cache: one layer,
 * [max_requests][Hkv][max_kv_len][D] bf16, or with k_scale / v_scale
 * (both or neither) the E4M3 cache of the model's kv_dtype: codes at the
 * same offsets in bytes and k_scale / v_scale [max_requests][Hkv]
 * [max_kv_len] fp32, a cached row read as bf16(code value x scale) in
 * fp32 (write-up Table 3 caption, FP8); out [n*canvas_len, Hq D] bf16.
 * kv_splits: number of key ranges processed by separate workgroups and
 * merged by log-sum-exp weights (0 = automatic, else 1..32). */
dg_status dg_op_canvas_attention(const void* qkv, int32_t n,
                                 int32_t canvas_len, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim,
                                 const void* k_cache, const void* v_cache,
                                 const float* k_scale, const float* v_scale,
                                 int32_t max_requests, int32_t max_kv_len,
                                 const int32_t* req, const int32_t* prefix_len,
                                 int32_t causal, int32_t kv_splits, void* out,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);
size_t dg_op_attention_workspace_bytes(int32_t n, int32_t canvas_len,
                                       int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t head_dim, int32_t kv_splits);

/* Router top-k (write-up Table 1: 8 of 128 experts per token): per token the
 * k largest logits, lower expert id first on ties, in rank order, and gate
 * weights = softmax over the k selected logits.
 * logits [T, E] fp32 -> idx [T, k] int32, w [T, k] fp32. */
dg_status dg_op_router_topk(const float* logits, int32_t tokens,
                            int32_t n_experts, int32_t top_k, int32_t* idx,
                            float* w, void* stream);

/* Mixture-of-experts FFN of one layer on normalised rows (write-up Table 1:
 * 8 of 128 experts active per token, "+ 1 shared"): router logits,
 * top-k, grouping of the (token, rank) pairs by expert (per-expert slots
 * when the experts average at most 32 pairs, else a stable counting-sort
 * permutation), grouped gate/up GEMM with SwiGLU, grouped down GEMM scaled
 * by the gate weight, un-permute summing each token's pairs in rank order.
 *   y_t = sum_j w_tj W_d,e (silu(W_g,e x_t) * W_u,e x_t),  e = idx_tj,
 * plus, with desc->n_shared_experts = 1, the shared expert (group E) with
 * weight 1 as the token's last pair.
 * desc: hidden, n_experts, top_k, expert_ffn, expert_dtype are used;
 * weights: w_router, w_gate_up, w_down (packed) and the e4m3 scales are used.
 * xhat [T, H] bf16 -> y [T, H] fp32.  route_idx [T, k] / route_w [T, k] /
 * counts [E] (tokens per expert) are optional outputs (NULL to skip). */
dg_status dg_op_moe(const dg_model_desc* desc, const dg_layer_weights* weights,
                    const void* xhat, int32_t tokens, float* y,
                    int32_t* route_idx, float* route_w, int32_t* counts,
                    void* workspace, size_t workspace_bytes, void* stream);
size_t dg_op_moe_workspace_bytes(const dg_model_desc* desc, int32_t tokens);

/* Tied LM head with fused vocabulary statistics (write-up Table 1: 262k
 * vocabulary): z = xhat E^T per row; lse = log sum exp z; entropy =
 * lse - sum softmax(z) z (nats, clamped at 0); argmax = lowest id of max z.
 * Logits are not materialised unless `logits` is non-NULL.
 * xhat [M, H] bf16, embed [V, H] bf16 packed -> entropy, lse [M] fp32,
 * argmax [M] int32, logits NULL or [M, V] fp32. */
dg_status dg_op_lmhead_entropy(const void* xhat, int32_t m, int32_t hidden,
                               const void* embed, int32_t vocab,
                               float* entropy, float* lse, int32_t* argmax,
                               float* logits, void* workspace,
                               size_t workspace_bytes, void* stream);
size_t dg_op_lmhead_workspace_bytes(int32_t m, int32_t vocab);

/* The E4M3 LM head (W8A8: the model's lm_dtype DG_FP8_E4M3, write-up
 * Table 3 and Figure 11 captions, FP8 serving): as dg_op_lmhead_entropy,
 * with the head's weights w8 [V, H] as E4M3 codes (packed,
 * dg_pack_weights with DG_FP8_E4M3) and one fp32 scale per vocabulary row
 * w_scale [V]; each row of xhat is quantised to E4M3 codes with its row
 * scale as dg_op_quantize_rows does, and logit v = s_row x w_scale[v] x
 * sum q_row q_v.  hidden a multiple of 128 up to 4096 (else DG_ERR_SHAPE);
 * workspace of dg_op_lmhead_e4m3_workspace_bytes(m, hidden, vocab), device
 * memory, 256-byte aligned. */
dg_status dg_op_lmhead_entropy_e4m3(const void* xhat, int32_t m, int32_t hidden,
                                    const void* w8, const float* w_scale,
                                    int32_t vocab, float* entropy, float* lse,
                                    int32_t* argmax, float* logits,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);
size_t dg_op_lmhead_e4m3_workspace_bytes(int32_t m, int32_t hidden, int32_t vocab);

/* Allocation-free variant of dg_op_lmhead_entropy, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments and
 * results as dg_op_lmhead_entropy without logits or workspace: the per-tile
 * partials go to a static device array of DG_STATIC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends (its address
 * is looked up once per device, on the first call with that device
 * current).  Calls nothing that allocates.  Limit: m * ceil(vocab / 128) *
 * 16 bytes must fit the array (256 rows at a 262144-token vocabulary hold
 * 8 MiB), else DG_ERR_CAPACITY before any launch.  Every call on one GPU
 * shares that GPU's array, which keeps the last call's partials: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * serialised by the caller.  DG_ERR_HIP if the array's address cannot be
 * obtained. */
#define DG_STATIC_SCRATCH_BYTES (16u << 20)
dg_status dg_op_lmhead_entropy_static(const void* xhat, int32_t m,
                                      int32_t hidden, const void* embed,
                                      int32_t vocab, float* entropy,
                                      float* lse, int32_t* argmax,
                                      void* stream);

/* Tied LM head with temperature sampling (the rule of dg_sampling, with
 * each row's temperature and counter given): xhat [M, H] bf16, embed
 * [V, H] bf16 packed, tau [M] fp32 (0 or >= 1e-6: smaller positive values
 * overflow z / tau, not checked), ctr [M, 3] int32 = (position,
 * step, canvas) words of the Philox counter, seed the 64-bit key ->
 * entropy, lse [M] of softmax(z / tau) (tau 0: entropy 0, lse of z),
 * argmax [M] of z, sample [M] drawn token.  All pointers are device
 * memory; workspace of dg_op_lmhead_sample_workspace_bytes(m, vocab). */
dg_status dg_op_lmhead_sample(const void* xhat, int32_t m, int32_t hidden,
                              const void* embed, int32_t vocab, const float* tau,
                              const int32_t* ctr, uint64_t seed, float* entropy,
                              float* lse, int32_t* argmax, int32_t* sample,
                              void* workspace, size_t workspace_bytes,
                              void* stream);
size_t dg_op_lmhead_sample_workspace_bytes(int32_t m, int32_t vocab);

/* Per-row E4M3 quantisation of activations (the FP8 rows of the expert
 * GEMMs when act_dtype is DG_FP8_E4M3; write-up Table 3 caption, FP8):
 * x [rows, K] bf16 (K a multiple of 8, at most 4096) -> scale [rows] fp32 = max|x_r| /
 * 448 (1 for a zero row) and codes [rows, K] = E4M3(x * (448 / max|x_r|)):
 * nearest, ties to even, saturating; the divisions and the product in
 * fp32.  codes or values (their bf16
 * values [rows, K]) may be NULL, not both. */
dg_status dg_op_quantize_rows(const void* x, int32_t rows, int32_t k,
                              uint8_t* codes, void* values, float* scale,
                              void* stream);

/* Entropy-bounded selection on explicit state (same rule as dg_eb_select)
 * over n canvases of C = canvas_len positions (0: 256):
 * entropy [n, C] fp32, argmax [n, C] int32, committed [n, C] uint8
 * in/out, tokens [n, C] int32 in/out, step [n] int32 in/out, gamma [n]
 * fp32, n_new [n] int32 out, done [n] uint8 out. */
dg_status dg_op_eb_select(int32_t n, int32_t canvas_len, const float* entropy,
                          const int32_t* argmax, uint8_t* committed,
                          int32_t* tokens, int32_t* step, const float* gamma,
                          int32_t step_cap, int32_t refine, int32_t* n_new,
                          uint8_t* done, void* stream);

/* KV append (write-up Figure 4 stage 3): copy the K and V of canvas b's
 * canvas_len rows from qkv into cache rows [row0[b], row0[b] + canvas_len)
 * of slot req[b] in one layer's k_cache / v_cache
 * ([max_requests][Hkv][max_kv_len][D] bf16; with k_scale / v_scale, both or
 * neither, an E4M3 cache: each row quantised as dg_op_quantize_rows does,
 * its codes at the same offsets in bytes and its scale in k_scale /
 * v_scale [max_requests][Hkv][max_kv_len]).  req, row0: (host) [n]. */
dg_status dg_op_kv_append(const void* qkv, int32_t n, int32_t canvas_len,
                          int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, void* k_cache, void* v_cache,
                          float* k_scale, float* v_scale,
                          int32_t max_requests, int32_t max_kv_len,
                          const int32_t* req, const int32_t* row0,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_OPS_H */
