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

/* Canvas attention of one layer (write-up Figure 4 stage 2: bidirectional
 * over the canvas plus attention to the cached context; model card "Model
 * Overview").  For canvas b, query head h, position i:
 *   o = sum_j softmax_j(q . k_j / sqrt(D)) v_j
 * over the prefix_len[b] cached keys of slot req[b] and the canvas_len
 * canvas keys (with causal != 0 only canvas keys j <= i), KV head
 * h / (Hq / Hkv).
 * qkv [n*canvas_len, (Hq + 2 Hkv) D] bf16 (Q, K, V of the canvas rows as
 * written by the Q/K/V projection); k_cache / v_cache: one layer,
 * [max_requests][Hkv][max_kv_len][D] bf16; out [n*canvas_len, Hq D] bf16.
 * kv_splits: number of key ranges processed by separate workgroups and
 * merged by log-sum-exp weights (0 = automatic, else 1..32). */
dg_status dg_op_canvas_attention(const void* qkv, int32_t n,
                                 int32_t canvas_len, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim,
                                 const void* k_cache, const void* v_cache,
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

/* Mixture-of-experts FFN of one layer on normalised rows: router logits,
 * top-k, grouping of the (token, rank) pairs by expert (per-expert slots
 * when the experts average at most 32 pairs, else a stable counting-sort
 * permutation), grouped gate/up GEMM with SwiGLU, grouped down GEMM scaled
 * by the gate weight, un-permute summing each token's pairs in rank order.
 *   y_t = sum_j w_tj W_d,e (silu(W_g,e x_t) * W_u,e x_t),  e = idx_tj.
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

/* Entropy-bounded selection on explicit state (same rule as dg_eb_select):
 * entropy [n, 256] fp32, argmax [n, 256] int32, committed [n, 256] uint8
 * in/out, tokens [n, 256] int32 in/out, step [n] int32 in/out, gamma [n]
 * fp32, n_new [n] int32 out, done [n] uint8 out. */
dg_status dg_op_eb_select(int32_t n, const float* entropy,
                          const int32_t* argmax, uint8_t* committed,
                          int32_t* tokens, int32_t* step, const float* gamma,
                          int32_t step_cap, int32_t refine, int32_t* n_new,
                          uint8_t* done, void* stream);

/* KV append (write-up Figure 4 stage 3): copy the K and V of canvas b's
 * canvas_len rows from qkv into cache rows [row0[b], row0[b] + canvas_len)
 * of slot req[b] in one layer's k_cache / v_cache
 * ([max_requests][Hkv][max_kv_len][D] bf16).  req, row0: (host) [n]. */
dg_status dg_op_kv_append(const void* qkv, int32_t n, int32_t canvas_len,
                          int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, void* k_cache, void* v_cache,
                          int32_t max_requests, int32_t max_kv_len,
                          const int32_t* req, const int32_t* row0,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DG_OPS_H */
