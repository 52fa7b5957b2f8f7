/*
 * libdg -- one block-diffusion denoising step over a 256-token canvas on
 * MI355X (gfx950), behind a plain C ABI.
 *
 * The calls follow the generation pipeline of the "DiffusionGemma Technical
 * Report" (write-up of the paper), Figure 4:
 *   1. context encoding: the prompt's K/V fill a per-request cache
 *      (dg_prefill_kv);
 *   2. denoising loop: a noisy canvas is refined by the decoder, which
 *      attends bidirectionally over the canvas and to the cache
 *      (dg_denoise_step), and the entropy-bounded sampler with adaptive
 *      stopping commits confident positions (dg_eb_select; write-up "What
 *      they did", model card "Benchmark Results");
 *   3. encode & append: the finished canvas is encoded causally and its K/V
 *      appended to the cache (dg_commit_block; write-up Figure 4 stage 3,
 *      model card "Model Overview").
 *
 * Conventions for every function in this header and in dg_ops.h:
 *   - Pointers are DEVICE pointers unless marked (host).
 *   - The caller owns every buffer (weights, caches, workspace, canvas state,
 *     outputs).  The library never allocates or frees device memory; a
 *     context owns host metadata only.
 *   - Calls enqueue work on the context's (or the given) HIP stream and
 *     return without synchronising; results are valid after that stream is
 *     synchronised.  A context is single-stream and not thread-safe.
 *   - Arguments, shapes and capacities are validated on the host before any
 *     launch; a failed validation returns an error status and enqueues
 *     nothing.  A failed launch returns DG_ERR_HIP.  Faults inside kernels
 *     surface at the caller's next synchronisation, or, with DG_DEBUG_SYNC=1
 *     in the environment (read once per process), as DG_ERR_HIP from the
 *     call that launched the faulting kernel: every launch is then followed
 *     by a device synchronisation.  Nothing aborts, exits or throws across
 *     the ABI.
 *   - Further debugging aids, also read once per process:
 *     DG_POISON=1: dg_prefill_kv (token mode), dg_denoise_step,
 *       dg_commit_block and dg_ar_step first fill the workspace's value
 *       regions (activations, partials, router logits, expert rows; not its
 *       indices and counts) with 0xFF bytes (NaN in fp32, bf16 and E4M3), so
 *       a read of scratch that no kernel of the call wrote shows up as NaN
 *       in the outputs;
 *     DG_CHECK=1: dg_commit_block reads the committed flags back (a stream
 *       synchronisation) and returns DG_ERR_STATE for a canvas with a
 *       position still uncommitted;
 *     DG_KV_SPLIT=s (1..32): the engine's attention splits every key range
 *       into s parts (at most what the workspace's partials hold) instead of
 *       choosing the count itself.
 *   - bf16 means IEEE bfloat16 stored as 16-bit words; e4m3 means OCP FP8
 *     E4M3 ("fn": no infinities, max 448) bytes.
 *   - Matrices are row-major [rows, cols] with cols contiguous; a weight
 *     matrix is [out, in] so that y = W x.
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_CANVAS 256     /* positions per canvas (write-up: 256-token blocks) */
#define DG_MAX_BATCH 64   /* canvases per call */

typedef struct dg_ctx dg_ctx;

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = 1, /* null pointer, bad enum, out-of-range scalar */
  DG_ERR_SHAPE = 2,       /* model shape the kernels do not support */
  DG_ERR_CAPACITY = 3,    /* KV cache, batch or workspace too small */
  DG_ERR_STATE = 4,       /* request slot in the wrong state */
  DG_ERR_HIP = 5,         /* a HIP runtime call or launch failed */
  DG_ERR_UNSUPPORTED = 6
} dg_status;

typedef enum { DG_BF16 = 0, DG_FP8_E4M3 = 1 } dg_dtype;

/* Model shape.  Mixture-of-experts transformer (write-up Table 1: 8 of 128
 * experts active, 262k vocabulary; the layer internals are the reading the
 * library implements: pre-norm RMSNorm blocks, grouped-query attention
 * without positional encoding, top-k softmax router over SwiGLU experts,
 * LM head tied to the embedding).
 * Supported: head_dim in {64, 128}; n_q_heads a multiple of n_kv_heads;
 * hidden, n_q_heads*head_dim and expert_ffn multiples of 64;
 * n_experts <= 256; 1 <= top_k <= min(n_experts, 16); vocab >= 1. */
typedef struct {
  int32_t n_layers;
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t n_experts;
  int32_t top_k;
  int32_t expert_ffn;
  int32_t vocab;
  float rms_eps;          /* e.g. 1e-6 */
  int32_t expert_dtype;   /* dg_dtype of w_gate_up / w_down */
  int32_t canvas_len;     /* positions per canvas, 1..256 (0: 256); the
                             write-up's Table 7 varies the canvas size (128
                             or 256).  Every [n, 256] array of the calls
                             below is [n, canvas_len]. */
  int32_t n_shared_experts; /* 0 or 1: a shared SwiGLU expert of width
                             expert_ffn that every token uses with weight 1
                             next to its top_k routed experts (write-up
                             Table 1, "+ 1 shared"); it is the last group of
                             w_gate_up / w_down (and of their scales) */
  int32_t act_dtype;      /* dg_dtype of the expert GEMMs' token rows (the
                             write-up serves in FP8: Table 3 and Figure 11
                             captions).  DG_FP8_E4M3 (W8A8; needs E4M3
                             experts and hidden, expert_ffn multiples of
                             128 up to 4096): each row (a token's FFN-norm output for
                             gate/up, a pair's SwiGLU output for down) is
                             quantised with scale s = max|row| / 448 (1 for
                             a zero row), codes = E4M3(row x (448 / max|row|))
                             to nearest, ties to even, saturating (fp32); the
                             product is s x w_scale[n] x sum q_row q_w,
                             on gfx950's FP8 MFMA where many rows share an
                             expert.  DG_BF16: bf16 rows. */
  int32_t kv_dtype;       /* dg_dtype of the KV cache.  DG_FP8_E4M3: every
                             cached key / value row (one head, one position)
                             is stored as E4M3 codes quantised like the
                             activation rows above, with its fp32 scale, and
                             attention reads it as bf16(code value x scale);
                             keys and values of the canvases in a call are
                             used as computed until they are committed.
                             See dg_kv_cache_bytes for the layout. */
  int32_t lm_dtype;       /* dg_dtype of the LM head (the write-up serves in
                             FP8: Table 3 and Figure 11 captions).
                             DG_FP8_E4M3 (W8A8; hidden a multiple of 128 up
                             to 4096): the head reads dg_weights.lm_head,
                             E4M3 codes of the tied table with one fp32
                             scale per vocabulary row, and takes each
                             final-normed row as E4M3 codes with its row
                             scale, quantised as the act_dtype rows above;
                             logit v = s_row x lm_head_scale[v] x
                             sum q_row q_v.  The embedding lookup keeps the
                             bf16 table.  DG_BF16: the bf16 table. */
  int32_t proj_dtype;     /* dg_dtype of the Q/K/V and output projections
                             (the same FP8 serving).  DG_FP8_E4M3 (W8A8;
                             hidden and n_q_heads*head_dim multiples of 128
                             up to 4096): w_qkv and w_o are E4M3 codes with
                             one fp32 scale per output row (qkv_scale,
                             o_scale) and each input row (a token's
                             attention-norm output, its attention output) is
                             quantised as the act_dtype rows above; out[n] =
                             s_row x scale[n] x sum q_row q_n, on gfx950's
                             FP8 MFMA from 1024 rows.  The router keeps bf16
                             weights and rows.  DG_BF16: bf16 projections. */
} dg_model_desc;

/* Packed weight layout.  Every weight matrix the kernels read (w_qkv, w_o,
 * w_router, w_gate_up, w_down and the embedding) is passed in a tiled form
 * made by dg_pack_weights from the row-major matrix [R, K] (per group for
 * the expert matrices): blocks of 1024 bytes, each 16 rows x 64/b values (b
 * = element bytes); in a block the 16 bytes at 16 * (r + 16 q) hold row
 * 16 rb + r, values kb * 64/b + q * 16/b .. + 16/b - 1, which is the operand
 * order of the 16x16x32 MFMA (one contiguous kilobyte per wave load).  Row
 * tiles come in groups of 4 (64 rows) and inside a group the blocks are
 * ordered by kb, then tile: block (rb, kb) is at byte
 * ((rb / 4) * 4 * KB + kb * 4 + rb % 4) * 1024, KB = K * b / 64, so the
 * tiles of a group streamed together in K order form one contiguous run.
 * Rows are zero-padded to a multiple of 64 (with groups > 1 the rows per
 * group must be a multiple of 64); K must be a multiple of 64/b. */
size_t dg_packed_bytes(int32_t groups, int32_t rows, int32_t cols, int32_t dtype);

/* Pack groups x [rows, cols] row-major (bf16 or e4m3 bytes, device memory)
 * into dst (dg_packed_bytes bytes, device, must not overlap src), enqueued
 * on stream.  DG_ERR_SHAPE for shapes the layout cannot hold,
 * DG_ERR_INVALID_ARG for NULL pointers or another dtype. */
dg_status dg_pack_weights(const void* src, int32_t groups, int32_t rows,
                          int32_t cols, int32_t dtype, void* dst, void* stream);

/* Weights of one layer (all device pointers, read-only, must outlive the
 * context).  Matrices are in the packed layout above. */
typedef struct {
  const float* attn_norm;     /* [H] fp32 RMSNorm gain before attention */
  const void* w_qkv;          /* [(Hq + 2 Hkv) D, H] bf16 (or e4m3, proj_dtype):
                                 Q rows, K rows, V rows */
  const void* w_o;            /* [H, Hq D] bf16 (or e4m3, proj_dtype) */
  const float* ffn_norm;      /* [H] fp32 RMSNorm gain before the MoE */
  const void* w_router;       /* [E, H] bf16 */
  const void* w_gate_up;      /* E + S groups of [2F, H] bf16 or e4m3: F gate rows, then
                                 F up rows (S = n_shared_experts; the shared expert last) */
  const void* w_down;         /* E + S groups of [H, F] bf16 or e4m3 */
  const float* gate_up_scale; /* [E + S, 2F] fp32 per-row scale (e4m3 only, else NULL) */
  const float* down_scale;    /* [E + S, H] fp32 per-row scale (e4m3 only, else NULL) */
  const float* qkv_scale;     /* proj_dtype DG_FP8_E4M3: [(Hq + 2 Hkv) D] fp32 per-row
                                 scale of w_qkv (then e4m3), else NULL */
  const float* o_scale;       /* proj_dtype DG_FP8_E4M3: [H] fp32 per-row scale of w_o */
} dg_layer_weights;

typedef struct {
  const void* embed;               /* [V, H] bf16, packed; also the tied LM head */
  const float* final_norm;         /* [H] fp32 */
  const dg_layer_weights* layers;  /* (host) array of n_layers entries, copied */
  const void* lm_head;             /* lm_dtype DG_FP8_E4M3: [V, H] e4m3, packed
                                      (else NULL, unused) */
  const float* lm_head_scale;      /* lm_dtype DG_FP8_E4M3: [V] fp32 per-row scale */
} dg_weights;

/* Bytes of device workspace a context needs for up to max_canvases canvases
 * per call (0 if the shape is unsupported). */
size_t dg_workspace_bytes(const dg_model_desc* desc, int32_t max_canvases);

/* Bytes of ONE of the two caches (K or V): layout
 * [n_layers][max_requests][n_kv_heads][max_kv_len][head_dim] bf16; with
 * kv_dtype DG_FP8_E4M3 the same array of E4M3 codes (one byte each)
 * followed by the fp32 scale of every row,
 * [n_layers][max_requests][n_kv_heads][max_kv_len]. */
size_t dg_kv_cache_bytes(const dg_model_desc* desc, int32_t max_requests,
                         int32_t max_kv_len);

/* Create a context over caller-owned memory.  k_cache / v_cache hold
 * dg_kv_cache_bytes each; workspace holds dg_workspace_bytes(desc,
 * max_canvases).  stream is a hipStream_t (NULL: the null stream).  All
 * request slots start with kv_len 0.  On error *out is set to NULL. */
dg_status dg_create(const dg_model_desc* desc, const dg_weights* weights,
                    int32_t max_requests, int32_t max_kv_len,
                    int32_t max_canvases, void* k_cache, void* v_cache,
                    void* workspace, size_t workspace_bytes, void* stream,
                    dg_ctx** out);
void dg_destroy(dg_ctx* ctx); /* frees host state only; NULL is a no-op */

/* Stage 1 (write-up Figure 4, "context encoding"; model card "Model
 * Overview": the causal encoder runs over the prompt and fills the cache).
 * Exactly one of {tokens} or {k, v} is given.
 * Install mode: k and v are [n_layers][n_kv_heads][n][head_dim] bf16
 * (already encoded prompt K/V) and are copied into cache rows [0, n) of
 * slot req.
 * Token mode: tokens is [n] int32 (device; ids outside [0, V) are clamped
 * when embedded); the prompt is encoded causally through every layer (the
 * same computation as dg_commit_block, position i seeing positions <= i) in
 * chunks of up to 256 tokens, each layer's K/V written to cache rows
 * [0, n).  Uses the context workspace (a denoise step's intermediate state
 * is overwritten).
 * Either way the slot's kv_len becomes n; DG_ERR_CAPACITY if n >
 * max_kv_len. */
dg_status dg_prefill_kv(dg_ctx* ctx, int32_t req, int32_t n,
                        const int32_t* tokens, const void* k, const void* v);

/* Canvas state of a batch of n canvases.  Several canvases may belong to
 * one request (multi-canvas sampling, model card feature list
 * "block-autoregressive multi-canvas sampling"; write-up Table 7, number of
 * canvases): they are contiguous in the batch, in block order, and canvas j
 * of a request attends to the request's cache, then to every position of
 * the request's canvases before it in the batch (earlier blocks fully
 * visible, later ones not), then to itself.  DG_ERR_INVALID_ARG if the
 * canvases of a request are not contiguous. */
typedef struct {
  int32_t n;               /* 1..max_canvases */
  const int32_t* req;      /* (host) [n] request slot of each canvas */
  int32_t* tokens;         /* [n, 256] int32 current canvas tokens in [0, V),
                              in/out (ids outside are clamped when embedded) */
  uint8_t* committed;      /* [n, 256] 1 = committed (frozen), in/out */
  int32_t* step;           /* [n] denoise steps taken in this block, in/out */
} dg_canvas_batch;

/* Optional per-layer captures for parity checks (each NULL to skip). */
typedef struct {
  void* attn_out;       /* [L, n*256, Hq*D] bf16 attention output before W_o */
  float* moe_out;       /* [L, n*256, H] fp32 MoE mixture added to the residual */
  int32_t* route_idx;   /* [L, n*256, top_k] selected experts, rank order */
  float* route_w;       /* [L, n*256, top_k] gate weights */
  float* router_logits; /* [L, n*256, E] fp32 */
  float* final_xhat;    /* [n*256, H] fp32 copy of the bf16 final-norm rows,
                           compacted in the order of the uncommitted rows */
} dg_capture;

/* Temperature sampling of a step (write-up Figure 9, annealed temperature,
 * and Figure 10, temperature 1).  At canvas b with step[b] = t steps taken
 * in its block the temperature is tau_t = tau0 (1 - t / budget) for
 * budget > 0 and tau0 for budget = 0, clamped at 0.  With tau_t > 0 the
 * step's entropy and lse are those of softmax(z / tau_t) and sample holds
 * the Gumbel-max draw argmax_v (z_v / tau_t + g_v): g_v = -ln(-ln u_v),
 * u_v = ((w >> 8) + 0.5) 2^-24 with w word (v mod 4) of Philox4x32-10
 * (Salmon et al., SC'11) of counter (v div 4, position, t, b) and key
 * (low, high 32 bits of seed).  With tau_t = 0: entropy 0, sample = argmax
 * and lse of the raw logits.  argmax stays the raw logits' argmax.  Pass
 * sample as the token candidates of dg_eb_select. */
typedef struct {
  float tau0;            /* 0 or finite >= 1e-6, else DG_ERR_INVALID_ARG */
  int32_t budget;        /* >= 0 */
  uint64_t seed;
  int32_t* sample;       /* [n, 256] drawn token (uncommitted positions only) */
} dg_sampling;

typedef struct {
  float* entropy;        /* [n, 256] nats, >= 0 (uncommitted positions only) */
  float* lse;            /* [n, 256] log-sum-exp of the logits */
  int32_t* argmax;       /* [n, 256] lowest vocab id of the largest logit */
  float* logits;         /* NULL or [n*256, V] fp32 (uncommitted rows only) */
  dg_capture* capture;   /* (host) NULL or capture pointers */
  const dg_sampling* sampling; /* (host) NULL: greedy step */
} dg_step_out;

/* Stage 2 forward (write-up Figure 4, "denoising loop"): embed the n
 * canvases, run every layer (canvas attention over prefix + canvas, MoE),
 * final RMSNorm of the uncommitted rows, tied LM head with a fused
 * log-sum-exp / entropy / argmax epilogue.  Values at committed positions of
 * the outputs are left untouched. */
dg_status dg_denoise_step(dg_ctx* ctx, const dg_canvas_batch* batch,
                          const dg_step_out* out);

/* Entropy-bounded selection (write-up "What they did"; model card "Entropy
 * Bound (EB) sampler"), per canvas over its uncommitted positions U: sort by
 * (entropy, position) ascending; n* = the length of the longest prefix whose
 * fp64 running entropy sum is <= gamma[b], at least 1; all of U when
 * step[b] + 1 >= step_cap (the step budget).  The first n* positions are
 * committed with token = argmax; with refine != 0 the other positions of U
 * take their argmax token too, otherwise they keep theirs.  step[b] += 1,
 * n_new[b] = n*, done[b] = (U now empty).  A canvas whose U is already empty
 * is left unchanged with n_new = 0, done = 1.
 * entropy / argmax: [n, 256] as written by dg_denoise_step; gamma: [n] fp32
 * (device); step_cap in 1..65535; n_new, done: [n] device outputs (any
 * device-accessible memory: done in pinned host memory lets a host loop
 * test it after a stream sync without a copy). */
dg_status dg_eb_select(dg_ctx* ctx, const dg_canvas_batch* batch,
                       const float* entropy, const int32_t* argmax,
                       const float* gamma, int32_t step_cap, int32_t refine,
                       int32_t* n_new, uint8_t* done);

/* Stage 3 (write-up Figure 4, "encode & append"): run the canvas tokens
 * causally (position i sees the cache, the request's earlier canvases of
 * the batch and its own canvas positions <= i) through the layers and write
 * each layer's K/V of the 256 positions into cache rows [kv_len + 256 j,
 * kv_len + 256 (j + 1)) of the canvas's slot, j = the canvas's index among
 * its request's canvases; kv_len += 256 per canvas.
 * DG_ERR_CAPACITY if a request's kv_len + 256 x its canvases > max_kv_len;
 * with DG_CHECK=1, DG_ERR_STATE if a canvas has an uncommitted position. */
dg_status dg_commit_block(dg_ctx* ctx, const dg_canvas_batch* batch);

/* AR mode (write-up "What they did": the same weights still decode left to
 * right; model card "Model Overview"): one causal decoding step for n
 * positions.  tokens [n] int32 (device): position b holds the token at the
 * next position of sequence req[b] (host [n]); positions of one sequence
 * are contiguous and in order (the j-th of them sits at kv_len + j and
 * sees the cache and the sequence's positions before it, like canvases of
 * one position in dg_commit_block).  Each layer's K/V of the n positions
 * are appended to the cache (kv_len += its positions per sequence) and the
 * final-normed rows go through the tied LM head: entropy, lse, argmax [n]
 * of each position's next-token distribution, logits NULL or [n, V].
 * out->capture and out->sampling must be NULL (DG_ERR_UNSUPPORTED).
 * n <= min(64, max_canvases x canvas_len), else DG_ERR_CAPACITY; a cache
 * without room for the positions is DG_ERR_CAPACITY before any launch.
 * Uses the context workspace like dg_denoise_step. */
dg_status dg_ar_step(dg_ctx* ctx, int32_t n, const int32_t* req,
                     const int32_t* tokens, const dg_step_out* out);

/* The stream the context's calls enqueue on from now on (the one given to
 * dg_create until then); the profiler's events are recorded on it too.
 * HIP graphs: dg_denoise_step and dg_eb_select enqueue kernel launches
 * only (no allocation, no host synchronisation, no memset unless
 * DG_POISON; a capture adds device-to-device copies), so a caller may
 * capture them on its own stream (set here first; capture cannot use the
 * legacy null stream) and replay the graph.  A replay reuses the host-side
 * values of the capture: the batch's request slots and kv_len (its key
 * ranges), so a graph holds for the steps of one block; dg_commit_block
 * and dg_ar_step advance kv_len on the host and are not for capture.
 * DG_ERR_INVALID_ARG for a NULL ctx. */
dg_status dg_set_stream(dg_ctx* ctx, void* stream);

dg_status dg_set_kv_len(dg_ctx* ctx, int32_t req, int32_t len);
int32_t dg_kv_len(const dg_ctx* ctx, int32_t req); /* -1 on a bad slot */

/* Instrumentation (not part of the method): per-kernel timing of the
 * context's launches with hipEvents recorded on its stream around every
 * kernel.  dg_profile_enable turns recording on or off (off by default;
 * recording adds a few microseconds per launch).  dg_profile_read waits for
 * the recorded events, writes the summed milliseconds and launch counts per
 * kernel kind into ms[DG_PROF_KINDS] and launches[DG_PROF_KINDS] (host
 * arrays), clears the record and returns 0, 1 if events were dropped
 * because more than 2^20 were recorded between reads, or -1 on error.
 * Kind k is named by dg_profile_kind_name(k).  The denoise step's row
 * compaction runs inside its embedding launch (kind "embed"); kind
 * "compact" counts no launches. */
#define DG_PROF_KINDS 17
dg_status dg_profile_enable(dg_ctx* ctx, int32_t on);
int32_t dg_profile_read(dg_ctx* ctx, float* ms, int32_t* launches);
const char* dg_profile_kind_name(int32_t kind);

const char* dg_status_string(dg_status s);
const char* dg_last_error(const dg_ctx* ctx); /* "" if none; NULL ctx: last
                                                  global error */

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
