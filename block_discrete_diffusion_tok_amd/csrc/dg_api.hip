// Host side of libdg: argument validation, workspace layout, per-layer
// orchestration of the kernels and the extern "C" entry points of dg.h and
// dg_ops.h.  No device memory is allocated here: every buffer comes from the
// caller.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "dg_internal.h"
#include "dg_ops.h"

using namespace dg;

// ------------------------------------------------------------------ errors
static thread_local std::string g_last_error;

// ------------------------------------------------------------------ timing
// Optional per-kernel timing: hipEvents recorded on the context's stream
// around every launch, accumulated per kernel kind when read back.
namespace {
const char* const kKindNames[DG_PROF_KINDS] = {
    "embed",      "rmsnorm",    "qkv_proj", "attention", "o_proj",
    "router",     "topk",       "permute",  "moe_gate_up", "moe_down",
    "unpermute",  "compact",    "lm_head",  "lm_merge",  "eb_select",
    "kv_append",  "kv_install"};
constexpr size_t kMaxEvents = 1 << 20;

struct Profiler {
  bool on = false;
  bool overflow = false;
  hipStream_t s = nullptr;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<int, size_t>> marks;
  hipEvent_t next() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
  ~Profiler() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};

struct ProfScope {
  Profiler* p;
  int kind;
  size_t idx = 0;
  ProfScope(Profiler* prof, int k) : p(nullptr), kind(k) {
    if (prof && prof->on && prof->used + 2 <= kMaxEvents) {
      p = prof;
      idx = p->used;
      hipEvent_t e = p->next();
      if (!e) { p = nullptr; return; }
      (void)hipEventRecord(e, p->s);
    } else if (prof && prof->on) {
      prof->overflow = true;
    }
  }
  ~ProfScope() {
    if (!p) return;
    hipEvent_t e = p->next();
    if (!e) return;
    (void)hipEventRecord(e, p->s);
    p->marks.push_back({kind, idx});
  }
};
}  // namespace

// Workspace of the MoE pipeline (carved by moe_layout).
struct MoeBufs {
  float* rlogits;
  int32_t* ridx;
  float* rw;
  int32_t* chunk_counts;
  int32_t* local_rank;
  int32_t* chunk_base;
  int32_t* offsets;
  int32_t* tile_offsets;
  int32_t* perm;
  uint16_t* act;
  float* y;
  // weight-streaming path: fixed-capacity expert slots filled by top-k
  int cap;              // slots per expert (0: the path is never taken)
  int32_t* counts;      // [E] tokens per expert (zeroed before the top-k)
  int32_t* slot_pair;   // [E*cap] pair index t*k + r of each slot
  float* slot_w;        // [E*cap] gate weight of each slot
  int32_t* slot_tok;    // [E*cap + kSlotPad] token of each slot
};
// slot_tok is read up to one pass of 32 slots past an expert's last slot
constexpr int kSlotPad = 64;

struct dg_ctx {
  dg_model_desc d;
  const uint16_t* embed;
  const float* final_norm;
  std::vector<dg_layer_weights> layers;
  int max_requests, max_kv_len, max_canvases;
  uint16_t* k_cache;
  uint16_t* v_cache;
  char* ws;
  size_t ws_bytes;
  hipStream_t stream;
  std::vector<int32_t> kv_len;
  std::string last_error;
  Profiler prof;
  // workspace carve-up
  float* x;
  uint16_t* xh;
  uint16_t* qkv;
  uint16_t* attn;
  float* opart;
  float* lpart;
  MoeBufs moe;
  int32_t* row_map;
  int32_t* pos_map;
  int32_t* m_dev;
  float4* lm_part;
};

static dg_status fail(dg_ctx* c, dg_status s, const std::string& msg) {
  g_last_error = msg;
  if (c) c->last_error = msg;
  return s;
}

// DG_DEBUG_SYNC=1 in the environment (read once per process): every HIP
// call the library checks is followed by a device synchronisation, so an
// asynchronous device fault is reported (DG_ERR_HIP, naming the call) by
// the entry point that launched the faulting kernel rather than at a later
// synchronisation of the caller's.
bool debug_sync() {
  static const bool on = [] {
    const char* v = getenv("DG_DEBUG_SYNC");
    return v && v[0] == '1';
  }();
  return on;
}

#define HIPCHK(ctx, expr)                                                    \
  do {                                                                       \
    hipError_t e_ = (expr);                                                  \
    if (e_ == hipSuccess && debug_sync()) e_ = hipDeviceSynchronize();       \
    if (e_ != hipSuccess)                                                    \
      return fail(ctx, DG_ERR_HIP, std::string(#expr ": ") +                 \
                                       hipGetErrorString(e_));               \
  } while (0)

// HIPCHK plus a timing scope of the given kernel kind.
#define KRUN(ctx, kind, expr)                                                \
  do {                                                                       \
    ProfScope ps_(&(ctx)->prof, kind);                                       \
    HIPCHK(ctx, expr);                                                       \
  } while (0)

// ------------------------------------------------------------------ layout
namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + std::max<size_t>(bytes, 1));
    return o;
  }
};

int lm_tiles(int vocab) { return (vocab + gemm_bn(EPI_LMSTATS) - 1) / gemm_bn(EPI_LMSTATS); }

// Largest splits(n) * n over batches 1..max_canvases (attention partials).
long long attn_split_rows(const dg_model_desc& d, int max_canvases) {
  long long best = 0;
  for (int n = 1; n <= max_canvases; ++n)
    best = std::max<long long>(
        best, (long long)attention_auto_splits(n, DG_CANVAS, d.n_q_heads,
                                               d.n_kv_heads, 0) * n);
  return best;
}


// Router logits are computed in up to kRouterSlabs K splits, each writing
// its own fp32 slab [T, E]; the top-k kernel adds them in order.
constexpr int kRouterSlabs = 8;
int router_splits(int K) {
  const int steps = K / 64;
  int s = 1;
  while (s * 2 <= kRouterSlabs && steps % (s * 2) == 0 && steps / (s * 2) >= 2) s *= 2;
  return s;
}

// Weight-streaming kernels when the expert matrices see few rows each (a
// batch of a few canvases): on average at most 32 (token, expert) pairs per
// expert, and K dimensions that are multiples of the streaming K chunk.
bool use_stream_moe(const dg_model_desc& d, int T) {
  const long long pairs = (long long)T * d.top_k;
  return pairs <= 32LL * d.n_experts && stream_moe_ok(d.hidden, d.expert_ffn);
}

// Workspace of the MoE pipeline for T tokens.
size_t moe_layout(const dg_model_desc& d, int T, char* base, MoeBufs* b) {
  Carve cv;
  const long long pairs = (long long)T * d.top_k;
  const int nc = permute_chunks((int)pairs);
  // slots per expert for the streaming path: every T it is taken for
  // (a token picks an expert at most once, so T slots always suffice)
  const int cap = stream_moe_ok(d.hidden, d.expert_ffn)
                      ? (int)std::min<long long>(T, 32LL * d.n_experts / d.top_k)
                      : 0;
  const long long slots = (long long)d.n_experts * cap;
  const size_t o_rl = cv.take((size_t)kRouterSlabs * T * d.n_experts * 4);
  const size_t o_ri = cv.take((size_t)pairs * 4);
  const size_t o_rw = cv.take((size_t)pairs * 4);
  const size_t o_cc = cv.take((size_t)nc * d.n_experts * 4);
  const size_t o_lr = cv.take((size_t)pairs * 4);
  const size_t o_cb = cv.take((size_t)nc * d.n_experts * 4);
  const size_t o_of = cv.take((size_t)(d.n_experts + 1) * 4);
  const size_t o_to = cv.take((size_t)(d.n_experts + 1) * 4);
  const size_t o_pm = cv.take((size_t)pairs * 4);
  const size_t o_ac = cv.take((size_t)std::max(pairs, slots) * d.expert_ffn * 2);
  const size_t o_y = cv.take((size_t)pairs * d.hidden * 4);
  const size_t o_cn = cv.take((size_t)d.n_experts * 4);
  const size_t o_sp = cv.take((size_t)slots * 4);
  const size_t o_sw = cv.take((size_t)slots * 4);
  const size_t o_st = cv.take((size_t)(slots + kSlotPad) * 4);
  if (b) {
    b->rlogits = (float*)(base + o_rl);
    b->ridx = (int32_t*)(base + o_ri);
    b->rw = (float*)(base + o_rw);
    b->chunk_counts = (int32_t*)(base + o_cc);
    b->local_rank = (int32_t*)(base + o_lr);
    b->chunk_base = (int32_t*)(base + o_cb);
    b->offsets = (int32_t*)(base + o_of);
    b->tile_offsets = (int32_t*)(base + o_to);
    b->perm = (int32_t*)(base + o_pm);
    b->act = (uint16_t*)(base + o_ac);
    b->y = (float*)(base + o_y);
    b->cap = cap;
    b->counts = (int32_t*)(base + o_cn);
    b->slot_pair = (int32_t*)(base + o_sp);
    b->slot_w = (float*)(base + o_sw);
    b->slot_tok = (int32_t*)(base + o_st);
  }
  return cv.off;
}

size_t ctx_layout(const dg_model_desc& d, int max_canvases, dg_ctx* c) {
  const long long T = (long long)max_canvases * DG_CANVAS;
  const int qkvN = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim;
  const long long split_rows = attn_split_rows(d, max_canvases) * d.n_q_heads * DG_CANVAS;
  Carve cv;
  const size_t o_x = cv.take(T * d.hidden * 4);
  const size_t o_xh = cv.take(T * d.hidden * 2);
  const size_t o_qkv = cv.take(T * qkvN * 2);
  const size_t o_at = cv.take(T * d.n_q_heads * d.head_dim * 2);
  const size_t o_op = cv.take(split_rows * d.head_dim * 4);
  const size_t o_lp = cv.take(split_rows * 4);
  const size_t o_rm = cv.take(T * 4);
  const size_t o_pm = cv.take(T * 4);
  const size_t o_md = cv.take(4);
  const size_t o_lm = cv.take(T * lm_tiles(d.vocab) * 16);
  const size_t o_moe = cv.take(moe_layout(d, (int)T, nullptr, nullptr));
  if (c) {
    char* w = c->ws;
    c->x = (float*)(w + o_x);
    c->xh = (uint16_t*)(w + o_xh);
    c->qkv = (uint16_t*)(w + o_qkv);
    c->attn = (uint16_t*)(w + o_at);
    c->opart = (float*)(w + o_op);
    c->lpart = (float*)(w + o_lp);
    c->row_map = (int32_t*)(w + o_rm);
    c->pos_map = (int32_t*)(w + o_pm);
    c->m_dev = (int32_t*)(w + o_md);
    c->lm_part = (float4*)(w + o_lm);
    moe_layout(d, (int)T, w + o_moe, &c->moe);
  }
  return cv.off;
}

std::string check_desc(const dg_model_desc* d) {
  if (!d) return "desc is NULL";
  if (d->n_layers < 1) return "n_layers must be >= 1";
  if (d->head_dim != 64 && d->head_dim != 128) return "head_dim must be 64 or 128";
  if (d->n_kv_heads < 1 || d->n_q_heads < d->n_kv_heads ||
      d->n_q_heads % d->n_kv_heads)
    return "n_q_heads must be a positive multiple of n_kv_heads";
  if (d->hidden < 64 || d->hidden % 64) return "hidden must be a multiple of 64";
  if ((d->n_q_heads * d->head_dim) % 64) return "n_q_heads*head_dim must be a multiple of 64";
  if (d->n_experts < 1 || d->n_experts > 256) return "n_experts must be in 1..256";
  if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->n_experts)
    return "top_k must be in 1..min(16, n_experts)";
  if (d->expert_ffn < 64 || d->expert_ffn % 64) return "expert_ffn must be a multiple of 64";
  if (d->vocab < 1) return "vocab must be >= 1";
  if (!(d->rms_eps >= 0.f)) return "rms_eps must be >= 0";
  if (d->expert_dtype != DG_BF16 && d->expert_dtype != DG_FP8_E4M3)
    return "expert_dtype must be DG_BF16 or DG_FP8_E4M3";
  return "";
}

std::string check_layer(const dg_model_desc& d, const dg_layer_weights& w,
                        bool moe_only) {
  if (!moe_only && (!w.attn_norm || !w.w_qkv || !w.w_o || !w.ffn_norm))
    return "layer attention weights must not be NULL";
  if (!w.w_router || !w.w_gate_up || !w.w_down)
    return "layer MoE weights must not be NULL";
  if (d.expert_dtype == DG_FP8_E4M3 && (!w.gate_up_scale || !w.down_scale))
    return "e4m3 experts need gate_up_scale and down_scale";
  return "";
}

GemmArgs gemm_dense(const uint16_t* A, int M, int K, const void* W, int N,
                    void* C, int ldc) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.A = A;
  g.lda = K;
  g.a_map_div = 1;
  g.B = W;
  g.M = M;
  g.N = N;
  g.K = K;
  g.C = C;
  g.ldc = ldc;
  return g;
}

int grid_m_dense(int M, int epi) { return (M + gemm_bm(epi) - 1) / gemm_bm(epi); }


// The LM head streams the tied embedding once per 128 rows; beyond 256 rows
// the tiled kernel reuses it better.
bool use_stream_lm(int rows, int hidden) {
  return rows <= 256 && stream_lm_ok(hidden);
}

// Run the LM head with the vocabulary statistics epilogue; returns the
// number of partials per row written to part.
hipError_t run_lm_head(const uint16_t* xh, int rows_max, const int32_t* m_dev,
                       int hidden, const void* embed, int vocab, float4* part,
                       float* logits, const int32_t* row_map, int* n_tiles,
                       hipStream_t s) {
  if (use_stream_lm(rows_max, hidden)) {
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.X = xh;
    a.ldx = hidden;
    a.W = embed;
    a.M = rows_max;
    a.M_dev = m_dev;
    a.N = vocab;
    a.K = hidden;
    a.part = part;
    a.n_tiles = (vocab + stream_rows_per_wg() - 1) / stream_rows_per_wg();
    a.logits = logits;
    a.row_map = row_map;
    *n_tiles = a.n_tiles;
    return launch_stream(EPI_LMSTATS, false, a, 1, s);
  }
  GemmArgs g = gemm_dense(xh, rows_max, hidden, embed, vocab, nullptr, 0);
  g.M_dev = m_dev;
  g.part = part;
  g.n_tiles = (vocab + gemm_bn(EPI_LMSTATS) - 1) / gemm_bn(EPI_LMSTATS);
  g.logits = logits;
  g.row_map = row_map;
  *n_tiles = g.n_tiles;
  return launch_gemm(EPI_LMSTATS, false, g, grid_m_dense(rows_max, EPI_LMSTATS), s);
}

// MoE FFN on xh [T, H] bf16: y mixture added into x (if x) and/or stored
// into moe_out (if moe_out).
// With next_g, the un-permute also applies the next RMSNorm (gain next_g)
// into next_xh (rows mapped by next_row, see launch_unpermute_norm).
// counts_zeroed: b.counts was cleared by an earlier kernel on the stream
// (the FFN RMSNorm of the layer); otherwise it is cleared here.
hipError_t run_moe(const dg_model_desc& d, const dg_layer_weights& w,
                   const uint16_t* xh, int T, const MoeBufs& b, float* x,
                   float* moe_out, int32_t* counts, hipStream_t s,
                   Profiler* prof = nullptr, const float* next_g = nullptr,
                   uint16_t* next_xh = nullptr, float* next_copy = nullptr,
                   const int32_t* next_row = nullptr, bool counts_zeroed = false) {
  const int H = d.hidden, E = d.n_experts, k = d.top_k, F = d.expert_ffn;
  const bool w8 = d.expert_dtype == DG_FP8_E4M3;
  const int pairs = T * k;
  hipError_t e;
  GemmArgs r = gemm_dense(xh, T, H, w.w_router, E, b.rlogits, E);
  r.splits = router_splits(H);
  r.split_stride = (long long)T * E;
  {
    ProfScope ps(prof, 5);
    if ((e = launch_gemm(EPI_STORE_F32, false, r, grid_m_dense(T, EPI_STORE_F32), s)) != hipSuccess) return e;
  }
  if (use_stream_moe(d, T)) {
    // Weight-streaming path: top-k hands every (token, rank) pair a slot of
    // its expert (fixed rows e*cap + i), so a GEMM workgroup finds its
    // tokens with one lookup and no prefix sum.
    if (T > b.cap) return hipErrorInvalidValue;
    if (!counts_zeroed && (e = launch_zero_i32(b.counts, E, s)) != hipSuccess) return e;
    {
      ProfScope ps(prof, 6);
      if ((e = launch_topk_slots(b.rlogits, T, E, k, r.splits, b.ridx, b.rw, b.counts,
                                 b.cap, b.slot_pair, b.slot_w, b.slot_tok, s)) != hipSuccess)
        return e;
    }
    if (counts &&
        (e = hipMemcpyAsync(counts, b.counts, (size_t)E * 4, hipMemcpyDeviceToDevice, s)) !=
            hipSuccess)
      return e;
    StreamArgs gu;
    memset(&gu, 0, sizeof(gu));
    gu.X = xh;
    gu.ldx = H;
    gu.M = T;
    gu.row_of = b.slot_tok;
    gu.W = w.w_gate_up;
    gu.w_group_stride = (long long)2 * F * H;
    gu.w_scale = w.gate_up_scale;
    gu.scale_rows = 2 * F;
    gu.N = 2 * F;
    gu.K = H;
    gu.group_count = b.counts;
    gu.cap = b.cap;
    gu.C = b.act;
    gu.ldc = F;
    gu.ffn = F;
    {
      ProfScope ps(prof, 8);
      if ((e = launch_stream(EPI_SWIGLU, w8, gu, E, s)) != hipSuccess) return e;
    }
    StreamArgs dn;
    memset(&dn, 0, sizeof(dn));
    dn.X = b.act;
    dn.ldx = F;
    dn.W = w.w_down;
    dn.w_group_stride = (long long)H * F;
    dn.w_scale = w.down_scale;
    dn.scale_rows = H;
    dn.N = H;
    dn.K = F;
    dn.group_count = b.counts;
    dn.cap = b.cap;
    dn.C = b.y;
    dn.ldc = H;
    dn.c_map = b.slot_pair;
    dn.row_scale = b.slot_w;
    {
      ProfScope ps(prof, 9);
      if ((e = launch_stream(EPI_DOWN, w8, dn, E, s)) != hipSuccess) return e;
    }
    ProfScope ps10(prof, 10);
    if (next_g)
      return launch_unpermute_norm(b.y, T, k, H, x, moe_out, next_g, d.rms_eps,
                                   next_xh, next_copy, next_row, s);
    return launch_unpermute(b.y, T, k, H, x, moe_out, s);
  }
  {
    ProfScope ps(prof, 6);
    if ((e = launch_topk(b.rlogits, T, E, k, r.splits, b.ridx, b.rw, s)) != hipSuccess) return e;
  }
  {
    ProfScope ps(prof, 7);
    if ((e = launch_permute(b.ridx, pairs, E, kGroupBM, b.chunk_counts,
                            b.local_rank, b.chunk_base, b.offsets,
                            b.tile_offsets, counts, b.perm, s)) != hipSuccess)
      return e;
  }
  const int grid_m = (pairs + kGroupBM - 1) / kGroupBM + std::min(E, pairs);
  GemmArgs gu = gemm_dense(xh, pairs, H, w.w_gate_up, 2 * F, b.act, F);
  gu.a_map = b.perm;
  gu.a_map_div = k;
  gu.b_group_stride = (long long)2 * F * H;
  gu.b_scale = w.gate_up_scale;
  gu.scale_rows = 2 * F;
  gu.n_groups = E;
  gu.group_offsets = b.offsets;
  gu.tile_offsets = b.tile_offsets;
  gu.ffn = F;
  {
    ProfScope ps(prof, 8);
    if ((e = launch_gemm(EPI_SWIGLU, w8, gu, grid_m, s)) != hipSuccess) return e;
  }
  GemmArgs dn = gemm_dense(b.act, pairs, F, w.w_down, H, b.y, H);
  dn.b_group_stride = (long long)H * F;
  dn.b_scale = w.down_scale;
  dn.scale_rows = H;
  dn.n_groups = E;
  dn.group_offsets = b.offsets;
  dn.tile_offsets = b.tile_offsets;
  dn.c_map = b.perm;
  dn.row_scale = b.rw;
  {
    ProfScope ps(prof, 9);
    if ((e = launch_gemm(EPI_DOWN, w8, dn, grid_m, s)) != hipSuccess) return e;
  }
  ProfScope ps10(prof, 10);
  if (next_g)
    return launch_unpermute_norm(b.y, T, k, H, x, moe_out, next_g, d.rms_eps,
                                 next_xh, next_copy, next_row, s);
  return launch_unpermute(b.y, T, k, H, x, moe_out, s);
}

const MoeBufs& ctx_moe_bufs(const dg_ctx* c) { return c->moe; }

dg_status check_batch(dg_ctx* c, const dg_canvas_batch* bt, bool distinct) {
  if (!bt) return fail(c, DG_ERR_INVALID_ARG, "batch is NULL");
  if (bt->n < 1 || bt->n > c->max_canvases)
    return fail(c, DG_ERR_CAPACITY, "batch size outside 1..max_canvases");
  if (!bt->req || !bt->tokens || !bt->committed || !bt->step)
    return fail(c, DG_ERR_INVALID_ARG, "batch pointers must not be NULL");
  for (int b = 0; b < bt->n; ++b) {
    const int r = bt->req[b];
    if (r < 0 || r >= c->max_requests)
      return fail(c, DG_ERR_INVALID_ARG, "request slot out of range");
    if (distinct)
      for (int q = 0; q < b; ++q)
        if (bt->req[q] == r)
          return fail(c, DG_ERR_INVALID_ARG, "request slots must be distinct");
  }
  return DG_OK;
}

// One decoder layer over the canvas rows in c->x, whose attention RMSNorm
// is already in c->xh (made by the embedding or the previous layer's
// un-permute).  The layer's un-permute makes the next layer's normed input,
// or after the last layer of a denoise step the final-norm rows of the
// uncommitted positions in compacted order (c->pos_map).  commit: write the
// layer's canvas K/V into the cache first, causal attention, and stop after
// the K/V of the last layer.
dg_status run_layer(dg_ctx* c, int l, int n, const int* req, const int* plen,
                    bool commit, const dg_capture* cap) {
  const dg_model_desc& d = c->d;
  const dg_layer_weights& w = c->layers[l];
  const int T = n * DG_CANVAS, H = d.hidden, D = d.head_dim;
  const int Hq = d.n_q_heads, Hkv = d.n_kv_heads;
  const int qkvN = (Hq + 2 * Hkv) * D;
  const long long head_stride = (long long)c->max_kv_len * D;
  const long long req_stride = (long long)Hkv * head_stride;
  const long long layer_stride = (long long)c->max_requests * req_stride;
  hipStream_t s = c->stream;
  GemmArgs g = gemm_dense(c->xh, T, H, w.w_qkv, qkvN, c->qkv, qkvN);
  KRUN(c, 2, launch_gemm(EPI_STORE_BF16, false, g, grid_m_dense(T, EPI_STORE_BF16), s));
  uint16_t* kc = c->k_cache + l * layer_stride;
  uint16_t* vc = c->v_cache + l * layer_stride;
  if (commit) {
    KRUN(c, 15, launch_kv_append(c->qkv, qkvN, Hq * D, (Hq + Hkv) * D, n,
                               DG_CANVAS, Hkv, D, kc, vc, req_stride,
                               head_stride, req, plen, s));
    if (l == d.n_layers - 1) return DG_OK;
  }
  AttnArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.qkv = c->qkv;
  aa.ldqkv = qkvN;
  aa.C = DG_CANVAS;
  aa.Hq = Hq;
  aa.Hkv = Hkv;
  aa.D = D;
  aa.kc = kc;
  aa.vc = vc;
  aa.req_stride = req_stride;
  aa.head_stride = head_stride;
  for (int b = 0; b < n; ++b) {
    aa.req[b] = req[b];
    aa.plen[b] = plen[b];
  }
  aa.n = n;
  int max_keys = 0;
  for (int b = 0; b < n; ++b) max_keys = std::max(max_keys, plen[b] + DG_CANVAS);
  aa.splits = attention_auto_splits(n, DG_CANVAS, Hq, Hkv, max_keys);
  aa.causal = commit ? 1 : 0;
  aa.out = c->attn;
  aa.opart = c->opart;
  aa.lpart = c->lpart;
  KRUN(c, 3, launch_attention(aa, s));
  if (cap && cap->attn_out)
    HIPCHK(c, hipMemcpyAsync((char*)cap->attn_out + (size_t)l * T * Hq * D * 2,
                             c->attn, (size_t)T * Hq * D * 2,
                             hipMemcpyDeviceToDevice, s));
  GemmArgs o = gemm_dense(c->attn, T, Hq * D, w.w_o, H, c->x, H);
  KRUN(c, 4, launch_gemm(EPI_ADD_F32, false, o, grid_m_dense(T, EPI_ADD_F32), s));
  const MoeBufs& mb = ctx_moe_bufs(c);
  KRUN(c, 1, launch_rmsnorm(c->x, T, H, w.ffn_norm, d.rms_eps, c->xh, nullptr,
                           nullptr, nullptr, s, mb.counts, d.n_experts));
  float* moe_out = (cap && cap->moe_out) ? cap->moe_out + (size_t)l * T * H : nullptr;
  const bool last = l == d.n_layers - 1;
  const float* next_g = last ? c->final_norm : c->layers[l + 1].attn_norm;
  float* next_copy = (last && cap && cap->final_xhat) ? cap->final_xhat : nullptr;
  HIPCHK(c, run_moe(d, w, c->xh, T, mb, c->x, moe_out, nullptr, s, &c->prof, next_g,
                    c->xh, next_copy, last ? c->pos_map : nullptr, true));
  if (cap) {
    const size_t tk = (size_t)T * d.top_k;
    if (cap->route_idx)
      HIPCHK(c, hipMemcpyAsync(cap->route_idx + l * tk, mb.ridx, tk * 4,
                               hipMemcpyDeviceToDevice, s));
    if (cap->route_w)
      HIPCHK(c, hipMemcpyAsync(cap->route_w + l * tk, mb.rw, tk * 4,
                               hipMemcpyDeviceToDevice, s));
    if (cap->router_logits)
      HIPCHK(c, hipMemcpyAsync(cap->router_logits + (size_t)l * T * d.n_experts,
                               mb.rlogits, (size_t)T * d.n_experts * 4,
                               hipMemcpyDeviceToDevice, s));
  }
  return DG_OK;
}

}  // namespace

// ------------------------------------------------------------------ dg.h
extern "C" {

const char* dg_status_string(dg_status s) {
  switch (s) {
    case DG_OK: return "DG_OK";
    case DG_ERR_INVALID_ARG: return "DG_ERR_INVALID_ARG";
    case DG_ERR_SHAPE: return "DG_ERR_SHAPE";
    case DG_ERR_CAPACITY: return "DG_ERR_CAPACITY";
    case DG_ERR_STATE: return "DG_ERR_STATE";
    case DG_ERR_HIP: return "DG_ERR_HIP";
    case DG_ERR_UNSUPPORTED: return "DG_ERR_UNSUPPORTED";
  }
  return "unknown dg_status";
}

const char* dg_last_error(const dg_ctx* c) {
  return c ? c->last_error.c_str() : g_last_error.c_str();
}

size_t dg_workspace_bytes(const dg_model_desc* d, int32_t max_canvases) {
  if (!check_desc(d).empty() || max_canvases < 1 || max_canvases > DG_MAX_BATCH)
    return 0;
  return ctx_layout(*d, max_canvases, nullptr);
}

size_t dg_kv_cache_bytes(const dg_model_desc* d, int32_t max_requests,
                         int32_t max_kv_len) {
  if (!check_desc(d).empty() || max_requests < 1 || max_kv_len < 1) return 0;
  return (size_t)d->n_layers * max_requests * d->n_kv_heads * max_kv_len *
         d->head_dim * 2;
}

size_t dg_packed_bytes(int32_t groups, int32_t rows, int32_t cols, int32_t dtype) {
  if (dtype != DG_BF16 && dtype != DG_FP8_E4M3) return 0;
  const int esz = dtype == DG_BF16 ? 2 : 1;
  if (groups < 1 || rows < 1 || cols < 1 || cols % pack_k(esz)) return 0;
  if (groups > 1 && rows % kPackRows) return 0;
  return (size_t)groups * ((rows + kPackRows - 1) / kPackRows * kPackRows) * cols * esz;
}

dg_status dg_pack_weights(const void* src, int32_t groups, int32_t rows,
                          int32_t cols, int32_t dtype, void* dst, void* stream) {
  if (!src || !dst) return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (dtype != DG_BF16 && dtype != DG_FP8_E4M3)
    return fail(nullptr, DG_ERR_INVALID_ARG, "dtype must be DG_BF16 or DG_FP8_E4M3");
  if (dg_packed_bytes(groups, rows, cols, dtype) == 0)
    return fail(nullptr, DG_ERR_SHAPE,
                "cols must be a multiple of 32 (bf16) or 64 (e4m3), rows per group a "
                "multiple of 64 when groups > 1");
  HIPCHK(nullptr, launch_pack(src, groups, rows, cols, dtype == DG_BF16 ? 2 : 1, dst,
                              (hipStream_t)stream));
  return DG_OK;
}

dg_status dg_create(const dg_model_desc* desc, const dg_weights* weights,
                    int32_t max_requests, int32_t max_kv_len,
                    int32_t max_canvases, void* k_cache, void* v_cache,
                    void* workspace, size_t workspace_bytes, void* stream,
                    dg_ctx** out) {
  if (!out) return fail(nullptr, DG_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  const std::string de = check_desc(desc);
  if (!de.empty()) return fail(nullptr, DG_ERR_SHAPE, de);
  if (!weights || !weights->embed || !weights->final_norm || !weights->layers)
    return fail(nullptr, DG_ERR_INVALID_ARG, "weights must not be NULL");
  for (int l = 0; l < desc->n_layers; ++l) {
    const std::string le = check_layer(*desc, weights->layers[l], false);
    if (!le.empty()) return fail(nullptr, DG_ERR_INVALID_ARG, le);
  }
  if (max_requests < 1 || max_kv_len < DG_CANVAS)
    return fail(nullptr, DG_ERR_INVALID_ARG,
                "max_requests must be >= 1 and max_kv_len >= 256");
  if (max_canvases < 1 || max_canvases > DG_MAX_BATCH || max_canvases > max_requests)
    return fail(nullptr, DG_ERR_INVALID_ARG,
                "max_canvases must be in 1..min(64, max_requests)");
  if (!k_cache || !v_cache || !workspace)
    return fail(nullptr, DG_ERR_INVALID_ARG, "cache and workspace must not be NULL");
  if (((uintptr_t)workspace % kAlign) != 0)
    return fail(nullptr, DG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t need = ctx_layout(*desc, max_canvases, nullptr);
  if (workspace_bytes < need)
    return fail(nullptr, DG_ERR_CAPACITY, "workspace too small");
  dg_ctx* c = new (std::nothrow) dg_ctx();
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "out of host memory");
  c->d = *desc;
  c->embed = (const uint16_t*)weights->embed;
  c->final_norm = weights->final_norm;
  c->layers.assign(weights->layers, weights->layers + desc->n_layers);
  c->max_requests = max_requests;
  c->max_kv_len = max_kv_len;
  c->max_canvases = max_canvases;
  c->k_cache = (uint16_t*)k_cache;
  c->v_cache = (uint16_t*)v_cache;
  c->ws = (char*)workspace;
  c->ws_bytes = workspace_bytes;
  c->stream = (hipStream_t)stream;
  c->kv_len.assign(max_requests, 0);
  c->prof.s = c->stream;
  ctx_layout(*desc, max_canvases, c);
  *out = c;
  return DG_OK;
}

void dg_destroy(dg_ctx* c) { delete c; }

dg_status dg_profile_enable(dg_ctx* c, int32_t on) {
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  c->prof.on = on != 0;
  return DG_OK;
}

int32_t dg_profile_read(dg_ctx* c, float* ms, int32_t* launches) {
  if (!c || !ms || !launches) return -1;
  for (int k = 0; k < DG_PROF_KINDS; ++k) {
    ms[k] = 0.f;
    launches[k] = 0;
  }
  Profiler& p = c->prof;
  if (p.used > 0 && hipEventSynchronize(p.pool[p.used - 1]) != hipSuccess) {
    fail(c, DG_ERR_HIP, "hipEventSynchronize failed in dg_profile_read");
    return -1;
  }
  for (const auto& m : p.marks) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, p.pool[m.second], p.pool[m.second + 1]) == hipSuccess) {
      ms[m.first] += t;
      launches[m.first] += 1;
    }
  }
  const int32_t overflow = p.overflow ? 1 : 0;
  p.used = 0;
  p.marks.clear();
  p.overflow = false;
  return overflow;
}

const char* dg_profile_kind_name(int32_t kind) {
  return (kind >= 0 && kind < DG_PROF_KINDS) ? kKindNames[kind] : "";
}

dg_status dg_set_kv_len(dg_ctx* c, int32_t req, int32_t len) {
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  if (req < 0 || req >= c->max_requests)
    return fail(c, DG_ERR_INVALID_ARG, "request slot out of range");
  if (len < 0 || len > c->max_kv_len)
    return fail(c, DG_ERR_CAPACITY, "kv_len outside 0..max_kv_len");
  c->kv_len[req] = len;
  return DG_OK;
}

int32_t dg_kv_len(const dg_ctx* c, int32_t req) {
  if (!c || req < 0 || req >= c->max_requests) return -1;
  return c->kv_len[req];
}

dg_status dg_prefill_kv(dg_ctx* c, int32_t req, int32_t n,
                        const int32_t* tokens, const void* k, const void* v) {
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  if (tokens) {
    if (k || v) return fail(c, DG_ERR_INVALID_ARG, "give either tokens or k/v");
    return fail(c, DG_ERR_UNSUPPORTED, "token-mode prefill is not provided");
  }
  if (!k || !v) return fail(c, DG_ERR_INVALID_ARG, "k and v must not be NULL");
  if (req < 0 || req >= c->max_requests)
    return fail(c, DG_ERR_INVALID_ARG, "request slot out of range");
  if (n < 0 || n > c->max_kv_len)
    return fail(c, DG_ERR_CAPACITY, "prefix longer than max_kv_len");
  const dg_model_desc& d = c->d;
  const long long head_stride = (long long)c->max_kv_len * d.head_dim;
  const long long req_stride = (long long)d.n_kv_heads * head_stride;
  const long long layer_stride = (long long)c->max_requests * req_stride;
  const long long src_layer = (long long)d.n_kv_heads * n * d.head_dim;
  for (int l = 0; l < d.n_layers; ++l) {
    const long long dst = l * layer_stride + req * req_stride;
    KRUN(c, 16, launch_kv_install((const uint16_t*)k + l * src_layer,
                                d.n_kv_heads, n, d.head_dim, c->k_cache + dst,
                                head_stride, c->stream));
    KRUN(c, 16, launch_kv_install((const uint16_t*)v + l * src_layer,
                                d.n_kv_heads, n, d.head_dim, c->v_cache + dst,
                                head_stride, c->stream));
  }
  c->kv_len[req] = n;
  return DG_OK;
}

dg_status dg_denoise_step(dg_ctx* c, const dg_canvas_batch* bt,
                          const dg_step_out* out) {
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(c, bt, false);
  if (st != DG_OK) return st;
  if (!out || !out->entropy || !out->lse || !out->argmax)
    return fail(c, DG_ERR_INVALID_ARG, "step outputs must not be NULL");
  const dg_model_desc& d = c->d;
  const int n = bt->n, T = n * DG_CANVAS, H = d.hidden;
  int req[DG_MAX_BATCH], plen[DG_MAX_BATCH];
  for (int b = 0; b < n; ++b) {
    req[b] = bt->req[b];
    plen[b] = c->kv_len[req[b]];
  }
  hipStream_t s = c->stream;
  KRUN(c, 0, launch_embed_norm(bt->tokens, T, c->embed, d.vocab, H, c->x,
                               c->layers[0].attn_norm, d.rms_eps, c->xh, s, bt->committed,
                               c->row_map, c->m_dev, c->pos_map));
  for (int l = 0; l < d.n_layers; ++l) {
    st = run_layer(c, l, n, req, plen, false, out->capture);
    if (st != DG_OK) return st;
  }
  int n_tiles = 0;
  KRUN(c, 12, run_lm_head(c->xh, T, c->m_dev, H, c->embed, d.vocab, c->lm_part,
                          out->logits, c->row_map, &n_tiles, s));
  KRUN(c, 13, launch_lm_merge(c->lm_part, n_tiles, c->m_dev, T, c->row_map,
                            out->entropy, out->lse, out->argmax, s));
  return DG_OK;
}

dg_status dg_eb_select(dg_ctx* c, const dg_canvas_batch* bt,
                       const float* entropy, const int32_t* argmax,
                       const float* gamma, int32_t step_cap, int32_t refine,
                       int32_t* n_new, uint8_t* done) {
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(c, bt, false);
  if (st != DG_OK) return st;
  if (!entropy || !argmax || !gamma || !n_new || !done)
    return fail(c, DG_ERR_INVALID_ARG, "sampler pointers must not be NULL");
  if (step_cap < 1 || step_cap > 65535)
    return fail(c, DG_ERR_INVALID_ARG, "step_cap must be in 1..65535");
  KRUN(c, 14, launch_eb_select(bt->n, entropy, argmax, bt->committed, bt->tokens,
                             bt->step, gamma, step_cap, refine, n_new, done,
                             c->stream));
  return DG_OK;
}

dg_status dg_commit_block(dg_ctx* c, const dg_canvas_batch* bt) {
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(c, bt, true);
  if (st != DG_OK) return st;
  const int n = bt->n, T = n * DG_CANVAS;
  int req[DG_MAX_BATCH], plen[DG_MAX_BATCH];
  for (int b = 0; b < n; ++b) {
    req[b] = bt->req[b];
    plen[b] = c->kv_len[req[b]];
    if (plen[b] + DG_CANVAS > c->max_kv_len)
      return fail(c, DG_ERR_CAPACITY, "KV cache full: kv_len + 256 > max_kv_len");
  }
  KRUN(c, 0, launch_embed_norm(bt->tokens, T, c->embed, c->d.vocab, c->d.hidden, c->x,
                               c->layers[0].attn_norm, c->d.rms_eps, c->xh, c->stream));
  for (int l = 0; l < c->d.n_layers; ++l) {
    st = run_layer(c, l, n, req, plen, true, nullptr);
    if (st != DG_OK) return st;
  }
  for (int b = 0; b < n; ++b) c->kv_len[req[b]] += DG_CANVAS;
  return DG_OK;
}

// ------------------------------------------------------------------ dg_ops.h

dg_status dg_op_rmsnorm(const float* x, int32_t rows, int32_t hidden,
                        const float* g, float eps, void* out, void* stream) {
  if (!x || !g || !out) return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (rows < 0 || hidden < 4 || hidden % 4)
    return fail(nullptr, DG_ERR_SHAPE, "hidden must be a positive multiple of 4");
  HIPCHK(nullptr, launch_rmsnorm(x, rows, hidden, g, eps, (uint16_t*)out,
                                 nullptr, nullptr, nullptr, (hipStream_t)stream));
  return DG_OK;
}

dg_status dg_op_linear(const void* x, int32_t m, int32_t k, const void* w,
                       int32_t n, int32_t mode, void* out, void* stream) {
  if (!x || !w || !out) return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (m < 0 || n < 1 || k < 64 || k % 64)
    return fail(nullptr, DG_ERR_SHAPE, "k must be a positive multiple of 64");
  int epi;
  if (mode == 0) epi = EPI_STORE_BF16;
  else if (mode == 1) epi = EPI_STORE_F32;
  else if (mode == 2) epi = EPI_ADD_F32;
  else return fail(nullptr, DG_ERR_INVALID_ARG, "mode must be 0, 1 or 2");
  GemmArgs g = gemm_dense((const uint16_t*)x, m, k, w, n, out, n);
  HIPCHK(nullptr, launch_gemm(epi, false, g, grid_m_dense(m, epi), (hipStream_t)stream));
  return DG_OK;
}

size_t dg_op_attention_workspace_bytes(int32_t n, int32_t canvas_len,
                                       int32_t n_q_heads, int32_t n_kv_heads,
                                       int32_t head_dim, int32_t kv_splits) {
  if (n < 1 || canvas_len < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1)
    return 0;
  const int s = kv_splits > 0 ? kv_splits
                              : attention_auto_splits(n, canvas_len, n_q_heads, n_kv_heads, 0);
  if (s == 1) return kAlign;
  const long long rows = (long long)s * n * n_q_heads * canvas_len;
  return align_up(rows * head_dim * 4) + align_up(rows * 4);
}

dg_status dg_op_canvas_attention(const void* qkv, int32_t n, int32_t canvas_len,
                                 int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, const void* k_cache,
                                 const void* v_cache, int32_t max_requests,
                                 int32_t max_kv_len, const int32_t* req,
                                 const int32_t* prefix_len, int32_t causal,
                                 int32_t kv_splits, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!qkv || !k_cache || !v_cache || !req || !prefix_len || !out)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (n < 1 || n > DG_MAX_BATCH) return fail(nullptr, DG_ERR_CAPACITY, "n outside 1..64");
  if (canvas_len < 1 || canvas_len > DG_CANVAS)
    return fail(nullptr, DG_ERR_SHAPE, "canvas_len outside 1..256");
  if (head_dim != 64 && head_dim != 128)
    return fail(nullptr, DG_ERR_SHAPE, "head_dim must be 64 or 128");
  if (n_kv_heads < 1 || n_q_heads < n_kv_heads || n_q_heads % n_kv_heads)
    return fail(nullptr, DG_ERR_SHAPE, "n_q_heads must be a multiple of n_kv_heads");
  if (kv_splits < 0 || kv_splits > 32)
    return fail(nullptr, DG_ERR_INVALID_ARG, "kv_splits outside 0..32");
  for (int b = 0; b < n; ++b) {
    if (req[b] < 0 || req[b] >= max_requests)
      return fail(nullptr, DG_ERR_INVALID_ARG, "request slot out of range");
    if (prefix_len[b] < 0 || prefix_len[b] > max_kv_len)
      return fail(nullptr, DG_ERR_CAPACITY, "prefix_len outside 0..max_kv_len");
  }
  const size_t need = dg_op_attention_workspace_bytes(n, canvas_len, n_q_heads,
                                                      n_kv_heads, head_dim, kv_splits);
  if (workspace_bytes < need || (need > kAlign && !workspace))
    return fail(nullptr, DG_ERR_CAPACITY, "workspace too small");
  AttnArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.qkv = (const uint16_t*)qkv;
  aa.ldqkv = (n_q_heads + 2 * n_kv_heads) * head_dim;
  aa.C = canvas_len;
  aa.Hq = n_q_heads;
  aa.Hkv = n_kv_heads;
  aa.D = head_dim;
  aa.kc = (const uint16_t*)k_cache;
  aa.vc = (const uint16_t*)v_cache;
  aa.head_stride = (long long)max_kv_len * head_dim;
  aa.req_stride = (long long)n_kv_heads * aa.head_stride;
  for (int b = 0; b < n; ++b) {
    aa.req[b] = req[b];
    aa.plen[b] = prefix_len[b];
  }
  aa.n = n;
  int max_keys = 0;
  for (int b = 0; b < n; ++b) max_keys = std::max(max_keys, prefix_len[b] + canvas_len);
  aa.splits = kv_splits > 0 ? kv_splits
                            : attention_auto_splits(n, canvas_len, n_q_heads, n_kv_heads,
                                                    max_keys);
  aa.causal = causal ? 1 : 0;
  aa.out = (uint16_t*)out;
  if (aa.splits > 1) {
    const long long rows = (long long)aa.splits * n * n_q_heads * canvas_len;
    aa.opart = (float*)workspace;
    aa.lpart = (float*)((char*)workspace + align_up(rows * head_dim * 4));
  }
  HIPCHK(nullptr, launch_attention(aa, (hipStream_t)stream));
  return DG_OK;
}

dg_status dg_op_router_topk(const float* logits, int32_t tokens,
                            int32_t n_experts, int32_t top_k, int32_t* idx,
                            float* w, void* stream) {
  if (!logits || !idx || !w) return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (tokens < 0 || n_experts < 1 || n_experts > 256 || top_k < 1 ||
      top_k > 16 || top_k > n_experts)
    return fail(nullptr, DG_ERR_SHAPE, "need 1 <= top_k <= min(16, n_experts), n_experts <= 256");
  if (tokens == 0) return DG_OK;
  HIPCHK(nullptr, launch_topk(const_cast<float*>(logits), tokens, n_experts, top_k, 1,
                              idx, w, (hipStream_t)stream));
  return DG_OK;
}

size_t dg_op_moe_workspace_bytes(const dg_model_desc* d, int32_t tokens) {
  if (!check_desc(d).empty() || tokens < 1) return 0;
  return moe_layout(*d, tokens, nullptr, nullptr);
}

dg_status dg_op_moe(const dg_model_desc* desc, const dg_layer_weights* w,
                    const void* xhat, int32_t tokens, float* y,
                    int32_t* route_idx, float* route_w, int32_t* counts,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const std::string de = check_desc(desc);
  if (!de.empty()) return fail(nullptr, DG_ERR_SHAPE, de);
  if (!w || !xhat || !y || !workspace)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  const std::string le = check_layer(*desc, *w, true);
  if (!le.empty()) return fail(nullptr, DG_ERR_INVALID_ARG, le);
  if (tokens < 1 || (long long)tokens * desc->top_k > (1LL << 24))
    return fail(nullptr, DG_ERR_SHAPE, "tokens outside 1..2^24/top_k");
  if (((uintptr_t)workspace % kAlign) != 0)
    return fail(nullptr, DG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < moe_layout(*desc, tokens, nullptr, nullptr))
    return fail(nullptr, DG_ERR_CAPACITY, "workspace too small");
  MoeBufs b;
  moe_layout(*desc, tokens, (char*)workspace, &b);
  hipStream_t s = (hipStream_t)stream;
  HIPCHK(nullptr, run_moe(*desc, *w, (const uint16_t*)xhat, tokens, b, nullptr,
                          y, counts, s));
  const size_t tk = (size_t)tokens * desc->top_k;
  if (route_idx)
    HIPCHK(nullptr, hipMemcpyAsync(route_idx, b.ridx, tk * 4, hipMemcpyDeviceToDevice, s));
  if (route_w)
    HIPCHK(nullptr, hipMemcpyAsync(route_w, b.rw, tk * 4, hipMemcpyDeviceToDevice, s));
  return DG_OK;
}

size_t dg_op_lmhead_workspace_bytes(int32_t m, int32_t vocab) {
  if (m < 1 || vocab < 1) return 0;
  return align_up((size_t)m * lm_tiles(vocab) * 16);
}

dg_status dg_op_lmhead_entropy(const void* xhat, int32_t m, int32_t hidden,
                               const void* embed, int32_t vocab,
                               float* entropy, float* lse, int32_t* argmax,
                               float* logits, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!xhat || !embed || !entropy || !lse || !argmax || !workspace)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (m < 1 || vocab < 1 || hidden < 64 || hidden % 64)
    return fail(nullptr, DG_ERR_SHAPE, "need m >= 1, vocab >= 1, hidden a multiple of 64");
  if (workspace_bytes < dg_op_lmhead_workspace_bytes(m, vocab))
    return fail(nullptr, DG_ERR_CAPACITY, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  int n_tiles = 0;
  HIPCHK(nullptr, run_lm_head((const uint16_t*)xhat, m, nullptr, hidden, embed,
                              vocab, (float4*)workspace, logits, nullptr,
                              &n_tiles, s));
  HIPCHK(nullptr, launch_lm_merge((const float4*)workspace, n_tiles, nullptr, m,
                                  nullptr, entropy, lse, argmax, s));
  return DG_OK;
}

dg_status dg_op_eb_select(int32_t n, const float* entropy,
                          const int32_t* argmax, uint8_t* committed,
                          int32_t* tokens, int32_t* step, const float* gamma,
                          int32_t step_cap, int32_t refine, int32_t* n_new,
                          uint8_t* done, void* stream) {
  if (!entropy || !argmax || !committed || !tokens || !step || !gamma ||
      !n_new || !done)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (n < 1 || n > 65535) return fail(nullptr, DG_ERR_CAPACITY, "n outside 1..65535");
  if (step_cap < 1 || step_cap > 65535)
    return fail(nullptr, DG_ERR_INVALID_ARG, "step_cap must be in 1..65535");
  HIPCHK(nullptr, launch_eb_select(n, entropy, argmax, committed, tokens, step,
                                   gamma, step_cap, refine, n_new, done,
                                   (hipStream_t)stream));
  return DG_OK;
}

dg_status dg_op_kv_append(const void* qkv, int32_t n, int32_t canvas_len,
                          int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, void* k_cache, void* v_cache,
                          int32_t max_requests, int32_t max_kv_len,
                          const int32_t* req, const int32_t* row0,
                          void* stream) {
  if (!qkv || !k_cache || !v_cache || !req || !row0)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (n < 1 || n > DG_MAX_BATCH) return fail(nullptr, DG_ERR_CAPACITY, "n outside 1..64");
  if (canvas_len < 1 || canvas_len > DG_CANVAS || head_dim % 8 || head_dim < 8 ||
      n_kv_heads < 1 || n_q_heads < 1)
    return fail(nullptr, DG_ERR_SHAPE, "bad attention shape");
  for (int b = 0; b < n; ++b) {
    if (req[b] < 0 || req[b] >= max_requests)
      return fail(nullptr, DG_ERR_INVALID_ARG, "request slot out of range");
    if (row0[b] < 0 || row0[b] + canvas_len > max_kv_len)
      return fail(nullptr, DG_ERR_CAPACITY, "rows beyond max_kv_len");
  }
  const long long head_stride = (long long)max_kv_len * head_dim;
  HIPCHK(nullptr, launch_kv_append((const uint16_t*)qkv,
                                   (n_q_heads + 2 * n_kv_heads) * head_dim,
                                   n_q_heads * head_dim,
                                   (n_q_heads + n_kv_heads) * head_dim, n,
                                   canvas_len, n_kv_heads, head_dim,
                                   (uint16_t*)k_cache, (uint16_t*)v_cache,
                                   (long long)n_kv_heads * head_stride,
                                   head_stride, req, row0, (hipStream_t)stream));
  return DG_OK;
}

}  // extern "C"
