// Host side of libdg: argument validation, workspace layout, per-layer
// orchestration of the kernels and the extern "C" entry points of dg.h and
// dg_ops.h.  No device memory is allocated here: every buffer comes from the
// caller.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

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
  // E4M3 activations (act_dtype DG_FP8_E4M3): the FFN-norm rows and the
  // SwiGLU rows quantised per row, as codes (large-tile path) or as their
  // bf16 values (streaming path), with the row scales
  uint8_t* xq8;         // [T, H]
  uint16_t* xq16;       // [T, H]
  float* xs;            // [T]
  uint8_t* aq8;         // [max(pairs, slots), F]
  uint16_t* aq16;       // [max(pairs, slots), F]
  float* as;            // [max(pairs, slots)]
  // byte ranges (offset from the MoE base, length) that hold values, not
  // indices or counts: what DG_POISON fills
  std::vector<std::pair<size_t, size_t>> value_ranges;
};
// slot_tok is read up to one pass of 32 slots past an expert's last slot
constexpr int kSlotPad = 64;

struct dg_ctx {
  dg_model_desc d;
  int C;                  // canvas positions (desc canvas_len, 0 -> 256)
  const uint16_t* embed;
  const float* final_norm;
  std::vector<dg_layer_weights> layers;
  int max_requests, max_kv_len, max_canvases;
  uint16_t* k_cache;     // bf16 values, or E4M3 codes (kv8) at the same offsets
  uint16_t* v_cache;
  bool kv8;              // E4M3 cache: codes, then one fp32 scale per row
  float* k_scales;       // [L][R][Hkv][S] after the codes (kv8)
  float* v_scales;
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
  float2* lm_spart;       // [T][V/128] sampled (score, id) per tile
  float* smp_tau;         // [T] temperature of each LM-head row
  int32_t* smp_ctr;       // [T][3] Philox counter words of each LM-head row
  // E4M3 LM head (lm_dtype DG_FP8_E4M3): its weights and scales
  const void* lm8_w;
  const float* lm8_scale;
  bool proj8;             // W8A8 Q/K/V and output projections (proj_dtype)
  // rows quantised for an E4M3 product (the LM head's, a projection's
  // input; one at a time on the stream): E4M3 codes (large-tile kernel),
  // the codes' bf16 values (streaming and 64 x 64 tile kernels), scales
  uint8_t* rq8;
  uint16_t* rq16;
  float* rqs;
  long long split_rows_cap;  // attention partial rows the workspace holds
  // workspace byte ranges that hold values (activations, partials, router
  // logits, gate weights, expert rows), not indices or counts
  std::vector<std::pair<size_t, size_t>> value_ranges;
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

// A roctx range (shown by rocprofv3 --marker-trace) for the lifetime of the
// object: each engine call, and each layer inside one.
struct RoctxRange {
  explicit RoctxRange(const char* name) { roctxRangePushA(name); }
  ~RoctxRange() { roctxRangePop(); }
  RoctxRange(const RoctxRange&) = delete;
  RoctxRange& operator=(const RoctxRange&) = delete;
};

// Debugging aids read once per process from the environment:
//   DG_POISON=1  every engine call that runs layers first fills the
//                workspace's value regions (activations, partials, router
//                logits, expert rows; not its indices and counts) with
//                0xFF bytes, NaN in fp32, bf16 and E4M3, so that a read of
//                scratch no kernel of the call wrote shows up as NaN;
//   DG_CHECK=1   dg_commit_block reads the committed flags back and refuses
//                (DG_ERR_STATE) a canvas with an uncommitted position;
//   DG_KV_SPLIT=s  the engine's attention uses s KV splits (1..32, at most
//                what the workspace's partials hold) instead of its own
//                choice.
static bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && v[0] == '1' && v[1] == 0;
}
bool poison_on() {
  static const bool on = env_flag("DG_POISON");
  return on;
}
bool check_on() {
  static const bool on = env_flag("DG_CHECK");
  return on;
}
int kv_split_override() {
  static const int s = [] {
    const char* v = getenv("DG_KV_SPLIT");
    const int x = v ? atoi(v) : 0;
    return x >= 1 && x <= 32 ? x : 0;
  }();
  return s;
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

int lm_tiles(int vocab) { return (vocab + 127) / 128; }

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
// (token, expert) pairs per token: the top_k routed experts and the shared
// experts (write-up Table 1: "+ 1 shared"), which every token uses with
// weight 1; the shared expert is group n_experts of the expert matrices.
int pairs_per_token(const dg_model_desc& d) { return d.top_k + d.n_shared_experts; }
int expert_groups(const dg_model_desc& d) { return d.n_experts + d.n_shared_experts; }

bool use_stream_moe(const dg_model_desc& d, int T) {
  const long long pairs = (long long)T * d.top_k;
  return pairs <= 32LL * d.n_experts && stream_moe_ok(d.hidden, d.expert_ffn);
}

// Workspace of the MoE pipeline for T tokens.
size_t moe_layout(const dg_model_desc& d, int T, char* base, MoeBufs* b) {
  Carve cv;
  const long long pairs = (long long)T * pairs_per_token(d);
  const int EG = expert_groups(d);
  const int nc = permute_chunks((int)pairs);
  // slots per expert for the streaming path: every T it is taken for
  // (a token picks an expert at most once, so T slots always suffice)
  const int cap = stream_moe_ok(d.hidden, d.expert_ffn)
                      ? (int)std::min<long long>(T, 32LL * d.n_experts / d.top_k)
                      : 0;
  const long long slots = (long long)EG * cap;
  const size_t o_rl = cv.take((size_t)kRouterSlabs * T * d.n_experts * 4);
  const size_t o_ri = cv.take((size_t)pairs * 4);
  const size_t o_rw = cv.take((size_t)pairs * 4);
  const size_t o_cc = cv.take((size_t)nc * EG * 4);
  const size_t o_lr = cv.take((size_t)pairs * 4);
  const size_t o_cb = cv.take((size_t)nc * EG * 4);
  const size_t o_of = cv.take((size_t)(EG + 1) * 4);
  const size_t o_to = cv.take((size_t)(EG + 1) * 4);
  const size_t o_pm = cv.take((size_t)pairs * 4);
  const size_t o_ac = cv.take((size_t)std::max(pairs, slots) * d.expert_ffn * 2);
  const size_t o_y = cv.take((size_t)pairs * d.hidden * 4);
  const size_t o_cn = cv.take((size_t)EG * 4);
  const size_t o_sp = cv.take((size_t)slots * 4);
  const size_t o_sw = cv.take((size_t)slots * 4);
  const size_t o_st = cv.take((size_t)(slots + kSlotPad) * 4);
  // E4M3 activation buffers only when the model asks for them
  const bool a8 = d.act_dtype == DG_FP8_E4M3;
  const long long arows = std::max(pairs, slots);
  const size_t o_x8 = a8 ? cv.take((size_t)T * d.hidden) : 0;
  const size_t o_x16 = a8 ? cv.take((size_t)T * d.hidden * 2) : 0;
  const size_t o_xs = a8 ? cv.take((size_t)T * 4) : 0;
  const size_t o_a8 = a8 ? cv.take((size_t)arows * d.expert_ffn) : 0;
  const size_t o_a16 = a8 ? cv.take((size_t)arows * d.expert_ffn * 2) : 0;
  const size_t o_as = a8 ? cv.take((size_t)arows * 4) : 0;
  if (b) {
    b->value_ranges = {{o_rl, o_ri - o_rl}, {o_rw, o_cc - o_rw}, {o_ac, o_cn - o_ac}};
    if (a8) b->value_ranges.push_back({o_x8, cv.off - o_x8});
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
    b->xq8 = a8 ? (uint8_t*)(base + o_x8) : nullptr;
    b->xq16 = a8 ? (uint16_t*)(base + o_x16) : nullptr;
    b->xs = a8 ? (float*)(base + o_xs) : nullptr;
    b->aq8 = a8 ? (uint8_t*)(base + o_a8) : nullptr;
    b->aq16 = a8 ? (uint16_t*)(base + o_a16) : nullptr;
    b->as = a8 ? (float*)(base + o_as) : nullptr;
    b->counts = (int32_t*)(base + o_cn);
    b->slot_pair = (int32_t*)(base + o_sp);
    b->slot_w = (float*)(base + o_sw);
    b->slot_tok = (int32_t*)(base + o_st);
  }
  return cv.off;
}

size_t ctx_layout(const dg_model_desc& d, int max_canvases, dg_ctx* c);

// DG_POISON: the workspace's value regions to NaN (see env_flag above)
static dg_status poison_workspace(dg_ctx* c) {
  if (!poison_on()) return DG_OK;
  for (const auto& r : c->value_ranges)
    if (r.second) HIPCHK(c, hipMemsetAsync(c->ws + r.first, 0xFF, r.second, c->stream));
  return DG_OK;
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
  const size_t o_sp = cv.take(T * lm_tiles(d.vocab) * 8);
  const size_t o_tau = cv.take(T * 4);
  const size_t o_ctr = cv.take(T * 12);
  const bool rq = d.lm_dtype == DG_FP8_E4M3 || d.proj_dtype == DG_FP8_E4M3;
  const long long KQ = std::max(d.hidden, d.n_q_heads * d.head_dim);
  const size_t o_lq8 = rq ? cv.take(T * KQ) : 0;
  const size_t o_lq16 = rq ? cv.take(T * KQ * 2) : 0;
  const size_t o_lxs = rq ? cv.take(T * 4) : 0;
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
    c->lm_spart = (float2*)(w + o_sp);
    c->smp_tau = (float*)(w + o_tau);
    c->smp_ctr = (int32_t*)(w + o_ctr);
    c->rq8 = rq ? (uint8_t*)(w + o_lq8) : nullptr;
    c->rq16 = rq ? (uint16_t*)(w + o_lq16) : nullptr;
    c->rqs = rq ? (float*)(w + o_lxs) : nullptr;
    c->split_rows_cap = split_rows;
    moe_layout(d, (int)T, w + o_moe, &c->moe);
    c->value_ranges = {{o_x, o_rm - o_x}, {o_lm, o_ctr - o_lm}};
    if (rq) c->value_ranges.push_back({o_lq8, o_moe - o_lq8});
    for (const auto& r : c->moe.value_ranges)
      c->value_ranges.push_back({o_moe + r.first, r.second});
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
  if (d->canvas_len < 0 || d->canvas_len > DG_CANVAS)
    return "canvas_len must be in 0..256 (0: 256)";
  if (d->act_dtype != DG_BF16 && d->act_dtype != DG_FP8_E4M3)
    return "act_dtype must be DG_BF16 or DG_FP8_E4M3";
  if (d->kv_dtype != DG_BF16 && d->kv_dtype != DG_FP8_E4M3)
    return "kv_dtype must be DG_BF16 or DG_FP8_E4M3";
  if (d->act_dtype == DG_FP8_E4M3 &&
      (d->expert_dtype != DG_FP8_E4M3 || d->hidden % 128 || d->expert_ffn % 128 ||
       d->hidden > 4096 || d->expert_ffn > 4096))
    return "E4M3 activations need E4M3 experts and hidden, expert_ffn multiples of "
           "128 up to 4096";
  if (d->lm_dtype != DG_BF16 && d->lm_dtype != DG_FP8_E4M3)
    return "lm_dtype must be DG_BF16 or DG_FP8_E4M3";
  if (d->lm_dtype == DG_FP8_E4M3 && (d->hidden % 128 || d->hidden > 4096))
    return "an E4M3 LM head needs hidden a multiple of 128 up to 4096";
  if (d->proj_dtype != DG_BF16 && d->proj_dtype != DG_FP8_E4M3)
    return "proj_dtype must be DG_BF16 or DG_FP8_E4M3";
  if (d->proj_dtype == DG_FP8_E4M3 &&
      (d->hidden % 128 || d->hidden > 4096 || (d->n_q_heads * d->head_dim) % 128 ||
       d->n_q_heads * d->head_dim > 4096))
    return "E4M3 projections need hidden and n_q_heads*head_dim multiples of 128 up "
           "to 4096";
  if (d->n_shared_experts < 0 || d->n_shared_experts > 1 ||
      d->n_experts + d->n_shared_experts > 256)
    return "n_shared_experts must be 0 or 1 (and n_experts + shared <= 256)";
  return "";
}

std::string check_layer(const dg_model_desc& d, const dg_layer_weights& w,
                        bool moe_only) {
  if (!moe_only && (!w.attn_norm || !w.w_qkv || !w.w_o || !w.ffn_norm))
    return "layer attention weights must not be NULL";
  if (!w.w_router || !w.w_gate_up || !w.w_down)
    return "layer MoE weights must not be NULL";
  if (!moe_only && d.proj_dtype == DG_FP8_E4M3 && (!w.qkv_scale || !w.o_scale))
    return "E4M3 projections need qkv_scale and o_scale";
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


// A W8A8 projection (proj_dtype DG_FP8_E4M3): x's M rows [M, K] bf16 are
// quantised per row, into E4M3 codes q8 for the large-tile kernel's FP8
// MFMA (thousands of rows) or into the codes' bf16 values q16 for the
// 64 x 64 tile kernel, with their scales xs; then epilogue epi of
// out = s_row w_scale[n] sum q q.  q8 / q16: [M, K], xs: [M].
hipError_t run_linear_e4m3(int epi, const uint16_t* x, int M, int K, const void* w8,
                           const float* w_scale, int N, void* out, int ldc,
                           uint8_t* q8, uint16_t* q16, float* xs, hipStream_t s) {
  GemmArgs g = gemm_dense(x, M, K, w8, N, out, ldc);
  const bool big = gemm_dense_on_mm(epi, g);
  hipError_t e = launch_quant_rows(x, K, M, K, nullptr, 0, big ? q8 : nullptr,
                                   big ? nullptr : q16, xs, s);
  if (e != hipSuccess) return e;
  if (big) g.A8 = q8;
  else g.A = q16;
  g.a_scale = xs;
  g.b_scale = w_scale;
  return launch_gemm(epi, true, g, grid_m_dense(M, epi), s);
}

// The LM head streams the tied embedding once per pass of up to 128 rows
// (k_stream.hip); above 128 rows the large-tile kernel (k_mm.hip) reads it
// once per 256 rows at a higher MFMA rate.  Both write one partial per row
// and 128 vocabulary rows.  When the row count is on the device (the
// uncommitted rows of a step) both are launched and each runs only for the
// row counts it takes.
constexpr int kLmStreamRows = 128;

// The E4M3 LM head: weights [V, H] e4m3 packed with per-row scales, and
// buffers for the rows' E4M3 codes [rows, H], their bf16 values [rows, H]
// and row scales [rows].
struct LmW8 {
  const void* w;
  const float* w_scale;
  uint8_t* q8;
  uint16_t* q16;
  float* xs;
};

// smp: temperature sampling (EPI_LMSAMPLE, see LmSample) or nullptr.
// w8: the E4M3 head (the rows are quantised first: only the live ones when
// their count is on the device) or nullptr for the bf16 table.
hipError_t run_lm_head(const uint16_t* xh, int rows_max, const int32_t* m_dev,
                       int hidden, const void* embed, int vocab, float4* part,
                       float* logits, const int32_t* row_map, int* n_tiles,
                       hipStream_t s, const LmSample* smp = nullptr,
                       const LmW8* w8 = nullptr) {
  *n_tiles = (vocab + 127) / 128;
  const int epi = smp ? EPI_LMSAMPLE : EPI_LMSTATS;
  const bool stream_ok = stream_lm_ok(hidden) && stream_rows_per_wg() == 128;
  const bool use_stream = stream_ok && (m_dev || rows_max <= kLmStreamRows);
  const bool use_mm = !stream_ok || rows_max > kLmStreamRows;
  if (w8) {
    const hipError_t e =
        launch_quant_rows(xh, hidden, rows_max, hidden, m_dev, m_dev ? rows_max : 0,
                          use_mm ? w8->q8 : nullptr, use_stream ? w8->q16 : nullptr,
                          w8->xs, s);
    if (e != hipSuccess) return e;
  }
  if (use_stream) {
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.X = w8 ? w8->q16 : xh;
    a.ldx = hidden;
    a.W = w8 ? w8->w : embed;
    if (w8) {
      a.w_scale = w8->w_scale;
      a.x_scale = w8->xs;
    }
    a.M = rows_max;
    a.M_dev = m_dev;
    a.N = vocab;
    a.K = hidden;
    a.part = part;
    a.n_tiles = *n_tiles;
    a.logits = logits;
    a.row_map = row_map;
    a.rows_le = use_mm ? kLmStreamRows : 0;
    if (smp) a.smp = *smp;
    hipError_t e = launch_stream(epi, w8 != nullptr, a, 1, s);
    if (e != hipSuccess) return e;
  }
  if (!use_mm) return hipSuccess;
  GemmArgs g = gemm_dense(xh, rows_max, hidden, w8 ? w8->w : embed, vocab, nullptr, 0);
  if (w8) {
    g.A8 = w8->q8;
    g.a_scale = w8->xs;
    g.b_scale = w8->w_scale;
  }
  g.M_dev = m_dev;
  g.rows_gt = use_stream ? kLmStreamRows : 0;
  g.part = part;
  g.n_tiles = *n_tiles;
  g.logits = logits;
  g.row_map = row_map;
  if (smp) g.smp = *smp;
  return launch_mm(epi, w8 != nullptr, g, (rows_max + mm_bm() - 1) / mm_bm(), s);
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
  const int S = d.n_shared_experts, K = k + S, EG = E + S;
  const bool w8 = d.expert_dtype == DG_FP8_E4M3;
  const int pairs = T * K;
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
    if (!counts_zeroed && (e = launch_zero_i32(b.counts, EG, s)) != hipSuccess) return e;
    {
      ProfScope ps(prof, 6);
      if ((e = launch_topk_slots(b.rlogits, T, E, k, r.splits, b.ridx, b.rw, b.counts,
                                 b.cap, b.slot_pair, b.slot_w, b.slot_tok, s, S)) !=
          hipSuccess)
        return e;
    }
    if (counts &&
        (e = hipMemcpyAsync(counts, b.counts, (size_t)E * 4, hipMemcpyDeviceToDevice, s)) !=
            hipSuccess)
      return e;
    const bool a8 = d.act_dtype == DG_FP8_E4M3;
    if (a8) {
      ProfScope ps(prof, 7);
      if ((e = launch_quant_rows(xh, H, T, H, nullptr, 0, nullptr, b.xq16, b.xs, s)) !=
          hipSuccess)
        return e;
    }
    StreamArgs gu;
    memset(&gu, 0, sizeof(gu));
    gu.X = a8 ? b.xq16 : xh;
    gu.x_scale = a8 ? b.xs : nullptr;
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
    // fewer (token, rank) pairs than expert groups: most groups are empty
    gu.count_first = pairs < EG ? 1 : 0;
    {
      ProfScope ps(prof, 8);
      if ((e = launch_stream(EPI_SWIGLU, w8, gu, EG, s)) != hipSuccess) return e;
    }
    if (a8) {
      ProfScope ps(prof, 7);
      if ((e = launch_quant_rows(b.act, F, EG * b.cap, F, b.counts, b.cap, nullptr, b.aq16,
                                 b.as, s)) != hipSuccess)
        return e;
    }
    StreamArgs dn;
    memset(&dn, 0, sizeof(dn));
    dn.X = a8 ? b.aq16 : b.act;
    dn.x_scale = a8 ? b.as : nullptr;
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
    dn.count_first = gu.count_first;
    {
      ProfScope ps(prof, 9);
      if ((e = launch_stream(EPI_DOWN, w8, dn, EG, s)) != hipSuccess) return e;
    }
    ProfScope ps10(prof, 10);
    if (next_g)
      return launch_unpermute_norm(b.y, T, K, H, x, moe_out, next_g, d.rms_eps,
                                   next_xh, next_copy, next_row, s);
    return launch_unpermute(b.y, T, K, H, x, moe_out, s);
  }
  {
    ProfScope ps(prof, 6);
    if ((e = launch_topk(b.rlogits, T, E, k, r.splits, b.ridx, b.rw, s, S)) != hipSuccess)
      return e;
  }
  // experts holding a few hundred rows each take the large-tile kernel
  // (256-row tiles), fewer the 64-row tiles; E4M3 activations always take
  // the large-tile kernel (its FP8 MFMA)
  const bool a8 = d.act_dtype == DG_FP8_E4M3;
  const bool big = a8 || (long long)T * k >= 192LL * E;
  const int bm = big ? mm_bm() : kGroupBM;
  {
    ProfScope ps(prof, 7);
    if ((e = launch_permute(b.ridx, pairs, EG, bm, b.chunk_counts,
                            b.local_rank, b.chunk_base, b.offsets,
                            b.tile_offsets, nullptr, b.perm, s)) != hipSuccess)
      return e;
    if (counts &&
        (e = launch_counts_from_offsets(b.offsets, E, counts, s)) != hipSuccess)
      return e;
  }
  const int grid_m = (pairs + bm - 1) / bm + std::min(EG, pairs);
  GemmArgs gu = gemm_dense(xh, pairs, H, w.w_gate_up, 2 * F, b.act, F);
  gu.a_map = b.perm;
  gu.a_map_div = K;
  gu.b_group_stride = (long long)2 * F * H;
  gu.b_scale = w.gate_up_scale;
  gu.scale_rows = 2 * F;
  gu.n_groups = EG;
  gu.group_offsets = b.offsets;
  gu.tile_offsets = b.tile_offsets;
  gu.ffn = F;
  if (a8) {
    ProfScope ps(prof, 7);
    if ((e = launch_quant_rows(xh, H, T, H, nullptr, 0, b.xq8, nullptr, b.xs, s)) !=
        hipSuccess)
      return e;
    gu.A8 = b.xq8;
    gu.a_scale = b.xs;
    gu.lda = H;
  }
  {
    ProfScope ps(prof, 8);
    if ((e = big ? launch_mm(EPI_SWIGLU, w8, gu, grid_m, s)
                 : launch_gemm(EPI_SWIGLU, w8, gu, grid_m, s)) != hipSuccess)
      return e;
  }
  GemmArgs dn = gemm_dense(b.act, pairs, F, w.w_down, H, b.y, H);
  dn.b_group_stride = (long long)H * F;
  dn.b_scale = w.down_scale;
  dn.scale_rows = H;
  dn.n_groups = EG;
  dn.group_offsets = b.offsets;
  dn.tile_offsets = b.tile_offsets;
  dn.c_map = b.perm;
  dn.row_scale = b.rw;
  if (a8) {
    ProfScope ps(prof, 7);
    if ((e = launch_quant_rows(b.act, F, pairs, F, nullptr, 0, b.aq8, nullptr, b.as, s)) !=
        hipSuccess)
      return e;
    dn.A8 = b.aq8;
    dn.a_scale = b.as;
    dn.lda = F;
  }
  {
    ProfScope ps(prof, 9);
    if ((e = big ? launch_mm(EPI_DOWN, w8, dn, grid_m, s)
                 : launch_gemm(EPI_DOWN, w8, dn, grid_m, s)) != hipSuccess)
      return e;
  }
  ProfScope ps10(prof, 10);
  if (next_g)
    return launch_unpermute_norm(b.y, T, K, H, x, moe_out, next_g, d.rms_eps,
                                 next_xh, next_copy, next_row, s);
  return launch_unpermute(b.y, T, K, H, x, moe_out, s);
}

// Copy of the routed experts' (idx, w) [T, k] out of the [T, k + S] pairs.
hipError_t copy_routing(void* dst, const void* src, int T, int k, int K, hipStream_t s) {
  if (k == K) return hipMemcpyAsync(dst, src, (size_t)T * k * 4, hipMemcpyDeviceToDevice, s);
  return hipMemcpy2DAsync(dst, (size_t)k * 4, src, (size_t)K * 4, (size_t)k * 4, T,
                          hipMemcpyDeviceToDevice, s);
}

const MoeBufs& ctx_moe_bufs(const dg_ctx* c) { return c->moe; }

// The canvases of one request (multi-canvas sampling) must be contiguous in
// the batch, in block order; returns false otherwise.  vis0[b] = the first
// canvas of b's request in the batch.
bool canvas_groups(int n, const int* req, int* vis0) {
  for (int b = 0; b < n; ++b) {
    vis0[b] = (b > 0 && req[b - 1] == req[b]) ? vis0[b - 1] : b;
    for (int q = 0; q < vis0[b]; ++q)
      if (req[q] == req[b]) return false;
  }
  return true;
}

dg_status check_batch(dg_ctx* c, const dg_canvas_batch* bt) {
  if (!bt) return fail(c, DG_ERR_INVALID_ARG, "batch is NULL");
  if (bt->n < 1 || bt->n > c->max_canvases)
    return fail(c, DG_ERR_CAPACITY, "batch size outside 1..max_canvases");
  if (!bt->req || !bt->tokens || !bt->committed || !bt->step)
    return fail(c, DG_ERR_INVALID_ARG, "batch pointers must not be NULL");
  for (int b = 0; b < bt->n; ++b) {
    const int r = bt->req[b];
    if (r < 0 || r >= c->max_requests)
      return fail(c, DG_ERR_INVALID_ARG, "request slot out of range");
  }
  int vis0[DG_MAX_BATCH];
  if (!canvas_groups(bt->n, bt->req, vis0))
    return fail(c, DG_ERR_INVALID_ARG,
                "the canvases of one request must be contiguous in the batch");
  return DG_OK;
}

// One decoder layer over the canvas rows in c->x, whose attention RMSNorm
// is already in c->xh (made by the embedding or the previous layer's
// un-permute).  The layer's un-permute makes the next layer's normed input,
// or after the last layer of a denoise step the final-norm rows of the
// uncommitted positions in compacted order (c->pos_map).  commit: write the
// layer's canvas K/V into the cache first, causal attention, and stop after
// the K/V of the last layer.
// commit: causal canvas attention, K/V appended to the cache; the last layer
// stops there unless full (AR mode, whose last layer also feeds the LM head,
// every row in place).
dg_status run_layer(dg_ctx* c, int l, int n, const int* req, const int* plen,
                    bool commit, const dg_capture* cap, int C = DG_CANVAS,
                    bool full = false) {
  const RoctxRange range("dg layer");
  const dg_model_desc& d = c->d;
  const dg_layer_weights& w = c->layers[l];
  const int T = n * C, H = d.hidden, D = d.head_dim;
  const int Hq = d.n_q_heads, Hkv = d.n_kv_heads;
  const int qkvN = (Hq + 2 * Hkv) * D;
  const long long head_stride = (long long)c->max_kv_len * D;
  const long long req_stride = (long long)Hkv * head_stride;
  const long long layer_stride = (long long)c->max_requests * req_stride;
  hipStream_t s = c->stream;
  if (c->proj8) {
    KRUN(c, 2, run_linear_e4m3(EPI_STORE_BF16, c->xh, T, H, w.w_qkv, w.qkv_scale, qkvN,
                               c->qkv, qkvN, c->rq8, c->rq16, c->rqs, s));
  } else {
    GemmArgs g = gemm_dense(c->xh, T, H, w.w_qkv, qkvN, c->qkv, qkvN);
    KRUN(c, 2, launch_gemm(EPI_STORE_BF16, false, g, grid_m_dense(T, EPI_STORE_BF16), s));
  }
  // layer l's cache: bf16 rows, or E4M3 codes (same offsets in bytes) and
  // one scale per row
  uint16_t* kc = c->kv8 ? (uint16_t*)((char*)c->k_cache + l * layer_stride)
                        : c->k_cache + l * layer_stride;
  uint16_t* vc = c->kv8 ? (uint16_t*)((char*)c->v_cache + l * layer_stride)
                        : c->v_cache + l * layer_stride;
  float* ks = c->kv8 ? c->k_scales + l * (layer_stride / D) : nullptr;
  float* vs = c->kv8 ? c->v_scales + l * (layer_stride / D) : nullptr;
  int vis0[DG_MAX_BATCH];
  canvas_groups(n, req, vis0);   // (checked by the caller)
  if (commit) {
    // canvas b is appended after its request's earlier canvases of the batch
    int row0[DG_MAX_BATCH];
    for (int b = 0; b < n; ++b) row0[b] = plen[b] + (b - vis0[b]) * C;
    if (c->kv8) {
      KvQuantArgs q;
      memset(&q, 0, sizeof(q));
      q.src_k = c->qkv + Hq * D;
      q.src_v = c->qkv + (Hq + Hkv) * D;
      q.src_b_stride = (long long)C * qkvN;
      q.src_row_stride = qkvN;
      q.src_head_stride = D;
      q.n = n;
      q.rows = C;
      q.Hkv = Hkv;
      q.D = D;
      q.S = c->max_kv_len;
      q.kc = (uint8_t*)kc;
      q.vc = (uint8_t*)vc;
      q.ks = ks;
      q.vs = vs;
      for (int b = 0; b < n; ++b) {
        q.req[b] = req[b];
        q.row0[b] = row0[b];
      }
      KRUN(c, 15, launch_kv_quant(q, s));
    } else {
      KRUN(c, 15, launch_kv_append(c->qkv, qkvN, Hq * D, (Hq + Hkv) * D, n,
                                 C, Hkv, D, kc, vc, req_stride,
                                 head_stride, req, row0, s));
    }
    if (l == d.n_layers - 1 && !full) return DG_OK;
  }
  AttnArgs aa;
  memset(&aa, 0, sizeof(aa));
  aa.qkv = c->qkv;
  aa.ldqkv = qkvN;
  aa.C = C;
  aa.Hq = Hq;
  aa.Hkv = Hkv;
  aa.D = D;
  aa.kc = kc;
  aa.vc = vc;
  aa.ks = ks;
  aa.vs = vs;
  aa.req_stride = req_stride;
  aa.head_stride = head_stride;
  for (int b = 0; b < n; ++b) {
    aa.req[b] = req[b];
    aa.plen[b] = plen[b];
    aa.vis0[b] = vis0[b];
  }
  aa.n = n;
  int max_keys = 0;
  for (int b = 0; b < n; ++b)
    max_keys = std::max(max_keys, plen[b] + (b - vis0[b] + 1) * C);
  aa.splits = kv_split_override() ? kv_split_override()
                                  : attention_auto_splits(n, C, Hq, Hkv, max_keys);
  // (shorter canvases than the workspace was sized for may ask for more
  // splits than its partials hold)
  aa.splits = (int)std::max<long long>(
      1, std::min<long long>(aa.splits, c->split_rows_cap / ((long long)n * Hq * C)));
  aa.causal = commit ? 1 : 0;
  aa.out = c->attn;
  aa.opart = c->opart;
  aa.lpart = c->lpart;
  KRUN(c, 3, launch_attention(aa, s));
  if (cap && cap->attn_out)
    HIPCHK(c, hipMemcpyAsync((char*)cap->attn_out + (size_t)l * T * Hq * D * 2,
                             c->attn, (size_t)T * Hq * D * 2,
                             hipMemcpyDeviceToDevice, s));
  if (c->proj8) {
    KRUN(c, 4, run_linear_e4m3(EPI_ADD_F32, c->attn, T, Hq * D, w.w_o, w.o_scale, H, c->x,
                               H, c->rq8, c->rq16, c->rqs, s));
  } else {
    GemmArgs o = gemm_dense(c->attn, T, Hq * D, w.w_o, H, c->x, H);
    KRUN(c, 4, launch_gemm(EPI_ADD_F32, false, o, grid_m_dense(T, EPI_ADD_F32), s));
  }
  const MoeBufs& mb = ctx_moe_bufs(c);
  KRUN(c, 1, launch_rmsnorm(c->x, T, H, w.ffn_norm, d.rms_eps, c->xh, nullptr,
                           nullptr, nullptr, s, mb.counts, expert_groups(d)));
  float* moe_out = (cap && cap->moe_out) ? cap->moe_out + (size_t)l * T * H : nullptr;
  const bool last = l == d.n_layers - 1;
  const float* next_g = last ? c->final_norm : c->layers[l + 1].attn_norm;
  float* next_copy = (last && cap && cap->final_xhat) ? cap->final_xhat : nullptr;
  HIPCHK(c, run_moe(d, w, c->xh, T, mb, c->x, moe_out, nullptr, s, &c->prof, next_g,
                    c->xh, next_copy, last && !full ? c->pos_map : nullptr, true));
  if (cap) {
    const size_t tk = (size_t)T * d.top_k;
    const int K = pairs_per_token(d);
    if (cap->route_idx)
      HIPCHK(c, copy_routing(cap->route_idx + l * tk, mb.ridx, T, d.top_k, K, s));
    if (cap->route_w)
      HIPCHK(c, copy_routing(cap->route_w + l * tk, mb.rw, T, d.top_k, K, s));
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
  const size_t rows = (size_t)d->n_layers * max_requests * d->n_kv_heads * max_kv_len;
  // E4M3: one byte per value, then one fp32 scale per row
  if (d->kv_dtype == DG_FP8_E4M3) return rows * d->head_dim + rows * 4;
  return rows * d->head_dim * 2;
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
  if (desc->lm_dtype == DG_FP8_E4M3 && (!weights->lm_head || !weights->lm_head_scale))
    return fail(nullptr, DG_ERR_INVALID_ARG,
                "an E4M3 LM head needs lm_head and lm_head_scale");
  for (int l = 0; l < desc->n_layers; ++l) {
    const std::string le = check_layer(*desc, weights->layers[l], false);
    if (!le.empty()) return fail(nullptr, DG_ERR_INVALID_ARG, le);
  }
  if (max_requests < 1 || max_kv_len < DG_CANVAS)
    return fail(nullptr, DG_ERR_INVALID_ARG,
                "max_requests must be >= 1 and max_kv_len >= 256");
  // (several canvases may belong to one request, so max_canvases may
  // exceed max_requests)
  if (max_canvases < 1 || max_canvases > DG_MAX_BATCH)
    return fail(nullptr, DG_ERR_INVALID_ARG, "max_canvases must be in 1..64");
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
  c->C = desc->canvas_len ? desc->canvas_len : DG_CANVAS;
  c->embed = (const uint16_t*)weights->embed;
  c->final_norm = weights->final_norm;
  c->lm8_w = desc->lm_dtype == DG_FP8_E4M3 ? weights->lm_head : nullptr;
  c->lm8_scale = desc->lm_dtype == DG_FP8_E4M3 ? weights->lm_head_scale : nullptr;
  c->proj8 = desc->proj_dtype == DG_FP8_E4M3;
  c->layers.assign(weights->layers, weights->layers + desc->n_layers);
  c->max_requests = max_requests;
  c->max_kv_len = max_kv_len;
  c->max_canvases = max_canvases;
  c->k_cache = (uint16_t*)k_cache;
  c->v_cache = (uint16_t*)v_cache;
  c->kv8 = desc->kv_dtype == DG_FP8_E4M3;
  if (c->kv8) {
    const size_t rows = (size_t)desc->n_layers * max_requests * desc->n_kv_heads * max_kv_len;
    c->k_scales = (float*)((char*)k_cache + rows * desc->head_dim);
    c->v_scales = (float*)((char*)v_cache + rows * desc->head_dim);
    if (((uintptr_t)c->k_scales | (uintptr_t)c->v_scales) % 4) {
      delete c;
      return fail(nullptr, DG_ERR_INVALID_ARG, "caches must be 4-byte aligned");
    }
  }
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

dg_status dg_set_stream(dg_ctx* c, void* stream) {
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  c->stream = (hipStream_t)stream;
  c->prof.s = c->stream;
  return DG_OK;
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
  const RoctxRange range("dg_prefill_kv");
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  if (tokens && (k || v)) return fail(c, DG_ERR_INVALID_ARG, "give either tokens or k/v");
  if (!tokens && (!k || !v)) return fail(c, DG_ERR_INVALID_ARG, "k and v must not be NULL");
  if (req < 0 || req >= c->max_requests)
    return fail(c, DG_ERR_INVALID_ARG, "request slot out of range");
  if (n < 0 || n > c->max_kv_len)
    return fail(c, DG_ERR_CAPACITY, "prefix longer than max_kv_len");
  const dg_model_desc& d = c->d;
  if (tokens) {
    // token mode: the causal encode of the commit, over chunks of up to 256
    // prompt tokens; chunk i attends to the cache rows the chunks before it
    // wrote and causally within itself, so the result is the causal encode
    // of the whole prompt
    int plen = 0;
    const dg_status ps = poison_workspace(c);
    if (ps != DG_OK) return ps;
    for (int off = 0; off < n; off += DG_CANVAS) {
      const int C = std::min(DG_CANVAS, n - off);
      KRUN(c, 0, launch_embed_norm(tokens + off, C, c->embed, d.vocab, d.hidden, c->x,
                                   c->layers[0].attn_norm, d.rms_eps, c->xh, c->stream));
      for (int l = 0; l < d.n_layers; ++l) {
        const dg_status st = run_layer(c, l, 1, &req, &plen, true, nullptr, C);
        if (st != DG_OK) return st;
      }
      plen += C;
    }
    c->kv_len[req] = n;
    return DG_OK;
  }
  const long long head_stride = (long long)c->max_kv_len * d.head_dim;
  const long long req_stride = (long long)d.n_kv_heads * head_stride;
  const long long layer_stride = (long long)c->max_requests * req_stride;
  const long long src_layer = (long long)d.n_kv_heads * n * d.head_dim;
  for (int l = 0; l < d.n_layers; ++l) {
    if (c->kv8) {   // E4M3 cache: each row quantised on the way in
      KvQuantArgs q;
      memset(&q, 0, sizeof(q));
      q.src_k = (const uint16_t*)k + l * src_layer;
      q.src_v = (const uint16_t*)v + l * src_layer;
      q.src_row_stride = d.head_dim;
      q.src_head_stride = (long long)n * d.head_dim;
      q.n = 1;
      q.rows = n;
      q.Hkv = d.n_kv_heads;
      q.D = d.head_dim;
      q.S = c->max_kv_len;
      q.kc = (uint8_t*)c->k_cache + l * layer_stride;
      q.vc = (uint8_t*)c->v_cache + l * layer_stride;
      q.ks = c->k_scales + l * (layer_stride / d.head_dim);
      q.vs = c->v_scales + l * (layer_stride / d.head_dim);
      q.req[0] = req;
      KRUN(c, 16, launch_kv_quant(q, c->stream));
      continue;
    }
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
  const RoctxRange range("dg_denoise_step");
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(c, bt);
  if (st != DG_OK) return st;
  if (!out || !out->entropy || !out->lse || !out->argmax)
    return fail(c, DG_ERR_INVALID_ARG, "step outputs must not be NULL");
  const dg_sampling* smp = out->sampling;
  if (smp) {
    if (!smp->sample) return fail(c, DG_ERR_INVALID_ARG, "sampling->sample is NULL");
    // tau0 below 1e-6 (other than 0) would overflow z / tau in fp32
    if (!std::isfinite(smp->tau0) || !(smp->tau0 == 0.f || smp->tau0 >= 1e-6f) ||
        smp->budget < 0)
      return fail(c, DG_ERR_INVALID_ARG, "need tau0 = 0 or finite >= 1e-6, budget >= 0");
  }
  const dg_model_desc& d = c->d;
  const int n = bt->n, C = c->C, T = n * C, H = d.hidden;
  int req[DG_MAX_BATCH], plen[DG_MAX_BATCH];
  for (int b = 0; b < n; ++b) {
    req[b] = bt->req[b];
    plen[b] = c->kv_len[req[b]];
  }
  hipStream_t s = c->stream;
  if ((st = poison_workspace(c)) != DG_OK) return st;
  KRUN(c, 0, launch_embed_norm(bt->tokens, T, c->embed, d.vocab, H, c->x,
                               c->layers[0].attn_norm, d.rms_eps, c->xh, s, bt->committed,
                               c->row_map, c->m_dev, c->pos_map));
  for (int l = 0; l < d.n_layers; ++l) {
    st = run_layer(c, l, n, req, plen, false, out->capture, C);
    if (st != DG_OK) return st;
  }
  int n_tiles = 0;
  LmSample ls = {};
  if (smp) {
    KRUN(c, 13, launch_sample_rows(c->row_map, c->m_dev, T, bt->step, C, smp->tau0,
                                   smp->budget, c->smp_tau, c->smp_ctr, s));
    ls.tau = c->smp_tau;
    ls.ctr = c->smp_ctr;
    ls.key0 = (uint32_t)smp->seed;
    ls.key1 = (uint32_t)(smp->seed >> 32);
    ls.spart = c->lm_spart;
  }
  const LmW8 lw8 = {c->lm8_w, c->lm8_scale, c->rq8, c->rq16, c->rqs};
  KRUN(c, 12, run_lm_head(c->xh, T, c->m_dev, H, c->embed, d.vocab, c->lm_part,
                          out->logits, c->row_map, &n_tiles, s, smp ? &ls : nullptr,
                          c->lm8_w ? &lw8 : nullptr));
  KRUN(c, 13, launch_lm_merge(c->lm_part, n_tiles, c->m_dev, T, c->row_map,
                              out->entropy, out->lse, out->argmax, s,
                              smp ? c->smp_tau : nullptr, smp ? c->lm_spart : nullptr,
                              smp ? smp->sample : nullptr));
  return DG_OK;
}

dg_status dg_eb_select(dg_ctx* c, const dg_canvas_batch* bt,
                       const float* entropy, const int32_t* argmax,
                       const float* gamma, int32_t step_cap, int32_t refine,
                       int32_t* n_new, uint8_t* done) {
  const RoctxRange range("dg_eb_select");
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(c, bt);
  if (st != DG_OK) return st;
  if (!entropy || !argmax || !gamma || !n_new || !done)
    return fail(c, DG_ERR_INVALID_ARG, "sampler pointers must not be NULL");
  if (step_cap < 1 || step_cap > 65535)
    return fail(c, DG_ERR_INVALID_ARG, "step_cap must be in 1..65535");
  KRUN(c, 14, launch_eb_select(bt->n, entropy, argmax, bt->committed, bt->tokens,
                             bt->step, gamma, step_cap, refine, n_new, done,
                             c->stream, c->C));
  return DG_OK;
}

dg_status dg_commit_block(dg_ctx* c, const dg_canvas_batch* bt) {
  const RoctxRange range("dg_commit_block");
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(c, bt);
  if (st != DG_OK) return st;
  const int n = bt->n, C = c->C, T = n * C;
  int req[DG_MAX_BATCH], plen[DG_MAX_BATCH], vis0[DG_MAX_BATCH];
  canvas_groups(n, bt->req, vis0);
  for (int b = 0; b < n; ++b) {
    req[b] = bt->req[b];
    plen[b] = c->kv_len[req[b]];
    if (plen[b] + (b - vis0[b] + 1) * C > c->max_kv_len)
      return fail(c, DG_ERR_CAPACITY,
                  "KV cache full: kv_len + canvas_len x canvases > max_kv_len");
  }
  if (check_on()) {
    // DG_CHECK: every position of every canvas committed (host read-back)
    std::vector<uint8_t> com((size_t)T);
    HIPCHK(c, hipMemcpyAsync(com.data(), bt->committed, (size_t)T, hipMemcpyDeviceToHost,
                             c->stream));
    HIPCHK(c, hipStreamSynchronize(c->stream));
    for (int i = 0; i < T; ++i)
      if (!com[i])
        return fail(c, DG_ERR_STATE, "DG_CHECK: commit of a canvas with uncommitted positions");
  }
  if ((st = poison_workspace(c)) != DG_OK) return st;
  KRUN(c, 0, launch_embed_norm(bt->tokens, T, c->embed, c->d.vocab, c->d.hidden, c->x,
                               c->layers[0].attn_norm, c->d.rms_eps, c->xh, c->stream));
  for (int l = 0; l < c->d.n_layers; ++l) {
    st = run_layer(c, l, n, req, plen, true, nullptr, C);
    if (st != DG_OK) return st;
  }
  for (int b = 0; b < n; ++b) c->kv_len[req[b]] += C;  // per canvas
  return DG_OK;
}

dg_status dg_ar_step(dg_ctx* c, int32_t n, const int32_t* req,
                     const int32_t* tokens, const dg_step_out* out) {
  const RoctxRange range("dg_ar_step");
  if (!c) return fail(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  if (!req || !tokens || !out || !out->entropy || !out->lse || !out->argmax)
    return fail(c, DG_ERR_INVALID_ARG, "NULL pointer");
  if (out->sampling || out->capture)
    return fail(c, DG_ERR_UNSUPPORTED, "AR steps take no sampling or capture");
  if (n < 1 || n > c->max_canvases * c->C)
    return fail(c, DG_ERR_CAPACITY, "n outside 1..max_canvases x canvas_len");
  if (n > DG_MAX_BATCH) return fail(c, DG_ERR_CAPACITY, "n above 64");
  for (int b = 0; b < n; ++b)
    if (req[b] < 0 || req[b] >= c->max_requests)
      return fail(c, DG_ERR_INVALID_ARG, "req outside 0..max_requests-1");
  const dg_model_desc& d = c->d;
  int rq[DG_MAX_BATCH], plen[DG_MAX_BATCH], vis0[DG_MAX_BATCH];
  if (!canvas_groups(n, req, vis0))
    return fail(c, DG_ERR_INVALID_ARG, "the positions of one sequence must be contiguous");
  for (int b = 0; b < n; ++b) {
    rq[b] = req[b];
    plen[b] = c->kv_len[req[b]];
    if (plen[b] + (b - vis0[b]) + 1 > c->max_kv_len)
      return fail(c, DG_ERR_CAPACITY, "KV cache full");
  }
  hipStream_t s = c->stream;
  const dg_status ps = poison_workspace(c);
  if (ps != DG_OK) return ps;
  KRUN(c, 0, launch_embed_norm(tokens, n, c->embed, d.vocab, d.hidden, c->x,
                               c->layers[0].attn_norm, d.rms_eps, c->xh, s));
  for (int l = 0; l < d.n_layers; ++l) {
    dg_status st = run_layer(c, l, n, rq, plen, true, nullptr, 1, true);
    if (st != DG_OK) return st;
  }
  int n_tiles = 0;
  const LmW8 lw8 = {c->lm8_w, c->lm8_scale, c->rq8, c->rq16, c->rqs};
  KRUN(c, 12, run_lm_head(c->xh, n, nullptr, d.hidden, c->embed, d.vocab, c->lm_part,
                          out->logits, nullptr, &n_tiles, s, nullptr,
                          c->lm8_w ? &lw8 : nullptr));
  KRUN(c, 13, launch_lm_merge(c->lm_part, n_tiles, nullptr, n, nullptr, out->entropy,
                              out->lse, out->argmax, s));
  for (int b = 0; b < n; ++b) c->kv_len[req[b]] += 1;
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

size_t dg_op_linear_e4m3_workspace_bytes(int32_t m, int32_t k) {
  if (m < 1 || k < 1) return 0;
  return align_up((size_t)m * k) + align_up((size_t)m * k * 2) + align_up((size_t)m * 4);
}

dg_status dg_op_linear_e4m3(const void* x, int32_t m, int32_t k, const void* w8,
                            const float* w_scale, int32_t n, int32_t mode,
                            void* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!x || !w8 || !w_scale || !out || !workspace)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (m < 1 || n < 1 || k < 128 || k % 128 || k > 4096)
    return fail(nullptr, DG_ERR_SHAPE,
                "need m, n >= 1 and k a multiple of 128 up to 4096");
  int epi;
  if (mode == 0) epi = EPI_STORE_BF16;
  else if (mode == 1) epi = EPI_STORE_F32;
  else if (mode == 2) epi = EPI_ADD_F32;
  else return fail(nullptr, DG_ERR_INVALID_ARG, "mode must be 0, 1 or 2");
  if (((uintptr_t)workspace % kAlign) != 0)
    return fail(nullptr, DG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < dg_op_linear_e4m3_workspace_bytes(m, k))
    return fail(nullptr, DG_ERR_CAPACITY, "workspace too small");
  char* ws = (char*)workspace;
  Carve cv;
  const size_t o_q8 = cv.take((size_t)m * k);
  const size_t o_q16 = cv.take((size_t)m * k * 2);
  const size_t o_xs = cv.take((size_t)m * 4);
  HIPCHK(nullptr, run_linear_e4m3(epi, (const uint16_t*)x, m, k, w8, w_scale, n, out, n,
                                  (uint8_t*)(ws + o_q8), (uint16_t*)(ws + o_q16),
                                  (float*)(ws + o_xs), (hipStream_t)stream));
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
                                 const void* v_cache, const float* k_scale,
                                 const float* v_scale, int32_t max_requests,
                                 int32_t max_kv_len, const int32_t* req,
                                 const int32_t* prefix_len, int32_t causal,
                                 int32_t kv_splits, void* out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (!qkv || !k_cache || !v_cache || !req || !prefix_len || !out)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (!k_scale != !v_scale)
    return fail(nullptr, DG_ERR_INVALID_ARG, "give both scale arrays or neither");
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
  int vis0[DG_MAX_BATCH];
  if (!canvas_groups(n, req, vis0))
    return fail(nullptr, DG_ERR_INVALID_ARG,
                "the canvases of one request must be contiguous in the batch");
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
  aa.ks = k_scale;
  aa.vs = v_scale;
  aa.head_stride = (long long)max_kv_len * head_dim;
  aa.req_stride = (long long)n_kv_heads * aa.head_stride;
  for (int b = 0; b < n; ++b) {
    aa.req[b] = req[b];
    aa.plen[b] = prefix_len[b];
    aa.vis0[b] = vis0[b];
  }
  aa.n = n;
  int max_keys = 0;
  for (int b = 0; b < n; ++b)
    max_keys = std::max(max_keys, prefix_len[b] + (b - vis0[b] + 1) * canvas_len);
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
  if (tokens < 1 || (long long)tokens * pairs_per_token(*desc) > (1LL << 24))
    return fail(nullptr, DG_ERR_SHAPE, "tokens outside 1..2^24/(top_k + shared)");
  if (((uintptr_t)workspace % kAlign) != 0)
    return fail(nullptr, DG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < moe_layout(*desc, tokens, nullptr, nullptr))
    return fail(nullptr, DG_ERR_CAPACITY, "workspace too small");
  MoeBufs b;
  moe_layout(*desc, tokens, (char*)workspace, &b);
  hipStream_t s = (hipStream_t)stream;
  HIPCHK(nullptr, run_moe(*desc, *w, (const uint16_t*)xhat, tokens, b, nullptr,
                          y, counts, s));
  const int K = pairs_per_token(*desc);
  if (route_idx)
    HIPCHK(nullptr, copy_routing(route_idx, b.ridx, tokens, desc->top_k, K, s));
  if (route_w)
    HIPCHK(nullptr, copy_routing(route_w, b.rw, tokens, desc->top_k, K, s));
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

size_t dg_op_lmhead_e4m3_workspace_bytes(int32_t m, int32_t hidden, int32_t vocab) {
  if (m < 1 || vocab < 1 || hidden < 1) return 0;
  return align_up((size_t)m * lm_tiles(vocab) * 16) + align_up((size_t)m * hidden) +
         align_up((size_t)m * hidden * 2) + align_up((size_t)m * 4);
}

dg_status dg_op_lmhead_entropy_e4m3(const void* xhat, int32_t m, int32_t hidden,
                                    const void* w8, const float* w_scale,
                                    int32_t vocab, float* entropy, float* lse,
                                    int32_t* argmax, float* logits,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream) {
  if (!xhat || !w8 || !w_scale || !entropy || !lse || !argmax || !workspace)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (m < 1 || vocab < 1 || hidden < 128 || hidden % 128 || hidden > 4096)
    return fail(nullptr, DG_ERR_SHAPE,
                "need m >= 1, vocab >= 1, hidden a multiple of 128 up to 4096");
  if (((uintptr_t)workspace % kAlign) != 0)
    return fail(nullptr, DG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < dg_op_lmhead_e4m3_workspace_bytes(m, hidden, vocab))
    return fail(nullptr, DG_ERR_CAPACITY, "workspace too small");
  char* ws = (char*)workspace;
  Carve cv;
  const size_t o_part = cv.take((size_t)m * lm_tiles(vocab) * 16);
  const size_t o_q8 = cv.take((size_t)m * hidden);
  const size_t o_q16 = cv.take((size_t)m * hidden * 2);
  const size_t o_xs = cv.take((size_t)m * 4);
  const LmW8 lw8 = {w8, w_scale, (uint8_t*)(ws + o_q8), (uint16_t*)(ws + o_q16),
                    (float*)(ws + o_xs)};
  hipStream_t s = (hipStream_t)stream;
  int n_tiles = 0;
  HIPCHK(nullptr, run_lm_head((const uint16_t*)xhat, m, nullptr, hidden, nullptr, vocab,
                              (float4*)(ws + o_part), logits, nullptr, &n_tiles, s,
                              nullptr, &lw8));
  HIPCHK(nullptr, launch_lm_merge((const float4*)(ws + o_part), n_tiles, nullptr, m,
                                  nullptr, entropy, lse, argmax, s));
  return DG_OK;
}

size_t dg_op_lmhead_sample_workspace_bytes(int32_t m, int32_t vocab) {
  if (m < 1 || vocab < 1) return 0;
  return align_up((size_t)m * lm_tiles(vocab) * 16) +
         align_up((size_t)m * lm_tiles(vocab) * 8);
}

dg_status dg_op_lmhead_sample(const void* xhat, int32_t m, int32_t hidden,
                              const void* embed, int32_t vocab, const float* tau,
                              const int32_t* ctr, uint64_t seed, float* entropy,
                              float* lse, int32_t* argmax, int32_t* sample,
                              void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!xhat || !embed || !tau || !ctr || !entropy || !lse || !argmax || !sample ||
      !workspace)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (m < 1 || vocab < 1 || hidden < 64 || hidden % 64)
    return fail(nullptr, DG_ERR_SHAPE, "need m >= 1, vocab >= 1, hidden a multiple of 64");
  if (workspace_bytes < dg_op_lmhead_sample_workspace_bytes(m, vocab))
    return fail(nullptr, DG_ERR_CAPACITY, "workspace too small");
  hipStream_t s = (hipStream_t)stream;
  float4* part = (float4*)workspace;
  LmSample ls = {};
  ls.tau = tau;
  ls.ctr = ctr;
  ls.key0 = (uint32_t)seed;
  ls.key1 = (uint32_t)(seed >> 32);
  ls.spart = (float2*)((char*)workspace + align_up((size_t)m * lm_tiles(vocab) * 16));
  int n_tiles = 0;
  HIPCHK(nullptr, run_lm_head((const uint16_t*)xhat, m, nullptr, hidden, embed,
                              vocab, part, nullptr, nullptr, &n_tiles, s, &ls));
  HIPCHK(nullptr, launch_lm_merge(part, n_tiles, nullptr, m, nullptr, entropy, lse,
                                  argmax, s, tau, ls.spart, sample));
  return DG_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ static scratch
// Device memory of the allocation-free LM-head entry point: one array per
// GPU, part of the library's code object, alive until the process ends.
// Host code never uses the array's name as an address: its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[DG_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of this device's scratch array; nullptr (and *err set) on
// failure.
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  *err = hipSuccess;
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

dg_status dg_op_lmhead_entropy_static(const void* xhat, int32_t m,
                                      int32_t hidden, const void* embed,
                                      int32_t vocab, float* entropy,
                                      float* lse, int32_t* argmax,
                                      void* stream) {
  if (!xhat || !embed || !entropy || !lse || !argmax)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (m < 1 || vocab < 1 || hidden < 64 || hidden % 64)
    return fail(nullptr, DG_ERR_SHAPE, "need m >= 1, vocab >= 1, hidden a multiple of 64");
  if (dg_op_lmhead_workspace_bytes(m, vocab) > (size_t)DG_STATIC_SCRATCH_BYTES)
    return fail(nullptr, DG_ERR_CAPACITY,
                "m * ceil(vocab / 128) * 16 bytes of partials exceed the static "
                "scratch (DG_STATIC_SCRATCH_BYTES)");
  hipError_t e = hipSuccess;
  void* ws = scratch_ptr(&e);
  if (!ws)
    return fail(nullptr, DG_ERR_HIP,
                std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
  hipStream_t s = (hipStream_t)stream;
  int n_tiles = 0;
  // every partial a row's merge reads is written first by the LM head of
  // this call (rows < m, all tiles), so nothing needs clearing
  HIPCHK(nullptr, run_lm_head((const uint16_t*)xhat, m, nullptr, hidden, embed,
                              vocab, (float4*)ws, nullptr, nullptr, &n_tiles, s));
  HIPCHK(nullptr, launch_lm_merge((const float4*)ws, n_tiles, nullptr, m, nullptr,
                                  entropy, lse, argmax, s));
  return DG_OK;
}

dg_status dg_op_quantize_rows(const void* x, int32_t rows, int32_t k,
                              uint8_t* codes, void* values, float* scale,
                              void* stream) {
  if (!x || !scale || (!codes && !values))
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (rows < 0 || k < 8 || k % 8 || k > 4096)
    return fail(nullptr, DG_ERR_SHAPE, "k must be a multiple of 8 in 8..4096");
  HIPCHK(nullptr, launch_quant_rows((const uint16_t*)x, k, rows, k, nullptr, 0, codes,
                                    (uint16_t*)values, scale, (hipStream_t)stream));
  return DG_OK;
}

dg_status dg_op_eb_select(int32_t n, int32_t canvas_len, const float* entropy,
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
  if (canvas_len < 0 || canvas_len > DG_CANVAS)
    return fail(nullptr, DG_ERR_SHAPE, "canvas_len outside 0..256");
  HIPCHK(nullptr, launch_eb_select(n, entropy, argmax, committed, tokens, step,
                                   gamma, step_cap, refine, n_new, done,
                                   (hipStream_t)stream,
                                   canvas_len ? canvas_len : DG_CANVAS));
  return DG_OK;
}

dg_status dg_op_kv_append(const void* qkv, int32_t n, int32_t canvas_len,
                          int32_t n_q_heads, int32_t n_kv_heads,
                          int32_t head_dim, void* k_cache, void* v_cache,
                          float* k_scale, float* v_scale,
                          int32_t max_requests, int32_t max_kv_len,
                          const int32_t* req, const int32_t* row0,
                          void* stream) {
  if (!qkv || !k_cache || !v_cache || !req || !row0)
    return fail(nullptr, DG_ERR_INVALID_ARG, "NULL pointer");
  if (!k_scale != !v_scale)
    return fail(nullptr, DG_ERR_INVALID_ARG, "give both scale arrays or neither");
  if (k_scale && head_dim != 64 && head_dim != 128)
    return fail(nullptr, DG_ERR_SHAPE, "an E4M3 cache needs head_dim 64 or 128");
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
  if (k_scale) {
    const int ld = (n_q_heads + 2 * n_kv_heads) * head_dim;
    KvQuantArgs q;
    memset(&q, 0, sizeof(q));
    q.src_k = (const uint16_t*)qkv + n_q_heads * head_dim;
    q.src_v = (const uint16_t*)qkv + (n_q_heads + n_kv_heads) * head_dim;
    q.src_b_stride = (long long)canvas_len * ld;
    q.src_row_stride = ld;
    q.src_head_stride = head_dim;
    q.n = n;
    q.rows = canvas_len;
    q.Hkv = n_kv_heads;
    q.D = head_dim;
    q.S = max_kv_len;
    q.kc = (uint8_t*)k_cache;
    q.vc = (uint8_t*)v_cache;
    q.ks = k_scale;
    q.vs = v_scale;
    for (int b = 0; b < n; ++b) {
      q.req[b] = req[b];
      q.row0[b] = row0[b];
    }
    HIPCHK(nullptr, launch_kv_quant(q, (hipStream_t)stream));
    return DG_OK;
  }
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
