// Canvas attention: for each canvas, query head h and canvas position i,
//   o = sum_j softmax_j(q . k_j / sqrt(D)) v_j
// over the request's cached prefix keys, the keys of the request's earlier
// canvases in the batch (multi-canvas sampling: earlier blocks are fully
// visible, later ones not; model card feature list), then the canvas's own
// keys (all of them, or j <= i in the causal encode pass), KV head
// h / (Hq / Hkv) (write-up Figure 4 stages 2 and 3; model card "Model
// Overview").
//
// Work decomposition.  The G = Hq / Hkv query heads sharing a KV head give
// G x C query rows per (canvas, KV head).  A workgroup (8 waves) takes
// 128 * QB of them (each wave 16 * QB rows) and one contiguous range of
// 64-key tiles (KV split); K and V tiles are staged in double-buffered LDS
// and shared by all its rows, the next tile's global loads issued before
// the current tile's MFMAs, one barrier per tile.  QB = 2 (256 rows per
// workgroup) halves the K/V bytes each query row costs against QB = 1; the
// workgroups that share one (canvas, KV head, split) are numbered so that
// they run on the same XCD (workgroups are dealt to the 8 XCDs round-robin
// by id), so their K/V tiles come from one L2.
//
// Per wave: S^T = K Q^T with bf16 MFMA 16x16x32 (K tile rows as the A
// operand, read from LDS once per tile and used for all QB query blocks),
// so that every lane owns one query column per block and 4 keys of each
// 16-key block: the running max of the online softmax is a per-lane
// scalar.  P^T is taken straight from the S^T accumulators (bf16) as the B
// operand of O^T = V^T P^T; V is stored in LDS as key octets (for each d,
// the 8 keys one lane's operand holds, adjacent) so that the matching A
// operand is one 16-byte read.  The running sum of the probabilities comes
// from the same product with an A operand of ones.  Scores are scaled
// inside the exponent (exp2 of s * log2(e)/sqrt(D) - m).  The running max is
// raised only when a tile's max exceeds it by more than 2^8 in the
// exponential (or at the first tile): exact, since every probability and
// the running sum use the same m, and it skips the rescale of the output
// accumulators on almost every tile.  Probabilities below 2^8 times the
// largest so far stay well inside bf16 / fp32 range.
//
// Splits write (O / l, log2 l + m) partials that a second kernel merges
// with log-sum-exp weights.
#include <math.h>

#include <algorithm>

#include "dg_internal.h"

namespace dg {
namespace {

constexpr int KT = 64;         // keys per tile
constexpr int kThreads = 512;  // 8 waves
constexpr float kLazy = 8.f;   // raise the running max only past this (log2)

__device__ __forceinline__ f32x4_t mfma_v(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Workgroup id -> (row chunk, KV head, canvas, split).  Groups of one
// (KV head, canvas, split) hold n_chunks workgroups; 8 groups at a time are
// laid out chunk-major so that the workgroups of one group have ids equal
// mod 8 (same XCD).  Ids of a partial last set of 8 groups past the end
// return false.
struct AttnTile {
  int chunk, g, b, split;
};
__device__ __forceinline__ bool attn_tile(const AttnArgs& a, int n_chunks, AttnTile& t) {
  const int id = blockIdx.x;
  const int per8 = 8 * n_chunks;
  const int group = (id / per8) * 8 + id % 8;
  t.chunk = (id % per8) / 8;
  const int n_groups = a.Hkv * a.n * a.splits;
  if (group >= n_groups) return false;
  t.g = group % a.Hkv;
  const int bs = group / a.Hkv;
  t.b = bs / a.splits;
  t.split = bs % a.splits;
  return true;
}

// 8 cached E4M3 codes of a K/V row -> the 8 bf16 values attention reads:
// the code values (exact in bf16, by gfx950's conversion) times the row's
// scale in fp32, rounded to the nearest bf16.
__device__ __forceinline__ u32x4_t deq8(const uint2 q, float sc) {
  uint32_t w[4];
  w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false));
  w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true));
  w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false));
  w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true));
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_bf2(bf2f((uint16_t)(w[i] & 0xFFFFu)) * sc, bf2f((uint16_t)(w[i] >> 16)) * sc);
  return o;
}

// KV8: the cache holds E4M3 codes with a scale per row (a.ks / a.vs).
template <int D, int QB, bool KV8>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a, int n_chunks) {
  constexpr int KP = D + 16;     // padded K row (elements)
  constexpr int VO = D * 8 + (D / 16) * 8;  // key-octet stride (elements)
  constexpr int DC = D / 32;     // 32-wide d chunks (MFMA k for S)
  constexpr int DT = D / 16;     // 16-wide d tiles (MFMA rows for O^T)
  constexpr int KITEMS = KT * (D / 8);           // K 16-byte chunks per tile
  constexpr int KCH = (KITEMS + kThreads - 1) / kThreads;
  constexpr int VITEMS = (KT / 4) * (D / 8);     // V items: 4 keys x 8 d
  constexpr int VIT = (VITEMS + kThreads - 1) / kThreads;
  constexpr int ROWS = 128 * QB;                 // query rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vo[2][(KT / 8) * VO];

  AttnTile tl;
  if (!attn_tile(a, n_chunks, tl)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int g = tl.g, b = tl.b, split = tl.split;
  const int C = a.C, G = a.Hq / a.Hkv;
  const int P = a.plen[b];
  const int b0 = a.vis0[b];
  const int PE = P + (b - b0) * C;   // prefix + earlier canvases of the request
  const int N = PE + C;
  const int n_rows = a.n * a.Hq * C;

  // ---- this wave's query columns: block qb's lane column is row r of the
  // (canvas, KV head)'s G*C rows (query head g*G + r / C, position r % C)
  int qpos[QB], qhead[QB], klim[QB];
  bool qvalid[QB];
  u32x4_t qf[QB][DC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = tl.chunk * ROWS + wave * (16 * QB) + qb * 16 + l16;
    qvalid[qb] = r < G * C;
    const int rr = qvalid[qb] ? r : 0;
    qpos[qb] = rr % C;
    qhead[qb] = g * G + rr / C;
    const uint16_t* qp =
        a.qkv + (long long)(b * C + qpos[qb]) * a.ldqkv + qhead[qb] * D + lg * 8;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[qb][dc] = *(const u32x4_t*)(qp + dc * 32);
    // keys kk < klim are visible to this lane's query (all keys, or the
    // prefix and canvas keys up to the query's own position when causal)
    klim[qb] = a.causal ? min(N, PE + qpos[qb] + 1) : N;
  }
  // smallest visible-key bound over the workgroup's possible queries:
  // tiles below it need no mask
  const int klim_all = a.causal ? PE + 1 : N;

  const int n_kt = (N + KT - 1) / KT;
  const int kt_begin = (int)((long long)split * n_kt / a.splits);
  const int kt_end = (int)((long long)(split + 1) * n_kt / a.splits);

  const uint16_t* kpre = a.kc + (long long)a.req[b] * a.req_stride +
                         (long long)g * a.head_stride;
  const uint16_t* vpre = a.vc + (long long)a.req[b] * a.req_stride +
                         (long long)g * a.head_stride;
  // canvas keys: the request's earlier canvases b0..b-1 and canvas b are
  // consecutive rows of qkv, so key kk >= P is canvas row b0*C + (kk - P)
  const uint16_t* kcan = a.qkv + (long long)(b0 * C) * a.ldqkv + (a.Hq + g) * D;
  const uint16_t* vcan =
      a.qkv + (long long)(b0 * C) * a.ldqkv + (a.Hq + a.Hkv + g) * D;
  // Key kk's row (keys past N read the last key: a valid row whose score
  // is masked to -inf, so its probability is exactly 0).
  auto krow = [&](const uint16_t* pre, const uint16_t* can, int kk) {
    kk = min(kk, N - 1);
    return kk < P ? pre + (long long)kk * D : can + (long long)(kk - P) * a.ldqkv;
  };
  // E4M3 cache: the slot and head's codes (bytes, same strides) and scales
  const long long cbase = (long long)a.req[b] * a.req_stride + (long long)g * a.head_stride;
  const uint8_t* k8 = (const uint8_t*)a.kc + cbase;
  const uint8_t* v8 = (const uint8_t*)a.vc + cbase;
  const float* ks8 = KV8 ? a.ks + cbase / D : nullptr;
  const float* vs8 = KV8 ? a.vs + cbase / D : nullptr;
  // 8 values of key kk from d0 on, as bf16
  auto kload = [&](const uint16_t* pre, const uint16_t* can, const uint8_t* c8,
                   const float* s8, int kk, int d0) -> u32x4_t {
    if (KV8) {
      const int kc = min(kk, N - 1);
      if (kc < P) return deq8(*(const uint2*)(c8 + (long long)kc * D + d0), s8[kc]);
    }
    return *(const u32x4_t*)(krow(pre, can, kk) + d0);
  };

  // ---- K/V tile staging: global -> registers (issued a tile ahead) ->
  // LDS.  V goes to key octets: octet o = 4 kc + lg holds, for each d, the
  // 8 keys 32 kc + 16 h + 4 lg + e (h = 0, 1; e = 0..3) in the order the
  // PV product's operand takes them, so that one 16-byte read forms it; an
  // octet is 16-byte d entries with 16 bytes of padding after every 16 d.
  // An item is a key quad q (keys 4q..4q+3, i.e. kc = q / 8, h = q / 4 % 2,
  // lg = q % 4) x 8 d: four 16-byte loads, stored as 8 half entries.  Items
  // are numbered so that the lanes of a wave that store the same d range
  // hold quads of both halves (all 64 banks, no conflict).
  static_assert(KT == 64, "the octet layout assumes 16 key quads");
  auto vquad = [](int it) {
    const int qi = it / (D / 8);
    return ((qi & 3) << 2) | (qi >> 2);
  };
  u32x4_t kr[KCH], vr[VIT][4];
  auto gload = [&](int kt) {
    const int key0 = kt * KT;
    if (KV8 && key0 + KT <= P) {
      // a tile of cached keys only (uniform over the workgroup): E4M3 rows,
      // no canvas loads and no per-key branch
      static_for<KCH>([&](auto j) {
        const int c = min(tid + kThreads * (int)j, KITEMS - 1);
        const int key = key0 + c / (D / 8), dc = c % (D / 8);
        kr[j] = deq8(*(const uint2*)(k8 + (long long)key * D + dc * 8), ks8[key]);
      });
      static_for<VIT>([&](auto j) {
        const int it = min(tid + kThreads * (int)j, VITEMS - 1);
        const int q = vquad(it), c8 = it % (D / 8);
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
          const int key = key0 + 4 * q + kq;
          vr[j][kq] = deq8(*(const uint2*)(v8 + (long long)key * D + c8 * 8), vs8[key]);
        }
      });
      return;
    }
    if (!KV8 && key0 + KT <= P) {
      // a tile of cached keys only: plain row addresses, no per-key choice
      static_for<KCH>([&](auto j) {
        const int c = min(tid + kThreads * (int)j, KITEMS - 1);
        const int key = c / (D / 8), dc = c % (D / 8);
        kr[j] = *(const u32x4_t*)(kpre + (long long)(key0 + key) * D + dc * 8);
      });
      static_for<VIT>([&](auto j) {
        const int it = min(tid + kThreads * (int)j, VITEMS - 1);
        const int q = vquad(it), c8 = it % (D / 8);
#pragma unroll
        for (int kq = 0; kq < 4; ++kq)
          vr[j][kq] = *(const u32x4_t*)(vpre + (long long)(key0 + 4 * q + kq) * D + c8 * 8);
      });
      return;
    }
    static_for<KCH>([&](auto j) {
      const int c = min(tid + kThreads * (int)j, KITEMS - 1);
      const int key = c / (D / 8), dc = c % (D / 8);
      kr[j] = kload(kpre, kcan, k8, ks8, key0 + key, dc * 8);
    });
    static_for<VIT>([&](auto j) {
      const int it = min(tid + kThreads * (int)j, VITEMS - 1);
      const int q = vquad(it), c8 = it % (D / 8);
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
        vr[j][kq] = kload(vpre, vcan, v8, vs8, key0 + 4 * q + kq, c8 * 8);
    });
  };
  auto lstore = [&](int buf) {
    static_for<KCH>([&](auto j) {
      const int c = tid + kThreads * (int)j;
      if (KITEMS % kThreads == 0 || c < KITEMS) {
        const int key = c / (D / 8), dc = c % (D / 8);
        *(u32x4_t*)&Ks[buf][key * KP + dc * 8] = kr[j];
      }
    });
    static_for<VIT>([&](auto j) {
      const int it = tid + kThreads * (int)j;
      if (VITEMS % kThreads == 0 || it < VITEMS) {
        const int q = vquad(it), c8 = it % (D / 8);
        uint16_t* dst = &Vo[buf][(4 * (q >> 3) + (q & 3)) * VO + 4 * ((q >> 2) & 1)];
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          // d = 8 c8 + dd: half dd % 2 of word dd / 2 of the quad's 4 keys
          const int d = 8 * c8 + dd, w = dd >> 1;
          const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
          *(uint2*)(dst + d * 8 + (d / 16) * 8) =
              make_uint2(__builtin_amdgcn_perm(vr[j][1][w], vr[j][0][w], sel),
                         __builtin_amdgcn_perm(vr[j][3][w], vr[j][2][w], sel));
        }
      }
    });
  };

  const float sc = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)
  // m_run: running max of the scaled scores of the lane's column; lacc:
  // the column's running sum of probabilities (as bf16, the values the PV
  // product weights V by), every element alike, formed by the same MFMA
  // with a V operand of ones
  float m_run[QB];
  f32x4_t oacc[QB][DT], lacc[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    lacc[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[qb][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  if (kt_begin < kt_end) {
    gload(kt_begin);
    lstore(0);
  }
  __syncthreads();
  // Two passes over the tiles: first those whose keys every query sees,
  // then the rest (the last tile, or causal), which test each score.  The
  // pass loop unrolls into two copies of the tile body, so the first copy
  // carries no per-score test.
  const int kt_split = min(max(klim_all / KT, kt_begin), kt_end);
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const bool masked = pass == 1;
    for (int kt = pass == 0 ? kt_begin : kt_split;
         kt < (pass == 0 ? kt_split : kt_end); ++kt) {
      const int key0 = kt * KT;
      const int buf = (kt - kt_begin) & 1;
      // next tile's loads (clamped: a redundant valid load on the last tile)
      gload(min(kt + 1, kt_end - 1));
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* ks = Ks[buf];
      const uint16_t* vo = Vo[buf];

      // ---- S^T = K Q^T: lane holds its query column of each block, keys
      // 16*t4 + 4*lg + e
      f32x4_t sacc[QB][4];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sacc[qb][t4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const u32x4_t kf = *(const u32x4_t*)&ks[(t4 * 16 + l16) * KP + dc * 32 + lg * 8];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sacc[qb][t4] = mfma_v(kf, qf[qb][dc], sacc[qb][t4]);
        }
      }

      // ---- online softmax of each column (a column with no visible key so
      // far keeps m = -inf, p = 0 and zero accumulators)
      u32x4_t pf[QB][2];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mt = -INFINITY;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (masked) {
              const int kk = key0 + t4 * 16 + lg * 4 + e;
              if (kk >= klim[qb]) sacc[qb][t4][e] = -INFINITY;
            }
            mt = fmaxf(mt, sacc[qb][t4][e]);
          }
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        mt *= sc;  // sc > 0: the max of the scaled scores
        // raise the running max (and rescale) only when some column of the
        // wave needs it
        if (__builtin_amdgcn_ballot_w64(mt > m_run[qb] + kLazy) != 0) {
          const float m_new = fmaxf(m_run[qb], mt);
          const float alpha =
              m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
          lacc[qb] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oacc[qb][dt] *= alpha;
          m_run[qb] = m_new;
        }
        // exponents are <= kLazy; results below 2^-126 flush to 0 (negligible)
        const float m_use = m_run[qb] == -INFINITY ? 0.f : m_run[qb];
        float p[4][4];
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            p[t4][e] = __builtin_amdgcn_exp2f(fmaf(sacc[qb][t4][e], sc, -m_use));
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
          pf[qb][kc] = u32x4_t{pack_bf2(p[2 * kc][0], p[2 * kc][1]),
                               pack_bf2(p[2 * kc][2], p[2 * kc][3]),
                               pack_bf2(p[2 * kc + 1][0], p[2 * kc + 1][1]),
                               pack_bf2(p[2 * kc + 1][2], p[2 * kc + 1][3])};
      }

      // ---- O^T += V^T P^T.  k-slot 4 h + e of lane group lg is key
      // 32 kc + 16 h + 4 lg + e (h = 0, 1), the order the S^T accumulators
      // hold the probabilities in; the V operand is octet 4 kc + lg at d.
      // The probability sums take a V operand of ones (bf16 1.0).
      constexpr uint32_t kOne2 = 0x3F803F80u;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          lacc[qb] = mfma_v(u32x4_t{kOne2, kOne2, kOne2, kOne2}, pf[qb][kc], lacc[qb]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int d = dt * 16 + l16;
          const u32x4_t vf = *(const u32x4_t*)&vo[(4 * kc + lg) * VO + d * 8 + dt * 8];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][dt] = mfma_v(vf, pf[qb][kc], oacc[qb][dt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // buffer buf ^ 1 was last read in the previous iteration, before the
      // barrier that ended it
      if (kt + 1 < kt_end) lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- finalise: lane holds its query column, d = 16*dt + 4*lg + e
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = lacc[qb][0];  // the whole column's sum in every lane
    if (!qvalid[qb]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (a.splits == 1) {
      uint16_t* op =
          a.out + (long long)(b * C + qpos[qb]) * (a.Hq * D) + qhead[qb] * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t o = oacc[qb][dt];
        *(uint2*)(op + dt * 16) =
            make_uint2(pack_bf2(o[0] * inv, o[1] * inv), pack_bf2(o[2] * inv, o[3] * inv));
      }
    } else {
      const int row_id = (b * a.Hq + qhead[qb]) * C + qpos[qb];
      float* op = a.opart + ((long long)split * n_rows + row_id) * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t o = oacc[qb][dt];
        *(float4*)(op + dt * 16) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
      }
      if (lg == 0)
        a.lpart[(long long)split * n_rows + row_id] =
            l > 0.f ? m_run[qb] + log2f(l) : -INFINITY;
    }
  }
}

// Merge of the KV-split partials: one wave per (canvas, head, position) row;
// the partials of up to 8 splits are loaded together, then added in split
// order.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int PER = D / 64;
  constexpr int U = 8;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_rows = a.n * a.Hq * a.C;
  const int row_id = blockIdx.x * 4 + wave;
  if (row_id >= n_rows) return;
  // lane s holds split s's log-sum (splits <= 64): one load for all of
  // them, the maximum by a wave reduction, split s's value by a broadcast
  const float l_my = a.lpart[(long long)(lane < a.splits ? lane : 0) * n_rows + row_id];
  float mx = lane < a.splits ? l_my : -INFINITY;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  // (a row with no visible key has every split at -inf: all are skipped)
  for (int s0 = 0; s0 < a.splits; s0 += U) {
    float o[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = s0 + u < a.splits ? s0 + u : 0;
      const float* op = a.opart + ((long long)sp * n_rows + row_id) * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[u][e] = op[lane + 64 * e];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = s0 + u;
      if (sp >= a.splits) break;
      const float lsp = __shfl(l_my, sp, 64);
      if (lsp == -INFINITY) continue;
      const float w = exp2f(lsp - mx);
      wsum += w;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += w * o[u][e];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int pos = row_id % a.C;
  const int bh = row_id / a.C;
  const int h = bh % a.Hq, b = bh / a.Hq;
  uint16_t* out = a.out + (long long)(b * a.C + pos) * (a.Hq * D) + h * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[lane + 64 * e] = f2bf(acc[e] * inv);
}

// Splits for qb query blocks per wave: one round of workgroups over the
// 256 CUs, each walking at least 4 key tiles (max_keys > 0).
int splits_for(int qb, int n, int C, int Hq, int Hkv, int max_keys) {
  const int G = Hq / Hkv;
  const int rows = 128 * qb;
  const int natural = n * Hkv * ((G * C + rows - 1) / rows);
  int s = (256 + natural - 1) / natural;
  if (s > 64) s = 64;
  if (max_keys > 0) {
    const int tiles = (max_keys + KT - 1) / KT;
    s = std::min(s, std::max(1, tiles / 4));
  }
  return std::max(s, 1);
}

// Query blocks per wave for a launch: 2 (256 rows per workgroup, half the
// K/V bytes per query row) when the key range is long enough that every
// workgroup still walks >= 8 tiles with the whole chip busy, else 1.
int attn_qb(int n, int C, int Hq, int Hkv, int max_keys) {
  const int G = Hq / Hkv;
  if (max_keys <= 0 || G * C <= 128) return 1;
  const int tiles = (max_keys + KT - 1) / KT;
  return tiles / splits_for(2, n, C, Hq, Hkv, 0) >= 8 ? 2 : 1;
}

}  // namespace

// Splits of a launch over canvases whose longest key range is max_keys;
// max_keys <= 0 asks for the largest count any key range can get (to size
// the partials' workspace).
int attention_auto_splits(int n, int C, int Hq, int Hkv, int max_keys) {
  if (max_keys <= 0)
    return std::max(splits_for(1, n, C, Hq, Hkv, 0), splits_for(2, n, C, Hq, Hkv, 0));
  return splits_for(attn_qb(n, C, Hq, Hkv, max_keys), n, C, Hq, Hkv, max_keys);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  int max_keys = 0;
  for (int b = 0; b < a.n; ++b)
    max_keys = std::max(max_keys, a.plen[b] + (b - a.vis0[b] + 1) * a.C);
  const int qb = attn_qb(a.n, a.C, a.Hq, a.Hkv, max_keys);
  const int n_chunks = (G * a.C + 128 * qb - 1) / (128 * qb);
  const int n_groups = a.Hkv * a.n * a.splits;
  const dim3 grid((unsigned)(((n_groups + 7) / 8) * 8 * n_chunks));
  const bool kv8 = a.ks != nullptr;
  if (kv8 && !a.vs) return hipErrorInvalidValue;
#define DG_ATTN(DD, QQ, K8) \
  hipLaunchKernelGGL((attn_kernel<DD, QQ, K8>), grid, dim3(kThreads), 0, s, a, n_chunks)
  if (a.D == 128) {
    if (kv8) {
      if (qb == 2) DG_ATTN(128, 2, true); else DG_ATTN(128, 1, true);
    } else {
      if (qb == 2) DG_ATTN(128, 2, false); else DG_ATTN(128, 1, false);
    }
  } else {
    if (kv8) {
      if (qb == 2) DG_ATTN(64, 2, true); else DG_ATTN(64, 1, true);
    } else {
      if (qb == 2) DG_ATTN(64, 2, false); else DG_ATTN(64, 1, false);
    }
  }
#undef DG_ATTN
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int n_rows = a.n * a.Hq * a.C;
  if (a.D == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3((n_rows + 3) / 4),
                       dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((n_rows + 3) / 4),
                       dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace dg
