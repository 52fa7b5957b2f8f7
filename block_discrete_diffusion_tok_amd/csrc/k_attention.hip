// Canvas attention: for each canvas, query head h and canvas position i,
//   o = sum_j softmax_j(q . k_j / sqrt(D)) v_j
// over the request's cached prefix keys followed by the canvas keys (all of
// them, or j <= i in the causal encode pass), KV head h / (Hq / Hkv).
//
// One workgroup (8 waves) takes one KV head of one canvas, 128 query rows
// (the G = Hq / Hkv query heads sharing that KV head x canvas positions) and
// one contiguous range of 64-key tiles (KV split).  K and V tiles are staged
// in double-buffered LDS and shared by all 128 rows; the next tile's global
// loads are issued before the current tile's MFMAs, one barrier per tile.
// Each wave computes S^T = K Q^T for its 16 query columns with bf16 MFMA
// (16 columns per wave keeps registers low enough for two waves per SIMD,
// which hides the LDS and MFMA latencies), so that every lane owns exactly one query
// column: the running max / sum of the online softmax are per-lane scalars
// and the rescale of the output accumulator is a per-lane multiply.  P^T is
// taken straight from the S^T accumulators as the B operand of O^T = V^T P^T;
// V is stored in LDS as key quads ([key/4][d][4]) so that the matching A
// operand is two 8-byte reads.  P enters the MFMA as two bf16 terms,
// P = hi + lo with hi = bf16(P) and lo = bf16(P - hi), so the probabilities
// keep ~16 significant bits instead of 8: rounding P to a single bf16 adds a
// relative error of ~2^-9 per weight, which survives the averaging over keys
// at full size and moves router logits downstream by more than 1e-3.
// Splits write (O / l, log2 l + max) partials that a second kernel merges
// with log-sum-exp weights.
#include <math.h>

#include <algorithm>

#include "dg_internal.h"

namespace dg {
namespace {

constexpr int KT = 64;        // keys per tile
constexpr int kThreads = 512;  // 8 waves of 16 query columns each
constexpr int kRows = 128;     // query rows (head x position) per workgroup

__device__ __forceinline__ f32x4_t mfma_v(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  constexpr int KP = D + 16;     // padded K row (elements; +16 measured ~0.5 us faster than +8)
  constexpr int VQ = D * 4 + 8;  // padded key-quad stride (elements; 16-byte rows)
  constexpr int DC = D / 32;     // 32-wide d chunks (MFMA k for S)
  constexpr int DT = D / 16;     // 16-wide d tiles (MFMA rows for O^T)
  constexpr int KITEMS = KT * (D / 8);           // K 16-byte chunks per tile
  constexpr int KCH = (KITEMS + kThreads - 1) / kThreads;
  constexpr int VITEMS = (KT / 4) * (D / 8);     // V items: 4 keys x 8 d
  constexpr int VIT = (VITEMS + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vq[2][(KT / 4) * VQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int qt = blockIdx.x, g = blockIdx.y;
  const int b = blockIdx.z / a.splits, split = blockIdx.z % a.splits;
  const int C = a.C, G = a.Hq / a.Hkv;
  const int P = a.plen[b];
  const int N = P + C;
  const int n_rows = a.n * a.Hq * C;

  // ---- this wave's 16 query columns: lane's column is row r of the
  // workgroup's 128 (query head g*G + r / C, canvas position r % C)
  const int r = qt * kRows + wave * 16 + l16;
  const bool qvalid = r < G * C;
  const int rr = qvalid ? r : 0;
  const int qpos = rr % C;
  const int qhead = g * G + rr / C;
  u32x4_t qf[DC];
  {
    const uint16_t* qp = a.qkv + (long long)(b * C + qpos) * a.ldqkv + qhead * D + lg * 8;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc] = *(const u32x4_t*)(qp + dc * 32);
  }
  // keys kk < klim are visible to this lane's query (all keys, or the
  // prefix and canvas keys up to the query's own position when causal)
  const int klim = a.causal ? min(N, P + qpos + 1) : N;

  const int n_kt = (N + KT - 1) / KT;
  const int kt_begin = (int)((long long)split * n_kt / a.splits);
  const int kt_end = (int)((long long)(split + 1) * n_kt / a.splits);

  const uint16_t* kpre = a.kc + (long long)a.req[b] * a.req_stride +
                         (long long)g * a.head_stride;
  const uint16_t* vpre = a.vc + (long long)a.req[b] * a.req_stride +
                         (long long)g * a.head_stride;
  const uint16_t* kcan = a.qkv + (long long)(b * C) * a.ldqkv + (a.Hq + g) * D;
  const uint16_t* vcan =
      a.qkv + (long long)(b * C) * a.ldqkv + (a.Hq + a.Hkv + g) * D;
  // Key kk's row (keys past N read the last key: a valid row whose score
  // is masked to -inf, so its probability is exactly 0).
  auto krow = [&](const uint16_t* pre, const uint16_t* can, int kk) {
    kk = min(kk, N - 1);
    return kk < P ? pre + (long long)kk * D : can + (long long)(kk - P) * a.ldqkv;
  };

  // ---- K/V tile staging: global -> registers (issued a tile ahead) ->
  // LDS.  V goes to key quads [key/4][d][4]: an item is 4 keys x 8 d (four
  // 16-byte loads) written as the 8 quads it forms.
  u32x4_t kr[KCH], vr[VIT][4];
  auto gload = [&](int kt) {
    const int key0 = kt * KT;
    static_for<KCH>([&](auto j) {
      const int c = min(tid + kThreads * (int)j, KITEMS - 1);
      const int key = c / (D / 8), dc = c % (D / 8);
      kr[j] = *(const u32x4_t*)(krow(kpre, kcan, key0 + key) + dc * 8);
    });
    static_for<VIT>([&](auto j) {
      const int it = min(tid + kThreads * (int)j, VITEMS - 1);
      const int q = it / (D / 8), c8 = it % (D / 8);
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
        vr[j][kq] = *(const u32x4_t*)(krow(vpre, vcan, key0 + 4 * q + kq) + c8 * 8);
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
        const int q = it / (D / 8), c8 = it % (D / 8);
        uint16_t* dst = &Vq[buf][q * VQ + c8 * 8 * 4];
#pragma unroll
        for (int dp = 0; dp < 4; ++dp) {  // d = 8 c8 + 2 dp, +1
          const uint32_t w0 = vr[j][0][dp], w1 = vr[j][1][dp];
          const uint32_t w2 = vr[j][2][dp], w3 = vr[j][3][dp];
          // quad of d (low halves), then quad of d + 1 (high halves)
          *(u32x4_t*)(dst + dp * 8) =
              u32x4_t{(w0 & 0xffffu) | (w1 << 16), (w2 & 0xffffu) | (w3 << 16),
                      (w0 >> 16) | (w1 & 0xffff0000u), (w2 >> 16) | (w3 & 0xffff0000u)};
        }
      }
    });
  };

  const float sc = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (kt_begin < kt_end) {
    gload(kt_begin);
    lstore(0);
  }
  __syncthreads();
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int key0 = kt * KT;
    const int buf = (kt - kt_begin) & 1;
    // next tile's loads (clamped: a redundant valid load on the last tile)
    gload(min(kt + 1, kt_end - 1));
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* ks = Ks[buf];
    const uint16_t* vq = Vq[buf];

    // ---- S^T = K Q^T: lane holds its query column, keys 16*t4 + 4*lg + e
    f32x4_t sacc[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      sacc[t4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const u32x4_t kf = *(const u32x4_t*)&ks[(t4 * 16 + l16) * KP + dc * 32 + lg * 8];
        sacc[t4] = mfma_v(kf, qf[dc], sacc[t4]);
      }
    }

    // ---- online softmax of the column (branch-free: a column with no
    // visible key so far keeps m = -inf, p = 0, and its zero accumulators)
    float sv[4][4];
    float mt = -INFINITY;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = key0 + t4 * 16 + lg * 4 + e;
        sv[t4][e] = kk < klim ? sacc[t4][e] * sc : -INFINITY;
        mt = fmaxf(mt, sv[t4][e]);
      }
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    // exponents are <= 0; results below 2^-126 flush to 0 (negligible)
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float p[4][4];
    float ls = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[t4][e] = __builtin_amdgcn_exp2f(sv[t4][e] - m_use);
        ls += p[t4][e];
      }
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
    u32x4_t pf[2], pl[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int h2 = 0; h2 < 4; ++h2) {
        const float a0 = p[2 * kc + (h2 >> 1)][2 * (h2 & 1)];
        const float a1 = p[2 * kc + (h2 >> 1)][2 * (h2 & 1) + 1];
        const uint32_t h = pack_bf2(a0, a1);
        hi[h2] = h;
        lo[h2] = pack_bf2(a0 - __uint_as_float(h << 16), a1 - __uint_as_float(h & 0xffff0000u));
      }
      pf[kc] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
      pl[kc] = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int d = dt * 16 + l16;
        const uint2 lo = *(const uint2*)&vq[(8 * kc + lg) * VQ + d * 4];
        const uint2 hi = *(const uint2*)&vq[(8 * kc + 4 + lg) * VQ + d * 4];
        const u32x4_t vf = u32x4_t{lo.x, lo.y, hi.x, hi.y};
        oacc[dt] = mfma_v(vf, pf[kc], oacc[dt]);
        oacc[dt] = mfma_v(vf, pl[kc], oacc[dt]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // buffer buf ^ 1 was last read in the previous iteration, before the
    // barrier that ended it
    if (kt + 1 < kt_end) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- finalise: lane holds its query column, d = 16*dt + 4*lg + e
  float l = l_run;
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  if (!qvalid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (a.splits == 1) {
    uint16_t* op = a.out + (long long)(b * C + qpos) * (a.Hq * D) + qhead * D + lg * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4_t o = oacc[dt];
      *(uint2*)(op + dt * 16) =
          make_uint2(pack_bf2(o[0] * inv, o[1] * inv), pack_bf2(o[2] * inv, o[3] * inv));
    }
  } else {
    const int row_id = (b * a.Hq + qhead) * C + qpos;
    float* op = a.opart + ((long long)split * n_rows + row_id) * D + lg * 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4_t o = oacc[dt];
      *(float4*)(op + dt * 16) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
    }
    if (lg == 0)
      a.lpart[(long long)split * n_rows + row_id] = l > 0.f ? m_run + log2f(l) : -INFINITY;
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
  // lane s holds split s's log-sum (splits <= 32): one load for all of
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

}  // namespace

int attention_auto_splits(int n, int C, int Hq, int Hkv, int max_keys) {
  // one round of workgroups (one per CU: the kernel's registers allow one
  // 4-wave workgroup per CU), each walking at least 4 key tiles
  const int G = Hq / Hkv;
  const int natural = n * Hkv * ((G * C + 127) / 128);
  int s = (256 + natural - 1) / natural;
  if (s > 16) s = 16;
  if (max_keys > 0) {
    const int tiles = (max_keys + KT - 1) / KT;
    s = std::min(s, std::max(1, tiles / 4));
  }
  if (s < 1) s = 1;
  return s;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  dim3 grid((G * a.C + 127) / 128, a.Hkv, a.n * a.splits);
  if (a.D == 128)
    hipLaunchKernelGGL(attn_kernel<128>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_kernel<64>, grid, dim3(kThreads), 0, s, a);
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
