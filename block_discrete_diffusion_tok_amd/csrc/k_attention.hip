// Canvas attention: for each canvas, query head h and canvas position i,
//   o = sum_j softmax_j(q . k_j / sqrt(D)) v_j
// over the request's cached prefix keys followed by the canvas keys (all of
// them, or j <= i in the causal encode pass), KV head h / (Hq / Hkv).
//
// One workgroup (4 waves) takes one KV head of one canvas, 128 query rows
// (the G = Hq / Hkv query heads sharing that KV head x canvas positions) and
// one contiguous range of 64-key tiles (KV split).  K and V tiles are staged
// in LDS and shared by all 128 rows.  Each wave computes S^T = K Q^T for its
// 32 query columns with bf16 MFMA, so that every lane owns exactly one query
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

#include "dg_internal.h"

namespace dg {
namespace {

constexpr int KT = 64;  // keys per tile

template <int D>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  constexpr int KP = D + 8;      // padded K row (elements)
  constexpr int VQ = D * 4 + 4;  // padded key-quad stride (elements)
  constexpr int DC = D / 32;     // 32-wide d chunks (MFMA k for S)
  constexpr int DT = D / 16;     // 16-wide d tiles (MFMA rows for O^T)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vq[(KT / 4) * VQ];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int qt = blockIdx.x, g = blockIdx.y;
  const int b = blockIdx.z / a.splits, split = blockIdx.z % a.splits;
  const int C = a.C, G = a.Hq / a.Hkv;
  const int P = a.plen[b];
  const int N = P + C;
  const int n_rows = a.n * a.Hq * C;

  // ---- this wave's two 16-query column tiles
  uint4 qf[2][DC];
  int qpos[2], qhead[2];
  bool qvalid[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int r = qt * 128 + wave * 32 + ct * 16 + l16;
    qvalid[ct] = r < G * C;
    const int rr = qvalid[ct] ? r : 0;
    qpos[ct] = rr % C;
    qhead[ct] = g * G + rr / C;
    const uint16_t* qp = a.qkv + (long long)(b * C + qpos[ct]) * a.ldqkv +
                         qhead[ct] * D + lg * 8;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[ct][dc] = qvalid[ct] ? *(const uint4*)(qp + dc * 32)
                              : make_uint4(0, 0, 0, 0);
  }

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

  const float sc = 1.4426950408889634f / sqrtf((float)D);  // log2(e)/sqrt(D)
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  f32x4_t oacc[DT][2];
#pragma unroll
  for (int i = 0; i < DT; ++i) {
    oacc[i][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    oacc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int key0 = kt * KT;
    __syncthreads();
    // ---- stage K: 64 keys x D/8 chunks of 16 bytes
#pragma unroll
    for (int j = 0; j < KT * (D / 8) / 256; ++j) {
      const int c = tid + 256 * j;
      const int key = c / (D / 8), dc = c % (D / 8);
      const int kk = key0 + key;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kk < P) v = *(const uint4*)(kpre + (long long)kk * D + dc * 8);
      else if (kk < N) v = *(const uint4*)(kcan + (long long)(kk - P) * a.ldqkv + dc * 8);
      *(uint4*)&Ks[key * KP + dc * 8] = v;
    }
    // ---- stage V as key quads: item = (quad, 4 consecutive d)
#pragma unroll
    for (int j = 0; j < (KT / 4) * (D / 4) / 256; ++j) {
      const int it = tid + 256 * j;
      const int q = it / (D / 4), dq = it % (D / 4);
      uint2 v[4];
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const int kk = key0 + 4 * q + kq;
        v[kq] = make_uint2(0, 0);
        if (kk < P) v[kq] = *(const uint2*)(vpre + (long long)kk * D + dq * 4);
        else if (kk < N)
          v[kq] = *(const uint2*)(vcan + (long long)(kk - P) * a.ldqkv + dq * 4);
      }
      uint16_t* dst = &Vq[q * VQ + dq * 16];
      // d = 4dq + 0 / +1 come from .x (low / high half), +2 / +3 from .y
      *(uint2*)(dst + 0) = make_uint2((v[0].x & 0xffffu) | (v[1].x << 16),
                                      (v[2].x & 0xffffu) | (v[3].x << 16));
      *(uint2*)(dst + 4) = make_uint2((v[0].x >> 16) | (v[1].x & 0xffff0000u),
                                      (v[2].x >> 16) | (v[3].x & 0xffff0000u));
      *(uint2*)(dst + 8) = make_uint2((v[0].y & 0xffffu) | (v[1].y << 16),
                                      (v[2].y & 0xffffu) | (v[3].y << 16));
      *(uint2*)(dst + 12) = make_uint2((v[0].y >> 16) | (v[1].y & 0xffff0000u),
                                       (v[2].y >> 16) | (v[3].y & 0xffff0000u));
    }
    __syncthreads();

    // ---- S^T = K Q^T: lane holds query column, keys 16*t4 + 4*lg + e
    f32x4_t sacc[4][2];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      sacc[t4][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      sacc[t4][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const uint4 kf = *(const uint4*)&Ks[(t4 * 16 + l16) * KP + dc * 32 + lg * 8];
        sacc[t4][0] = mfma16x16x32(kf, qf[0][dc], sacc[t4][0]);
        sacc[t4][1] = mfma16x16x32(kf, qf[1][dc], sacc[t4][1]);
      }
    }

    // ---- online softmax per query column
    uint4 pf[2][2], pl[2][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float sv[4][4];
      float mt = -INFINITY;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = key0 + t4 * 16 + lg * 4 + e;
          const bool vis = kk < N && (!a.causal || kk < P || (kk - P) <= qpos[ct]);
          sv[t4][e] = vis ? sacc[t4][ct][e] * sc : -INFINITY;
          mt = fmaxf(mt, sv[t4][e]);
        }
      mt = fmaxf(mt, shfl_xor(mt, 16));
      mt = fmaxf(mt, shfl_xor(mt, 32));
      const float m_new = fmaxf(m_run[ct], mt);
      float alpha = 1.f;
      float p[4][4];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
          for (int e = 0; e < 4; ++e) p[t4][e] = 0.f;
      } else {
        alpha = exp2f(m_run[ct] - m_new);
        float ls = 0.f;
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[t4][e] = exp2f(sv[t4][e] - m_new);
            ls += p[t4][e];
          }
        l_run[ct] = l_run[ct] * alpha + ls;
      }
      m_run[ct] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt][ct] *= alpha;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int h2 = 0; h2 < 4; ++h2) {
          const float a0 = p[2 * kc + (h2 >> 1)][2 * (h2 & 1)];
          const float a1 = p[2 * kc + (h2 >> 1)][2 * (h2 & 1) + 1];
          const uint16_t b0 = f2bf(a0), b1 = f2bf(a1);
          hi[h2] = (uint32_t)b0 | ((uint32_t)b1 << 16);
          lo[h2] = pack_bf2(a0 - bf2f(b0), a1 - bf2f(b1));
        }
        pf[ct][kc] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        pl[ct][kc] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int d = dt * 16 + l16;
        const uint2 lo = *(const uint2*)&Vq[(8 * kc + lg) * VQ + d * 4];
        const uint2 hi = *(const uint2*)&Vq[(8 * kc + 4 + lg) * VQ + d * 4];
        const uint4 vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
        oacc[dt][0] = mfma16x16x32(vf, pf[0][kc], oacc[dt][0]);
        oacc[dt][1] = mfma16x16x32(vf, pf[1][kc], oacc[dt][1]);
        oacc[dt][0] = mfma16x16x32(vf, pl[0][kc], oacc[dt][0]);
        oacc[dt][1] = mfma16x16x32(vf, pl[1][kc], oacc[dt][1]);
      }
    }
  }

  // ---- finalise: lane holds query column, d = 16*dt + 4*lg + e
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    float l = l_run[ct];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (!qvalid[ct]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (a.splits == 1) {
      uint16_t* op = a.out + (long long)(b * C + qpos[ct]) * (a.Hq * D) +
                     qhead[ct] * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t o = oacc[dt][ct];
        *(uint2*)(op + dt * 16) =
            make_uint2(pack_bf2(o[0] * inv, o[1] * inv), pack_bf2(o[2] * inv, o[3] * inv));
      }
    } else {
      const int row_id = (b * a.Hq + qhead[ct]) * C + qpos[ct];
      float* op = a.opart + ((long long)split * n_rows + row_id) * D + lg * 4;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4_t o = oacc[dt][ct];
        *(float4*)(op + dt * 16) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
      }
      if (lg == 0)
        a.lpart[(long long)split * n_rows + row_id] =
            l > 0.f ? m_run[ct] + log2f(l) : -INFINITY;
    }
  }
}

// Merge of the KV-split partials: one wave per (canvas, head, position) row.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n_rows = a.n * a.Hq * a.C;
  const int row_id = blockIdx.x * 4 + wave;
  if (row_id >= n_rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < a.splits; ++s)
    mx = fmaxf(mx, a.lpart[(long long)s * n_rows + row_id]);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < a.splits; ++s) {
      const float ls = a.lpart[(long long)s * n_rows + row_id];
      if (ls == -INFINITY) continue;
      const float w = exp2f(ls - mx);
      wsum += w;
      const float* op = a.opart + ((long long)s * n_rows + row_id) * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += w * op[lane + 64 * e];
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

int attention_auto_splits(int n, int C, int Hq, int Hkv) {
  const int G = Hq / Hkv;
  const int natural = n * Hkv * ((G * C + 127) / 128);
  int s = (512 + natural - 1) / natural;
  if (s < 1) s = 1;
  if (s > 16) s = 16;
  return s;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  dim3 grid((G * a.C + 127) / 128, a.Hkv, a.n * a.splits);
  if (a.D == 128)
    hipLaunchKernelGGL(attn_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_kernel<64>, grid, dim3(256), 0, s, a);
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
