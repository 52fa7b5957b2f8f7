// Tiled bf16 MFMA GEMM  C = A W^T  (A: activations [rows, K]; W: weights
// [N, K]), fp32 accumulation, with the epilogues the denoising step needs:
//   - Q/K/V projection (bf16 out), router logits (fp32 out), output
//     projection added into the fp32 residual stream;
//   - grouped (per-expert) gate/up projection with the SwiGLU product fused
//     and the token rows gathered through the expert permutation;
//   - grouped down projection scaled by the gate weight, rows scattered back
//     to their (token, rank) slot;
//   - tied LM head with the vocabulary statistics fused: per row and tile of
//     vocabulary columns the partial (max, sum e^(z-max), sum e^(z-max)(z-max),
//     argmax), so that logits never have to be written.
// Expert weights may be OCP E4M3 bytes: they are widened to bf16 exactly on
// their way into LDS and the per-row scale is applied in the epilogue.
//
// Workgroup: 256 threads = 4 waves in a 2x2 grid over a BM x BN tile; each
// wave owns (BM/2) x (BN/2) as (BM/32) x (BN/32) MFMA 16x16x32 tiles.
// K is walked in steps of 64 with the next step's global loads issued before
// the current step's MFMAs.
#include <math.h>

#include "dg_internal.h"

namespace dg {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row pitch in elements (144 B)

__device__ __forceinline__ void stats_merge(float& m, float& s, float& t,
                                            int& am, float m2, float s2,
                                            float t2, int am2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both sides empty
  const bool take2 = (m2 > m) || (m2 == m && am2 < am);
  const float d1 = (m == -INFINITY) ? 0.f : (m - mn);
  const float d2 = (m2 == -INFINITY) ? 0.f : (m2 - mn);
  const float e1 = (m == -INFINITY) ? 0.f : __expf(d1);
  const float e2 = (m2 == -INFINITY) ? 0.f : __expf(d2);
  t = e1 * (t + s * d1) + e2 * (t2 + s2 * d2);
  s = s * e1 + s2 * e2;
  if (take2) am = am2;
  m = mn;
}

__device__ __forceinline__ float silu(float v) { return v / (1.f + __expf(-v)); }

template <int BM, int BN, int EPI, bool W8>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];
  constexpr int TM = BM / 32;  // MFMA row tiles per wave (= A chunks/thread)
  constexpr int TN = BN / 32;  // MFMA col tiles per wave (= B chunks/thread)
  constexpr int NB8 = BN / 64; // e4m3 B chunks (16 bytes) per thread

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, lg = lane >> 4;
  const int nt = blockIdx.x, mt = blockIdx.y;

  // ---- which rows this tile covers
  int group = 0, row_begin, row_end;
  if (a.group_offsets) {
    const int total = a.tile_offsets[a.n_groups];
    if (mt >= total) return;
    int lo = 0, hi = a.n_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tile_offsets[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    group = lo;
    row_begin = a.group_offsets[group] + (mt - a.tile_offsets[group]) * BM;
    row_end = a.group_offsets[group + 1];
  } else {
    const int m_rows = a.M_dev ? *a.M_dev : a.M;
    row_begin = mt * BM;
    if (row_begin >= m_rows) return;
    row_end = m_rows;
  }

  // ---- per-thread global source pointers (fixed over K)
  const uint16_t* a_src[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int c = tid + 256 * j, r = c >> 3, kc = c & 7;
    const int row = row_begin + r;
    a_src[j] = nullptr;
    if (row < row_end) {
      const int src = a.a_map ? a.a_map[row] / a.a_map_div : row;
      a_src[j] = a.A + (long long)src * a.lda + kc * 8;
    }
  }
  auto weight_row = [&](int r, bool& ok) -> int {
    if (EPI == EPI_SWIGLU) {
      const int grp = r >> 5, half = (r >> 4) & 1;
      const int ch = nt * (BN / 2) + grp * 16 + (r & 15);
      ok = ch < a.ffn;
      return half ? a.ffn + ch : ch;
    }
    const int wr = nt * BN + r;
    ok = wr < a.N;
    return wr;
  };
  constexpr int NBL = W8 ? NB8 : TN;
  const char* b_src[NBL];
#pragma unroll
  for (int j = 0; j < NBL; ++j) {
    const int c = tid + 256 * j;
    const int r = W8 ? (c >> 2) : (c >> 3);
    const int kc = W8 ? (c & 3) : (c & 7);
    bool ok;
    const int wr = weight_row(r, ok);
    b_src[j] = nullptr;
    if (ok) {
      const long long elem = (long long)group * a.b_group_stride +
                             (long long)wr * a.K + (W8 ? kc * 16 : kc * 8);
      b_src[j] = (const char*)a.B + elem * (W8 ? 1 : 2);
    }
  }

  uint4 ra[TM], rb[NBL];
  const uint4 zero = make_uint4(0, 0, 0, 0);
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < TM; ++j)
      ra[j] = a_src[j] ? *(const uint4*)(a_src[j] + k0) : zero;
#pragma unroll
    for (int j = 0; j < NBL; ++j)
      rb[j] = b_src[j] ? *(const uint4*)(b_src[j] + (long long)k0 * (W8 ? 1 : 2))
                       : zero;
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int c = tid + 256 * j, r = c >> 3, kc = c & 7;
      *(uint4*)&As[r * LDK + kc * 8] = ra[j];
    }
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
      const int c = tid + 256 * j;
      if (W8) {
        const int r = c >> 2, kc = c & 3;
        const uint32_t w[4] = {rb[j].x, rb[j].y, rb[j].z, rb[j].w};
        uint32_t o[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          o[2 * q] = (uint32_t)e4m3_to_bf(w[q] & 0xff) |
                     ((uint32_t)e4m3_to_bf((w[q] >> 8) & 0xff) << 16);
          o[2 * q + 1] = (uint32_t)e4m3_to_bf((w[q] >> 16) & 0xff) |
                         ((uint32_t)e4m3_to_bf(w[q] >> 24) << 16);
        }
        *(uint4*)&Bs[r * LDK + kc * 16] = make_uint4(o[0], o[1], o[2], o[3]);
        *(uint4*)&Bs[r * LDK + kc * 16 + 8] = make_uint4(o[4], o[5], o[6], o[7]);
      } else {
        const int r = c >> 3, kc = c & 7;
        *(uint4*)&Bs[r * LDK + kc * 8] = rb[j];
      }
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / BK;
  gload(0);
  lstore();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const uint4*)&As[(wm * (BM / 2) + i * 16 + l16) * LDK +
                                   ks * 32 + lg * 8];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *(const uint4*)&Bs[(wn * (BN / 2) + j * 16 + l16) * LDK +
                                    ks * 32 + lg * 8];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma16x16x32(af[i], bfr[j], acc[i][j]);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      lstore();
      __syncthreads();
    }
  }

  // ---- epilogues.  Lane holds column l16 of each 16x16 tile, rows 4*lg+i.
  if (EPI == EPI_LMSTATS) {
    float4* red = (float4*)As;  // [2][BM]; the loop ended with a barrier
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r_loc = wm * (BM / 2) + i * 16 + lg * 4 + e;
        const int row = row_begin + r_loc;
        float m = -INFINITY;
        int am = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = nt * BN + wn * (BN / 2) + j * 16 + l16;
          const float v = acc[i][j][e];
          if (col < a.N && v > m) { m = v; am = col; }
          if (a.logits && col < a.N && row < row_end) {
            const int lrow = a.row_map ? a.row_map[row] : row;
            a.logits[(long long)lrow * a.N + col] = v;
          }
        }
        float s = 0.f, t = 0.f;
        if (m != -INFINITY) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = nt * BN + wn * (BN / 2) + j * 16 + l16;
            if (col < a.N) {
              const float d = acc[i][j][e] - m;
              const float ex = __expf(d);
              s += ex;
              t += ex * d;
            }
          }
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
          const float m2 = shfl_xor(m, off), s2 = shfl_xor(s, off);
          const float t2 = shfl_xor(t, off);
          const int am2 = shfl_xor(am, off);
          stats_merge(m, s, t, am, m2, s2, t2, am2);
        }
        if (l16 == 0) red[wn * BM + r_loc] = make_float4(m, s, t, __int_as_float(am));
      }
    }
    __syncthreads();
    if (tid < BM) {
      const int row = row_begin + tid;
      if (row < row_end) {
        float4 p = red[tid];
        const float4 q = red[BM + tid];
        float m = p.x, s = p.y, t = p.z;
        int am = __float_as_int(p.w);
        stats_merge(m, s, t, am, q.x, q.y, q.z, __float_as_int(q.w));
        a.part[(long long)row * a.n_tiles + nt] =
            make_float4(m, s, t, __int_as_float(am));
      }
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row_begin + wm * (BM / 2) + i * 16 + lg * 4 + e;
      if (row >= row_end) continue;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < TN; j += 2) {
          const int grp = (wn * (BN / 2) + j * 16) >> 5;
          const int ch = nt * (BN / 2) + grp * 16 + l16;
          if (ch >= a.ffn) continue;
          float gate = acc[i][j][e], up = acc[i][j + 1][e];
          if (W8) {
            const float* sc = a.b_scale + (long long)group * a.scale_rows;
            gate *= sc[ch];
            up *= sc[a.ffn + ch];
          }
          ((uint16_t*)a.C)[(long long)row * a.ldc + ch] = f2bf(silu(gate) * up);
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = nt * BN + wn * (BN / 2) + j * 16 + l16;
          if (col >= a.N) continue;
          const float v = acc[i][j][e];
          if (EPI == EPI_STORE_BF16) {
            ((uint16_t*)a.C)[(long long)row * a.ldc + col] = f2bf(v);
          } else if (EPI == EPI_STORE_F32) {
            ((float*)a.C)[(long long)row * a.ldc + col] = v;
          } else if (EPI == EPI_ADD_F32) {
            ((float*)a.C)[(long long)row * a.ldc + col] += v;
          } else if (EPI == EPI_DOWN) {
            const int pair = a.c_map[row];
            float y = v * a.row_scale[pair];
            if (W8) y *= a.b_scale[(long long)group * a.scale_rows + col];
            ((float*)a.C)[(long long)pair * a.ldc + col] = y;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int EPI, bool W8>
hipError_t launch_one(const GemmArgs& a, int grid_m, hipStream_t s) {
  int grid_n;
  if (EPI == EPI_SWIGLU) grid_n = (a.ffn + BN / 2 - 1) / (BN / 2);
  else grid_n = (a.N + BN - 1) / BN;
  if (grid_m <= 0 || grid_n <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI, W8>), dim3(grid_n, grid_m),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int gemm_bm(int epi) { return epi == EPI_LMSTATS ? 128 : 64; }
int gemm_bn(int epi) { return epi == EPI_LMSTATS ? 128 : 64; }

hipError_t launch_gemm(int epi, bool w8, const GemmArgs& a, int grid_m,
                       hipStream_t s) {
  switch (epi) {
    case EPI_STORE_BF16: return launch_one<64, 64, EPI_STORE_BF16, false>(a, grid_m, s);
    case EPI_STORE_F32: return launch_one<64, 64, EPI_STORE_F32, false>(a, grid_m, s);
    case EPI_ADD_F32: return launch_one<64, 64, EPI_ADD_F32, false>(a, grid_m, s);
    case EPI_SWIGLU:
      return w8 ? launch_one<64, 64, EPI_SWIGLU, true>(a, grid_m, s)
                : launch_one<64, 64, EPI_SWIGLU, false>(a, grid_m, s);
    case EPI_DOWN:
      return w8 ? launch_one<64, 64, EPI_DOWN, true>(a, grid_m, s)
                : launch_one<64, 64, EPI_DOWN, false>(a, grid_m, s);
    case EPI_LMSTATS: return launch_one<128, 128, EPI_LMSTATS, false>(a, grid_m, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
