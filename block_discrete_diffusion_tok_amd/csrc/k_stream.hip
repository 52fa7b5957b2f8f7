// Weight-streaming MFMA GEMM for few token rows per weight matrix:
//   C[t][n] = sum_k X[t][k] W[n][k]
// for the tokens t of a group (the rows routed to one expert, or the
// uncommitted rows of the LM head) and every weight row n of that group's
// matrix.  At batch 1 these products move far more weight bytes than they
// compute (a weight element is used by ~16 tokens in the experts, by <= 128
// in the LM head), so the kernel is organised around HBM streaming:
//
//   * each wave owns RT x 16 weight rows and reads them straight from HBM
//     into registers, 64 contiguous bytes per lane per row tile and 128-wide
//     K chunk, two chunks ahead of the MFMAs (weights are used once, so they
//     never pass through LDS);
//   * the group's token rows (gathered through the expert permutation when
//     needed) are staged per K chunk in double-buffered LDS and shared by the
//     4 waves;
//   * MFMA 16x16x32 bf16 with the weights as the A operand, so a lane's
//     accumulators hold one token column and 4 consecutive weight rows: the
//     epilogues (SwiGLU of paired gate/up rows, gate-weight scaling with the
//     scatter back to (token, rank) slots, vocabulary statistics) work on
//     contiguous outputs.
//
// The K-slot permutation: in a K chunk of KC starting at k0, lane group lg
// (lanes 16*lg..16*lg+15) feeds k = k0 + (KC/4)*lg + 8*j + [0, 8) to MFMA
// sub-step j (j = 0..KC/32-1) for both operands, so a lane's weight bytes for
// the chunk are one contiguous run of KC/4 values.  The dot product is the
// same sum in a different order.
#include <math.h>

#include "dg_internal.h"

namespace dg {
namespace {


__device__ __forceinline__ void smerge(float& m, float& s, float& t, int& am,
                                       float m2, float s2, float t2, int am2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
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

// Widen 16 e4m3 bytes (one uint4) to 16 bf16 (two uint4).
__device__ __forceinline__ void widen_e4m3(const uint4 q, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = (uint32_t)e4m3_to_bf(w[i] & 0xff) |
               ((uint32_t)e4m3_to_bf((w[i] >> 8) & 0xff) << 16);
    o[2 * i + 1] = (uint32_t)e4m3_to_bf((w[i] >> 16) & 0xff) |
                   ((uint32_t)e4m3_to_bf(w[i] >> 24) << 16);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// Loads of one K chunk.  Every address is a valid one: rows outside the
// matrix or the token set read a clamped row whose results are never stored,
// so the loads stay plain global loads with no null test (a select between a
// global and a private "zero" would turn them into flat loads, which the
// waitcnt pass can only wait for all at once).
template <int RT, int WREGS, int ESZ, int KC>
__device__ __forceinline__ void load_w(uint4 (&w)[RT][WREGS],
                                       const char* const (&src)[RT], int kc) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q = 0; q < WREGS; ++q)
      w[rt][q] = *(const uint4*)(src[rt] + (long long)kc * KC * ESZ + 16 * q);
}

// Token loads of one K chunk into xr[0..XPT) and their store into an LDS
// buffer, with compile-time indices so that xr stays in registers.
#define DG_LOAD_X(kc)                                                      \
  static_for<XPT>([&](auto j) {                                            \
    xr[j] = *(const u32x4_t*)(xsrc[j] + (kc) * KC);                          \
  });
#define DG_STORE_X(xs)                                                     \
  static_for<XPT>([&](auto j) {                                            \
    const int it = tid + 256 * j;                                          \
    const int row = it / (KC / 8), kc8 = it % (KC / 8);                    \
    *(u32x4_t*)&(xs)[row * XP + kc8 * 8] = xr[j];                            \
  });

template <int RT, int NT, int KC, int XP, int WREGS, bool W8>
__device__ __forceinline__ void mfma_chunk(f32x4_t (&acc)[RT][NT],
                                           const uint4 (&w)[RT][WREGS],
                                           const uint16_t* xs,
                                           int l16, int lg) {
#pragma unroll
  for (int j = 0; j < KC / 32; ++j) {
    uint4 af[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (W8) {
        uint4 lo, hi;
        widen_e4m3(w[rt][j >> 1], lo, hi);
        af[rt] = (j & 1) ? hi : lo;
      } else {
        af[rt] = w[rt][j];
      }
    }
    // Every token tile is computed: tiles past the last token hold clamped
    // (valid) rows whose results the epilogues drop, and a uniform branch
    // here would serialise the LDS reads behind one wait each.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint4 bx = *(const uint4*)&xs[(nt * 16 + l16) * XP + (KC / 4) * lg + 8 * j];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][nt] = mfma16x16x32(af[rt], bx, acc[rt][nt]);
    }
  }
}

template <int RT, int NT, int KC, int EPI, bool W8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void stream_kernel(StreamArgs a) {
  static_assert(RT % 2 == 0, "gate/up pairing needs an even number of row tiles");
  static_assert(KC == 64 || KC == 128, "K chunk");
  constexpr int XP = KC + 8;          // LDS token-row pitch (elements)
  constexpr int WROWS = 4 * RT * 16;  // weight rows per workgroup
  constexpr int ESZ = W8 ? 1 : 2;     // bytes per weight element
  // uint4 per row tile per chunk: a lane's KC/4 contiguous k values
  constexpr int WREGS = (KC / 4) * ESZ / 16;
  constexpr int XITEMS = NT * 16 * (KC / 8);  // 16-byte token items per chunk
  static_assert(XITEMS % 256 == 0, "token items per thread");
  constexpr int XPT = XITEMS / 256;
  __shared__ __attribute__((aligned(16))) uint16_t Xs[2][NT * 16 * XP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int group = blockIdx.y;

  // ---- token rows of this group
  int t_begin, t_end;
  if (a.group_offsets) {
    t_begin = a.group_offsets[group];
    t_end = a.group_offsets[group + 1];
  } else {
    t_begin = 0;
    t_end = a.M;
    if (a.M_dev) t_end = min(t_end, a.M_dev[0]);
  }
  if (t_end <= t_begin) return;

  // ---- this lane's weight rows (r < n_valid) and their source pointers
  const int n_base = blockIdx.x * WROWS;
  const char* wgroup = (const char*)a.W + (long long)group * a.w_group_stride * ESZ;
  const char* wsrc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int r;
    bool ok;
    if (EPI == EPI_SWIGLU) {
      // tiles [0, RT/2) are gate rows of channels c0 + 16*rt + l16, tiles
      // [RT/2, RT) the up rows of the same channels
      const int c0 = blockIdx.x * (WROWS / 2) + wave * (8 * RT);
      const int ch = c0 + (rt % (RT / 2)) * 16 + l16;
      ok = ch < a.ffn;
      r = (rt < RT / 2) ? ch : a.ffn + ch;
    } else {
      r = n_base + (wave * RT + rt) * 16 + l16;
      ok = r < a.N;
    }
    wsrc[rt] = wgroup + ((long long)(ok ? r : 0) * a.K + (KC / 4) * lg) * ESZ;
  }
  const int nk = a.K / KC;

  for (int t0 = t_begin; t0 < t_end; t0 += NT * 16) {
    const int nt_rows = min(NT * 16, t_end - t0);
    const int nt_act = (nt_rows + 15) >> 4;

    const uint16_t* xsrc[XPT];
    const uint16_t* const xbase = a.X;
    const int32_t* const xmap = a.x_map;
    const int xdiv = a.x_map_div, ldx = a.ldx;
    static_for<XPT>([&](auto j) {
      const int it = tid + 256 * j;
      const int row = it / (KC / 8), kc8 = it % (KC / 8);
      const int trow = t0 + (row < nt_rows ? row : 0);
      const int src = xmap ? xmap[trow] / xdiv : trow;
      xsrc[j] = xbase + (long long)src * ldx + kc8 * 8;
    });
    u32x4_t xr[XPT];
    uint4 wa[RT][WREGS], wb[RT][WREGS];

    f32x4_t acc[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // prologue: chunk 0 in wa / Xs[0], chunk 1 in wb
    __syncthreads();  // the previous pass is done with Xs
    load_w<RT, WREGS, ESZ, KC>(wa, wsrc, 0);
    DG_LOAD_X(0);
    DG_STORE_X(Xs[0]);
    load_w<RT, WREGS, ESZ, KC>(wb, wsrc, min(1, nk - 1));
    __syncthreads();
    // Issue order per half step: next token chunk (L2), MFMAs of this
    // chunk, weight chunk two ahead (HBM), then the LDS store of the next
    // token chunk, so that the store waits only for the token loads and the
    // weight loads stay in flight across the next MFMAs.  Chunk indices past
    // the end are clamped to the last chunk (a redundant, valid load) so that
    // the body is straight-line code the compiler cannot regroup.
    const int last = nk - 1;
    for (int kc = 0; kc < nk; kc += 2) {
      // even chunk kc: weights in wa, tokens in Xs[0]
      DG_LOAD_X(min(kc + 1, last));
      __builtin_amdgcn_sched_barrier(0);
      mfma_chunk<RT, NT, KC, XP, WREGS, W8>(acc, wa, Xs[0], l16, lg);
      __builtin_amdgcn_sched_barrier(0);
      load_w<RT, WREGS, ESZ, KC>(wa, wsrc, min(kc + 2, last));
      __builtin_amdgcn_sched_barrier(0);
      DG_STORE_X(Xs[1]);
      __syncthreads();
      if (kc + 1 >= nk) break;
      // odd chunk kc + 1: weights in wb, tokens in Xs[1]
      DG_LOAD_X(min(kc + 2, last));
      __builtin_amdgcn_sched_barrier(0);
      mfma_chunk<RT, NT, KC, XP, WREGS, W8>(acc, wb, Xs[1], l16, lg);
      __builtin_amdgcn_sched_barrier(0);
      load_w<RT, WREGS, ESZ, KC>(wb, wsrc, min(kc + 3, last));
      __builtin_amdgcn_sched_barrier(0);
      DG_STORE_X(Xs[0]);
      __syncthreads();
    }

    // ---- epilogues: lane holds token column t0 + 16*nt + l16 and weight
    // rows 4*lg + e of each row tile
    if (EPI == EPI_LMSTATS) {
      float4* red = (float4*)&Xs[0][0];  // [4 waves][NT*16]
      static_assert(4 * NT * 16 * 16 <= 2 * NT * 16 * XP * 2, "LDS reuse");
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float m = -INFINITY, s = 0.f, t = 0.f;
        int am = 0x7fffffff;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = n_base + (wave * RT + rt) * 16 + 4 * lg + e;
            const float v = acc[rt][nt][e];
            if (n < a.N && v > m) { m = v; am = n; }
          }
        if (m != -INFINITY) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int n = n_base + (wave * RT + rt) * 16 + 4 * lg + e;
              if (n < a.N) {
                const float d = acc[rt][nt][e] - m;
                const float ex = __expf(d);
                s += ex;
                t += ex * d;
              }
            }
        }
#pragma unroll
        for (int off = 16; off < 64; off <<= 1) {
          const float m2 = shfl_xor(m, off), s2 = shfl_xor(s, off);
          const float t2 = shfl_xor(t, off);
          const int am2 = shfl_xor(am, off);
          smerge(m, s, t, am, m2, s2, t2, am2);
        }
        if (lg == 0) red[wave * NT * 16 + nt * 16 + l16] = make_float4(m, s, t, __int_as_float(am));
        if (a.logits) {
          const int tok = t0 + nt * 16 + l16;
          if (tok < t_end) {
            const int lrow = a.row_map ? a.row_map[tok] : tok;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int n = n_base + (wave * RT + rt) * 16 + 4 * lg + e;
                if (n < a.N) a.logits[(long long)lrow * a.N + n] = acc[rt][nt][e];
              }
          }
        }
      }
      __syncthreads();
      if (tid < NT * 16 && t0 + tid < t_end) {
        float4 p = red[tid];
        float m = p.x, s = p.y, t = p.z;
        int am = __float_as_int(p.w);
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const float4 q = red[w * NT * 16 + tid];
          smerge(m, s, t, am, q.x, q.y, q.z, __float_as_int(q.w));
        }
        a.part[(long long)(t0 + tid) * a.n_tiles + blockIdx.x] =
            make_float4(m, s, t, __int_as_float(am));
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tok = t0 + nt * 16 + l16;
        if (nt >= nt_act || tok >= t_end) continue;
        if (EPI == EPI_SWIGLU) {
          const int c0 = blockIdx.x * (WROWS / 2) + wave * (8 * RT);
#pragma unroll
          for (int h = 0; h < RT / 2; ++h) {
            const int ch = c0 + h * 16 + 4 * lg;
            if (ch >= a.ffn) continue;
            float g[4], u[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              g[e] = acc[h][nt][e];
              u[e] = acc[RT / 2 + h][nt][e];
              if (W8) {
                const float* sc = a.w_scale + (long long)group * a.scale_rows;
                g[e] *= sc[ch + e];
                u[e] *= sc[a.ffn + ch + e];
              }
            }
            *(uint2*)((uint16_t*)a.C + (long long)tok * a.ldc + ch) =
                make_uint2(pack_bf2(silu(g[0]) * u[0], silu(g[1]) * u[1]),
                           pack_bf2(silu(g[2]) * u[2], silu(g[3]) * u[3]));
          }
        } else {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int n = n_base + (wave * RT + rt) * 16 + 4 * lg;
            if (n >= a.N) continue;
            f32x4_t v = acc[rt][nt];
            if (EPI == EPI_DOWN) {
              const int pair = a.c_map[tok];
              const float wgt = a.row_scale[pair];
              float sc4[4] = {1.f, 1.f, 1.f, 1.f};
              if (W8) {
                const float* sc = a.w_scale + (long long)group * a.scale_rows + n;
                sc4[0] = sc[0]; sc4[1] = sc[1]; sc4[2] = sc[2]; sc4[3] = sc[3];
              }
              *(float4*)((float*)a.C + (long long)pair * a.ldc + n) =
                  make_float4(v[0] * wgt * sc4[0], v[1] * wgt * sc4[1],
                              v[2] * wgt * sc4[2], v[3] * wgt * sc4[3]);
            } else if (EPI == EPI_STORE_BF16) {
              *(uint2*)((uint16_t*)a.C + (long long)tok * a.ldc + n) =
                  make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
            } else if (EPI == EPI_STORE_F32) {
              *(float4*)((float*)a.C + (long long)tok * a.ldc + n) =
                  make_float4(v[0], v[1], v[2], v[3]);
            } else if (EPI == EPI_ADD_F32) {
              float4* cp = (float4*)((float*)a.C + (long long)tok * a.ldc + n);
              float4 o = *cp;
              o.x += v[0]; o.y += v[1]; o.z += v[2]; o.w += v[3];
              *cp = o;
            }
          }
        }
      }
    }
  }
}

template <int RT, int NT, int KC, int EPI, bool W8>
hipError_t launch_s(const StreamArgs& a, int groups, hipStream_t s) {
  constexpr int WROWS = 4 * RT * 16;
  int grid_x;
  if (EPI == EPI_SWIGLU) grid_x = (a.ffn + WROWS / 2 - 1) / (WROWS / 2);
  else grid_x = (a.N + WROWS - 1) / WROWS;
  if (grid_x <= 0 || groups <= 0) return hipSuccess;
  hipLaunchKernelGGL((stream_kernel<RT, NT, KC, EPI, W8>), dim3(grid_x, groups),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

constexpr int kDenseRT = 2, kMoeRT = 2;
constexpr int kDenseKC = 64, kMoeKC = 128;
int stream_rows_per_wg() { return 4 * kDenseRT * 16; }
int stream_k_chunk() { return kMoeKC > kDenseKC ? kMoeKC : kDenseKC; }

#undef DG_LOAD_X
#undef DG_STORE_X

hipError_t launch_stream(int epi, bool w8, int nt, const StreamArgs& a,
                         int groups, hipStream_t s) {
  if (nt == 8) {
    switch (epi) {
      case EPI_LMSTATS: return launch_s<kDenseRT, 8, kDenseKC, EPI_LMSTATS, false>(a, groups, s);
      case EPI_STORE_BF16: return launch_s<kDenseRT, 8, kDenseKC, EPI_STORE_BF16, false>(a, groups, s);
      case EPI_STORE_F32: return launch_s<kDenseRT, 8, kDenseKC, EPI_STORE_F32, false>(a, groups, s);
      case EPI_ADD_F32: return launch_s<kDenseRT, 8, kDenseKC, EPI_ADD_F32, false>(a, groups, s);
    }
  } else if (nt == 2) {
    switch (epi) {
      case EPI_SWIGLU:
        return w8 ? launch_s<kMoeRT, 2, kMoeKC, EPI_SWIGLU, true>(a, groups, s)
                  : launch_s<kMoeRT, 2, kMoeKC, EPI_SWIGLU, false>(a, groups, s);
      case EPI_DOWN:
        return w8 ? launch_s<kMoeRT, 2, kMoeKC, EPI_DOWN, true>(a, groups, s)
                  : launch_s<kMoeRT, 2, kMoeKC, EPI_DOWN, false>(a, groups, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
