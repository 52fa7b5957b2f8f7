// Tiled bf16 MFMA GEMM  C = A W^T  (A: token rows [rows, K]; W: weights
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
// Weights are in the packed (MFMA-tiled) layout of 1 KB blocks, so every
// weight load instruction reads contiguous kilobytes.  Expert weights may be
// OCP E4M3 bytes: they are widened to bf16 exactly on their way into LDS and
// the per-row scale is applied in the epilogue.
//
// Workgroup: 256 threads = 4 waves in a 2x2 grid over a BM (tokens) x BN
// (weight rows) tile; each wave owns (BM/2) x (BN/2) as MFMA 16x16x32 tiles
// with the weights as the A operand, so a lane's accumulators hold one token
// and 4 consecutive output columns (vector stores in every epilogue).
// K is walked in steps of 64 through double-buffered LDS: later steps'
// global loads are issued before the current step's MFMAs and the next
// step is stored into the other buffer after them, one barrier per step.  Every load address is
// valid (rows past the end are clamped and their results dropped), so the
// loads stay plain global loads with per-load waits.
// The loop keeps P K steps of global loads in flight in registers (4 for
// 64x64 tiles, 2 for 128x128), so a workgroup waits about a quarter of a
// memory latency per step instead of a whole one.
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

__device__ __forceinline__ f32x4_t mfma_v(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Global loads of K step kt into staging register set p, and the store of
// set p into LDS buffer b.  Token chunk j of thread tid covers row c/8, 8 k
// values at (c%8)*8 with c = tid + 256 j.  Weight piece c of a K step is
// lane c%64 of packed block c/64: for bf16 the BN/16 row tiles x 2 blocks of
// 32 k values (block b: row tile b/2, k values 32*(b%2) + 8*(lane/16)), for
// e4m3 BN/16 row tiles x 1 block of 64 (k values 16*(lane/16), widened to
// bf16 on the way into LDS); the piece's row is 16 * tile + lane % 16.
#define DG_GLOAD(p, kt)                                                       \
  static_for<XA>([&](auto j) {                                                \
    tr[p][j] = *(const u32x4_t*)(tsrc[j] + (long long)(kt) * BK);             \
  });                                                                         \
  static_for<XB>([&](auto j) {                                                \
    wr[p][j] = *(const u32x4_t*)(wsrc[j] + (long long)(kt) * ESZ * kPackKStride); \
  });
#define DG_LSTORE(b, p)                                                       \
  static_for<XA>([&](auto j) {                                                \
    const int c = tid + 256 * j;                                              \
    *(u32x4_t*)&Ts[b][(c >> 3) * LDK + (c & 7) * 8] = tr[p][j];               \
  });                                                                         \
  static_for<XB>([&](auto j) {                                                \
    const int c = tid + 256 * j, blk = c >> 6, ln = c & 63;                   \
    if (W8) {                                                                 \
      u32x4_t lo, hi;                                                         \
      widen_e4m3x16(wr[p][j], lo, hi);                                              \
      const int o = (blk * 16 + (ln & 15)) * LDK + (ln >> 4) * 16;            \
      *(u32x4_t*)&Ws[b][o] = lo;                                              \
      *(u32x4_t*)&Ws[b][o + 8] = hi;                                          \
    } else {                                                                  \
      const int o = ((blk >> 1) * 16 + (ln & 15)) * LDK + (blk & 1) * 32 + (ln >> 4) * 8; \
      *(u32x4_t*)&Ws[b][o] = wr[p][j];                                        \
    }                                                                         \
  });

template <int BM, int BN, int EPI, bool W8>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
  constexpr int TM = BM / 32;                 // token tiles per wave
  constexpr int TN = BN / 32;                 // weight-row tiles per wave
  constexpr int XA = BM / 32;                 // token 16-byte loads per thread
  constexpr int XB = W8 ? BN / 64 : BN / 32;  // weight 16-byte loads per thread
  constexpr int ESZ = W8 ? 1 : 2;
  static_assert(BM % 32 == 0 && BN % 64 == 0, "tile");
  __shared__ __attribute__((aligned(16))) uint16_t Ts[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Ws[2][BN * LDK];

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

  // ---- K range of this split (router logits: each split writes its own
  // slab; the consumer adds them) and the per-thread source addresses
  const int nk = a.K / BK / (int)gridDim.z;
  const long long k0 = (long long)blockIdx.z * nk * BK;
  if (EPI == EPI_STORE_F32) a.C = (float*)a.C + blockIdx.z * a.split_stride;
  const uint16_t* tsrc[XA];
  const int32_t* const amap = a.a_map;
  static_for<XA>([&](auto j) {
    const int c = tid + 256 * j;
    const int row = min(row_begin + (c >> 3), row_end - 1);
    const int src = amap ? amap[row] / a.a_map_div : row;
    tsrc[j] = a.A + (long long)src * a.lda + k0 + (c & 7) * 8;
  });
  const char* wsrc[XB];
  const char* const wgroup = (const char*)a.B + (long long)group * a.b_group_stride * ESZ;
  static_for<XB>([&](auto j) {
    const int c = tid + 256 * j, blk = c >> 6, ln = c & 63;
    const int tile = W8 ? blk : (blk >> 1);     // 16-row tile within the BN rows
    const int kb = W8 ? 0 : (blk & 1);          // k block within the K step
    int rb;                                     // global 16-row tile
    if (EPI == EPI_SWIGLU) {
      // 16 gate rows then the 16 matching up rows, per 32-row block
      const int cb = min(nt * (BN / 32) + (tile >> 1), a.ffn / 16 - 1);
      rb = (tile & 1) ? a.ffn / 16 + cb : cb;
    } else {
      rb = min(nt * (BN / 16) + tile, (a.N + 15) / 16 - 1);  // zero-padded last tile
    }
    wsrc[j] = wgroup + pack_block_offset(rb, kb, a.K, ESZ) + (k0 / BK) * ESZ * kPackKStride + 16 * ln;
  });

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // P register sets keep the global loads of P K steps in flight (one
  // step's loads alone would leave the loop waiting a full memory latency
  // per step).  Invariant at step k: set (k+1) % P holds step k+1.
  constexpr int P = BM <= 64 ? 4 : 2;
  static_assert(P % 2 == 0, "LDS buffer parity follows the step parity");
  u32x4_t tr[P][XA], wr[P][XB];
  const uint16_t* const tfrag = &Ts[0][(wm * (BM / 2) + l16) * LDK + lg * 8];
  const uint16_t* const wfrag = &Ws[0][(wn * (BN / 2) + l16) * LDK + lg * 8];
  auto compute = [&](int b) {
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      u32x4_t wf[TN], tf[TM];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        wf[j] = *(const u32x4_t*)(wfrag + b * BN * LDK + j * 16 * LDK + ks * 32);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        tf[i] = *(const u32x4_t*)(tfrag + b * BM * LDK + i * 16 * LDK + ks * 32);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_v(wf[j], tf[i], acc[i][j]);
    }
  };

  // Step indices past the end are clamped to the last step (a redundant,
  // valid load) so that the body stays straight-line code.
  const int last = nk - 1;
  static_for<P>([&](auto p) { DG_GLOAD(p, min((int)p, last)); });
  DG_LSTORE(0, 0);
  DG_GLOAD(0, min(P, last));
  __syncthreads();
  // Main loop over whole groups of P steps (straight-line, so the waits
  // before each LDS store cover only the oldest register set), then the
  // remaining nk % P steps.
  auto step = [&](auto p, int kt) {
    constexpr int q = (p + 1) % P;
    __builtin_amdgcn_sched_barrier(0);
    compute(p & 1);
    __builtin_amdgcn_sched_barrier(0);
    DG_LSTORE((p + 1) & 1, q);
    DG_GLOAD(q, min(kt + p + 1 + P, last));
    __syncthreads();
  };
  int kt = 0;
  for (; kt + P <= nk; kt += P)
    static_for<P>([&](auto p) { step(p, kt); });
  if (kt < nk)
    static_for<P - 1>([&](auto p) {
      if (kt + p < nk) step(p, kt);
    });

  // ---- epilogues.  acc[i][j][e]: token row_begin + wm*BM/2 + 16 i + l16,
  // weight row (output column) wn*BN/2 + 16 j + 4 lg + e of the tile.
  if (EPI == EPI_LMSTATS) {
    float4* red = (float4*)&Ts[0][0];  // [2 (wn)][BM]; the loop ended with a barrier
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int t_loc = wm * (BM / 2) + i * 16 + l16;
      const int row = row_begin + t_loc;
      float m = -INFINITY, s = 0.f, t = 0.f;
      int am = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = nt * BN + wn * (BN / 2) + j * 16 + 4 * lg + e;
          const float v = acc[i][j][e];
          if (col < a.N && v > m) { m = v; am = col; }
        }
      if (m != -INFINITY) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int col = nt * BN + wn * (BN / 2) + j * 16 + 4 * lg + e;
            if (col < a.N) {
              const float d = acc[i][j][e] - m;
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
        stats_merge(m, s, t, am, m2, s2, t2, am2);
      }
      if (lg == 0) red[wn * BM + t_loc] = make_float4(m, s, t, __int_as_float(am));
      if (a.logits && row < row_end) {
        const int lrow = a.row_map ? a.row_map[row] : row;
        float* lp = a.logits + (long long)lrow * a.N;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = nt * BN + wn * (BN / 2) + j * 16 + 4 * lg;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < a.N) lp[col + e] = acc[i][j][e];
        }
      }
    }
    __syncthreads();
    if (tid < BM) {
      const int row = row_begin + tid;
      if (row < row_end) {
        const float4 p = red[tid];
        const float4 q = red[BM + tid];
        float m = p.x, s = p.y, t = p.z;
        int am = __float_as_int(p.w);
        stats_merge(m, s, t, am, q.x, q.y, q.z, __float_as_int(q.w));
        a.part[(long long)row * a.n_tiles + nt] = make_float4(m, s, t, __int_as_float(am));
      }
    }
    return;
  }

  const bool vec = ((a.ldc | a.N) & 3) == 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int row = row_begin + wm * (BM / 2) + i * 16 + l16;
    if (row >= row_end) continue;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        // tiles j (gate) and j+1 (up) cover the same 16 channels
        const int ch = nt * (BN / 2) + ((wn * (BN / 2) + j * 16) >> 5) * 16 + 4 * lg;
        if (ch >= a.ffn) continue;  // ffn is a multiple of 64
        float g[4], u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g[e] = acc[i][j][e];
          u[e] = acc[i][j + 1][e];
          if (W8) {
            const float* sc = a.b_scale + (long long)group * a.scale_rows;
            g[e] *= sc[ch + e];
            u[e] *= sc[a.ffn + ch + e];
          }
        }
        *(uint2*)((uint16_t*)a.C + (long long)row * a.ldc + ch) =
            make_uint2(pack_bf2(silu(g[0]) * u[0], silu(g[1]) * u[1]),
                       pack_bf2(silu(g[2]) * u[2], silu(g[3]) * u[3]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = nt * BN + wn * (BN / 2) + j * 16 + 4 * lg;
        if (n >= a.N) continue;
        f32x4_t v = acc[i][j];
        if (W8 && EPI != EPI_DOWN) {
          // dense e4m3 product: the weight rows' scales and the token
          // row's (a_scale, when its values are E4M3 codes)
          const float xs = a.a_scale ? a.a_scale[row] : 1.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= a.b_scale[min(n + e, a.N - 1)] * xs;
        }
        if (EPI == EPI_DOWN) {
          // N (hidden) is a multiple of 64 on this path
          const int pair = a.c_map[row];
          const float wgt = a.row_scale[pair];
          float sc4[4] = {1.f, 1.f, 1.f, 1.f};
          if (W8) {
            const float* sc = a.b_scale + (long long)group * a.scale_rows + n;
            sc4[0] = sc[0]; sc4[1] = sc[1]; sc4[2] = sc[2]; sc4[3] = sc[3];
          }
          *(float4*)((float*)a.C + (long long)pair * a.ldc + n) =
              make_float4(v[0] * wgt * sc4[0], v[1] * wgt * sc4[1],
                          v[2] * wgt * sc4[2], v[3] * wgt * sc4[3]);
        } else if (vec) {
          if (EPI == EPI_STORE_BF16) {
            *(uint2*)((uint16_t*)a.C + (long long)row * a.ldc + n) =
                make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
          } else if (EPI == EPI_STORE_F32) {
            *(float4*)((float*)a.C + (long long)row * a.ldc + n) =
                make_float4(v[0], v[1], v[2], v[3]);
          } else if (EPI == EPI_ADD_F32) {
            float4* cp = (float4*)((float*)a.C + (long long)row * a.ldc + n);
            float4 o = *cp;
            o.x += v[0]; o.y += v[1]; o.z += v[2]; o.w += v[3];
            *cp = o;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e >= a.N) break;
            const long long o = (long long)row * a.ldc + n + e;
            if (EPI == EPI_STORE_BF16) ((uint16_t*)a.C)[o] = f2bf(v[e]);
            else if (EPI == EPI_STORE_F32) ((float*)a.C)[o] = v[e];
            else if (EPI == EPI_ADD_F32) ((float*)a.C)[o] += v[e];
          }
        }
      }
    }
  }
}

#undef DG_GLOAD
#undef DG_LSTORE

template <int BM, int BN, int EPI, bool W8>
hipError_t launch_one(const GemmArgs& a, int grid_m, hipStream_t s) {
  int grid_n;
  if (EPI == EPI_SWIGLU) grid_n = (a.ffn + BN / 2 - 1) / (BN / 2);
  else grid_n = (a.N + BN - 1) / BN;
  if (grid_m <= 0 || grid_n <= 0) return hipSuccess;
  const int splits = (EPI == EPI_STORE_F32 && a.splits > 1) ? a.splits : 1;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, EPI, W8>), dim3(grid_n, grid_m, splits),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int gemm_bm(int epi) { return epi == EPI_LMSTATS ? 128 : 64; }
int gemm_bn(int epi) { return epi == EPI_LMSTATS ? 128 : 64; }

// Dense products whose 64 x 64 tiles would leave most CUs without a
// workgroup (a few hundred token rows) run 32 x 64 tiles instead.
static bool small_dense(const GemmArgs& a, int grid_m) {
  const long long tiles = (long long)grid_m * ((a.N + 63) / 64) * (a.splits > 1 ? a.splits : 1);
  return a.group_offsets == nullptr && !a.M_dev && tiles < 192;
}

// Dense products over thousands of token rows run on the large-tile
// kernel (k_mm.hip): its 256 x 256 tiles read each operand byte from L2
// 4x less often per flop than the 64 x 64 tiles here.
static bool use_mm_dense(int epi, const GemmArgs& a) {
  return a.group_offsets == nullptr && !a.M_dev && (a.splits <= 1) &&
         a.M >= 1024 && a.N >= 256 &&
         (epi == EPI_STORE_BF16 || epi == EPI_STORE_F32 || epi == EPI_ADD_F32);
}

bool gemm_dense_on_mm(int epi, const GemmArgs& a) { return use_mm_dense(epi, a); }

hipError_t launch_gemm(int epi, bool w8, const GemmArgs& a, int grid_m,
                       hipStream_t s) {
  if (use_mm_dense(epi, a)) return launch_mm(epi, w8, a, (a.M + mm_bm() - 1) / mm_bm(), s);
  const int grid_m32 = (a.M + 31) / 32;
  switch (epi) {
    // (dense e4m3 weights: scales from b_scale and, when given, a_scale)
    case EPI_STORE_BF16:
      if (w8)
        return small_dense(a, grid_m) ? launch_one<32, 64, EPI_STORE_BF16, true>(a, grid_m32, s)
                                      : launch_one<64, 64, EPI_STORE_BF16, true>(a, grid_m, s);
      return small_dense(a, grid_m) ? launch_one<32, 64, EPI_STORE_BF16, false>(a, grid_m32, s)
                                    : launch_one<64, 64, EPI_STORE_BF16, false>(a, grid_m, s);
    case EPI_STORE_F32:
      if (w8)
        return small_dense(a, grid_m) ? launch_one<32, 64, EPI_STORE_F32, true>(a, grid_m32, s)
                                      : launch_one<64, 64, EPI_STORE_F32, true>(a, grid_m, s);
      return small_dense(a, grid_m) ? launch_one<32, 64, EPI_STORE_F32, false>(a, grid_m32, s)
                                    : launch_one<64, 64, EPI_STORE_F32, false>(a, grid_m, s);
    case EPI_ADD_F32:
      if (w8)
        return small_dense(a, grid_m) ? launch_one<32, 64, EPI_ADD_F32, true>(a, grid_m32, s)
                                      : launch_one<64, 64, EPI_ADD_F32, true>(a, grid_m, s);
      return small_dense(a, grid_m) ? launch_one<32, 64, EPI_ADD_F32, false>(a, grid_m32, s)
                                    : launch_one<64, 64, EPI_ADD_F32, false>(a, grid_m, s);
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
