// Large-tile bf16 MFMA GEMM  C = A W^T  for the MFMA-bound shapes: many
// token rows per weight matrix (a batch of canvases: the dense projections
// at thousands of rows, the grouped expert GEMMs at hundreds of rows per
// expert, the LM head over thousands of rows).
//
// A workgroup (8 waves) computes a 256 (weight rows) x 256 (token rows)
// tile; wave (wn, wt) owns 128 weight rows x 64 tokens, 32 accumulator
// tiles of MFMA 16x16x32 with the weights as the A operand, so a lane's
// accumulators hold one token and 4 consecutive output columns (as in the
// other GEMM kernels, every epilogue stores contiguous outputs).  Both
// operands go HBM/L2 -> LDS by LDS-DMA (global_load_lds_dwordx4, no
// registers), each instruction moving one MFMA operand block of 1 KB:
//   - weights: the packed layout already stores 1 KB blocks in operand
//     order, so a wave copies whole blocks;
//   - tokens: lane l of a block loads the 16 bytes of token row t0 + l % 16
//     at the block's k offset + 8 (l / 16), which is the B operand's order;
//     token rows may be gathered (an expert's rows through the
//     permutation), since each lane names its own address.
// Every LDS read is a ds_read_b128 of 64 consecutive 16-byte pieces (no
// bank conflicts, no padding).  K is walked through NS LDS stages (bf16:
// 4 stages of 32 k, 32 KB each; e4m3 weights: 3 of 64 k, 48 KB; e4m3
// tokens: 2 of 128 k, 64 KB): step s + NS - 1's DMA is issued after the
// barrier that opens step s.  With bf16 weights the operand fragments of
// step s + 1 are read from LDS while step s's MFMAs run.  Each wave issues
// 32 MFMAs per 32 k against 12 KB of LDS reads.
//
// E4M3 weights: a packed e4m3 block holds 16 rows x 64 k; lane l's 16
// bytes are k 16 (l/16) .. +15 of row l % 16, widened to bf16 in registers
// (exact) as the A operand of two MFMAs: k 16 (l/16) + [0, 8) and
// 16 (l/16) + 8 + [0, 8); the token blocks of an e4m3 step use the same k
// assignment.  The per-row scale is applied in the epilogue.
#include <math.h>

#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kMmThreads = 512;
constexpr int kMmBN = 256;   // weight rows per workgroup
constexpr int kMmBM = 256;   // token rows per workgroup
constexpr int kMmBK = 64;    // k per step of the e4m3-weight path (32 bf16, 128 FP8)
constexpr int kSwzM = 8;     // token tiles per block of the tile order

__device__ __forceinline__ f32x4_t mfma_v(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef int i32x8_t __attribute__((ext_vector_type(8)));
// FP8 MFMA: D(16x16) += A(16x128) * B(128x16), both E4M3 (format 0), unit
// block scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x4_t mfma_f8(const i32x8_t a, const i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

#ifndef DG_LDS_PTR
#define DG_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#endif
__device__ __forceinline__ void dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, DG_LDS_PTR(lds_wave_base), 16, 0, 0);
}

// s_waitcnt immediate: vmcnt(n), the other counters untouched
constexpr int vm_wait_imm(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

// merge of two (max, sum e^(z-max), sum e^(z-max)(z-max), argmax) partials
__device__ __forceinline__ void mm_stats_merge(float& m, float& s, float& t, int& am,
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

__device__ __forceinline__ float mm_silu(float v) { return v / (1.f + __expf(-v)); }

// A8: token rows are E4M3 codes (a.A8) with a per-row scale (a.a_scale),
// e4m3 weights, the FP8 MFMA 16x16x128 (k 128 per step).
template <int EPI, bool W8, bool A8 = false>
__global__ __launch_bounds__(kMmThreads) void mm_kernel(GemmArgs a) {
  static_assert(!A8 || W8, "e4m3 tokens need e4m3 weights");
  // k per step: 32 (bf16: one 1 KB block per row tile and per token tile),
  // 64 (e4m3 weights: one block per row tile, two per token tile), 128
  // (e4m3 tokens: two of each)
  constexpr int BK = A8 ? 2 * kMmBK : (W8 ? kMmBK : kMmBK / 2);
  constexpr int ESZ = W8 ? 1 : 2;
  constexpr int WBLK = 16 * (BK * ESZ / 64);      // weight blocks per step (16 / 16 / 32)
  constexpr int TBLK = 16 * (W8 ? 2 : 1);         // token blocks per step (16 tiles x 1 or 2)
  constexpr int WPW = WBLK / 8, TPW = TBLK / 8;   // DMA instructions per wave
  constexpr int LOADS = WPW + TPW;
  constexpr int STAGE = (WBLK + TBLK) * 1024;     // bytes per LDS stage (32 / 48 / 64 KB)
  // LDS stages (128 / 144 / 128 KB): step s + NS - 1's DMA is issued when
  // step s begins, so a stage's loads have NS - 1 steps of MFMAs to land
  constexpr int NS = A8 ? 2 : (W8 ? 3 : 4);
  __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int wn = wave & 1, wt = wave >> 1;        // 2 x 4 waves
  // ---- tile of this workgroup.  Workgroups are dealt to the 8 XCDs
  // round-robin by linear id, each XCD with its own L2.  Tiles are ordered
  // in blocks of kSwzM token tiles (for each block, every weight tile, for
  // each the block's token tiles) and each XCD runs one contiguous run of
  // that order: the ~32 tiles an XCD has in flight are ~4 weight tiles x 8
  // token tiles, so each operand tile comes into its L2 once for several
  // workgroups instead of once per workgroup.
  // The order covers only the tiles that hold rows (the grid is sized for
  // the most the device-side row counts allow): an expert GEMM's tile count
  // and a live-row count are read first, and the workgroups past them leave,
  // so the work spreads evenly over the XCDs.
  int nt, mt;
  {
    const int gn = gridDim.x;
    int gm = gridDim.y;
    if (a.group_offsets) {
      gm = min(gm, a.tile_offsets[a.n_groups]);
    } else if (a.M_dev) {
      const int m_rows = min(*a.M_dev, a.M);
      if (m_rows <= a.rows_gt) return;   // another kernel's rows
      gm = min(gm, (m_rows + kMmBM - 1) / kMmBM);
    }
    const int total = gn * gm;
    const int lin = blockIdx.x + gn * blockIdx.y;
    if (lin >= total) return;
    const int x = lin & 7, q = total >> 3, r = total & 7;
    const int o = x * q + min(x, r) + (lin >> 3);
    const int bm = min(kSwzM, gm);
    const int tb = o / (gn * bm);
    const int rem = o - tb * gn * bm;
    const int rows_in = min(bm, gm - tb * bm);
    nt = rem / rows_in;
    mt = tb * bm + rem % rows_in;
  }

  // ---- which token rows this tile covers
  int group = 0, row_begin, row_end;
  if (a.group_offsets) {
    int lo = 0, hi = a.n_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tile_offsets[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    group = lo;
    row_begin = a.group_offsets[group] + (mt - a.tile_offsets[group]) * kMmBM;
    row_end = a.group_offsets[group + 1];
  } else {
    const int m_rows = a.M_dev ? min(*a.M_dev, a.M) : a.M;
    row_begin = mt * kMmBM;
    if (row_begin >= m_rows) return;
    row_end = m_rows;
  }

  // ---- per-lane DMA sources.  Token block (tt, h) of a step: token tile
  // tt (rows row_begin + 16 tt + l16, clamped), k offset 32 h + 8 lg
  // (bf16 weights) or 16 lg + 8 h (e4m3 weights).  Wave w copies token
  // blocks w*TPW .. +TPW-1 and weight blocks w*WPW .. +WPW-1.
  // (e4m3 tokens: k offset 64 h + 16 lg, in bytes)
  const char* tsrc[TPW];
  static_for<TPW>([&](auto j) {
    const int blk = wave * TPW + j;
    const int tt = TBLK == 16 ? blk : blk >> 1, h = TBLK == 16 ? 0 : blk & 1;
    const int row = min(row_begin + 16 * tt + l16, row_end - 1);
    const int src = a.a_map ? a.a_map[row] / a.a_map_div : row;
    if (A8) {
      tsrc[j] = (const char*)a.A8 + (long long)src * a.lda + 64 * h + 16 * lg;
    } else {
      const int koff = W8 ? 16 * lg + 8 * h : 32 * h + 8 * lg;
      tsrc[j] = (const char*)(a.A + (long long)src * a.lda + koff);
    }
  });
  // Weight block (rt, kb) of a step: row tile rt of the workgroup's 16,
  // k block kb of the step (bf16: 2 per step, e4m3: 1, e4m3 with e4m3
  // tokens: 2).
  const char* wsrc[WPW];
  const char* const wgroup = (const char*)a.B + (long long)group * a.b_group_stride * ESZ;
  const int KB = a.K * ESZ / 64;   // packed blocks per row tile
  static_for<WPW>([&](auto j) {
    const int blk = wave * WPW + j;
    const int rt = WBLK == 16 ? blk : (blk >> 1);
    const int kb = WBLK == 16 ? 0 : (blk & 1);
    int rb;
    if (EPI == EPI_SWIGLU) {
      // 16 gate rows then the 16 matching up rows, per 32-row block
      const int cb = min(nt * (kMmBN / 32) + (rt >> 1), a.ffn / 16 - 1);
      rb = (rt & 1) ? a.ffn / 16 + cb : cb;
    } else {
      rb = min(nt * (kMmBN / 16) + rt, (a.N + 15) / 16 - 1);
    }
    wsrc[j] = wgroup + (((long long)(rb / kPackTiles) * KB + kb) * kPackTiles + rb % kPackTiles) *
                           kPackBlock + 16 * lane;
  });
  // bytes between consecutive steps of one weight block stream
  constexpr long long kWStep = (long long)(BK * ESZ / 64) * kPackKStride;

  auto issue = [&](int step, int stage) {
    char* st = lds + stage * STAGE;
    static_for<WPW>([&](auto j) {
      dma16(wsrc[j] + step * kWStep, st + (wave * WPW + j) * 1024);
    });
    // (BK values of every token row per step: 64 or 128 bytes)
    static_for<TPW>([&](auto j) {
      dma16(tsrc[j] + (long long)step * (BK * (A8 ? 1 : 2)), st + (WBLK + wave * TPW + j) * 1024);
    });
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / BK;
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nk) issue(s, s);
  if constexpr (!W8) {
    // bf16: step k + 1's fragments are read from LDS while step k's MFMAs
    // run (two register sets, indexed by the step's parity; the loop takes
    // steps in pairs so that the index is a constant).  Before the reads,
    // this wave's DMA for step k + 1 has landed (issued NS - 2 steps
    // earlier; those of the later steps may still be in flight) and the
    // barrier makes every wave's visible; the stage refilled after it,
    // step k - 1's, was read before the previous barrier.
    u32x4_t wf[2][8], tf[2][4];
    auto frags = [&](auto b, int k) {
      const char* st = lds + (k % NS) * STAGE;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        wf[b][i] = *(const u32x4_t*)(st + (wn * 8 + i) * 1024 + 16 * lane);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        tf[b][j] = *(const u32x4_t*)(st + (WBLK + wt * 4 + j) * 1024 + 16 * lane);
    };
    // step k's DMA visible to every wave, with the steps up to `last`
    // issued: this wave's DMAs of the steps after k may stay in flight
    static_assert(NS <= 4, "at most two later steps in flight");
    auto sync = [&](int k, int last) {
      const int later = min(last, nk - 1) - k;
      if (later >= 2)
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(2 * LOADS));
      else if (later == 1)
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(LOADS));
      else
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    sync(0, NS - 2);
    frags(std::integral_constant<int, 0>(), 0);
    for (int ks = 0; ks < nk; ks += 2) {
      static_for<2>([&](auto b) {
        const int k = ks + (int)b;
        if (k < nk) {
          if (k + 1 < nk) {
            __builtin_amdgcn_sched_barrier(0);
            sync(k + 1, k + NS - 2);
            if (k + NS - 1 < nk) issue(k + NS - 1, (k + NS - 1) % NS);
            __builtin_amdgcn_sched_barrier(0);
            frags(std::integral_constant<int, 1 - decltype(b)::value>(), k + 1);
          }
#pragma unroll
          for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_v(wf[b][i], tf[b][j], acc[i][j]);
        }
      });
    }
  } else
  for (int ks = 0; ks < nk; ++ks) {
    // this wave's DMA for step ks has landed (its DMAs complete in issue
    // order; those of the NS - 2 later steps may still be in flight); the
    // barrier makes every wave's visible and ends every wave's reads of
    // step ks - 1's stage, which step ks + NS - 1 then refills
    if (ks + NS - 2 < nk)
      __builtin_amdgcn_s_waitcnt(vm_wait_imm((NS - 2) * LOADS));
    else
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (ks + NS - 1 < nk) issue(ks + NS - 1, (ks + NS - 1) % NS);
    __builtin_amdgcn_sched_barrier(0);
    const char* st = lds + (ks % NS) * STAGE;
    if (A8) {
      // one 128-k FP8 MFMA per tile pair: a lane's 32 bytes are k
      // 16 lg + [0, 16) (block 0) and 64 + 16 lg + [0, 16) (block 1) of
      // both operands (any k-slot assignment works when A and B share it)
      i32x8_t tf8[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tt = wt * 4 + j;
        const u32x4_t lo = *(const u32x4_t*)(st + (WBLK + tt * 2) * 1024 + 16 * lane);
        const u32x4_t hi = *(const u32x4_t*)(st + (WBLK + tt * 2 + 1) * 1024 + 16 * lane);
        tf8[j] = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                         (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rt = wn * 8 + i;
        const u32x4_t lo = *(const u32x4_t*)(st + (rt * 2) * 1024 + 16 * lane);
        const u32x4_t hi = *(const u32x4_t*)(st + (rt * 2 + 1) * 1024 + 16 * lane);
        const i32x8_t wf8 = i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f8(wf8, tf8[j], acc[i][j]);
      }
      continue;
    }
    // 32-k MFMA sub-steps: one (bf16), two (e4m3 weights: the two halves
    // of each widened block)
#pragma unroll
    for (int h = 0; h < BK / 32; ++h) {
      u32x4_t wf[8], tf[4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int rt = wn * 8 + i;
        if (W8) {
          const u32x4_t q = *(const u32x4_t*)(st + rt * 1024 + 16 * lane);
          u32x4_t lo, hi;
          widen_e4m3x16(q, lo, hi);
          wf[i] = h ? hi : lo;
        } else {
          wf[i] = *(const u32x4_t*)(st + rt * 1024 + 16 * lane);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tt = wt * 4 + j;
        tf[j] = *(const u32x4_t*)(st + (WBLK + tt * (TBLK / 16) + h) * 1024 + 16 * lane);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_v(wf[i], tf[j], acc[i][j]);
    }
  }

  // ---- epilogues.  acc[i][j][e]: token row_begin + 64 wt + 16 j + l16,
  // weight row (output column) 128 wn + 16 i + 4 lg + e of the tile.
  if (epi_is_lm(EPI)) {
    // each wave holds a full 128-row half of the tile for its 64 tokens:
    // its partial is the tile half's (index 2 nt + wn of the row's
    // ceil(N / 128) partials).  EPI_LMSAMPLE: statistics of z / tau and the
    // Gumbel-max token of the half (see LmSample).
    constexpr bool smp = EPI == EPI_LMSAMPLE;
    const int half = nt * 2 + wn;
    // E4M3 head: each logit is scaled by its vocabulary row's scale and its
    // token row's scale first (every statistic below is of the scaled z)
    float wsc[8][4];
    if (A8) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          wsc[i][e] = a.b_scale[min(half * 128 + i * 16 + 4 * lg + e, a.N - 1)];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = row_begin + wt * 64 + j * 16 + l16;
      const int srow = min(row, row_end - 1);
      if (A8) {
        const float xs = a.a_scale[srow];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][e] *= wsc[i][e] * xs;
      }
      float tau = 1.f;
      uint32_t c1 = 0, c2 = 0, c3 = 0;
      if (smp) {
        tau = a.smp.tau[srow];
        c1 = a.smp.ctr[3 * srow];
        c2 = a.smp.ctr[3 * srow + 1];
        c3 = a.smp.ctr[3 * srow + 2];
      }
      const float scale = tau > 0.f ? 1.f / tau : 1.f;
      float m = -INFINITY, s = 0.f, t = 0.f;
      int am = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = half * 128 + i * 16 + 4 * lg + e;
          const float v = smp ? acc[i][j][e] * scale : acc[i][j][e];
          if (col < a.N && v > m) { m = v; am = col; }
        }
      if (m != -INFINITY) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int col = half * 128 + i * 16 + 4 * lg + e;
            if (col < a.N) {
              const float v = smp ? acc[i][j][e] * scale : acc[i][j][e];
              const float d = v - m;
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
        mm_stats_merge(m, s, t, am, m2, s2, t2, am2);
      }
      float g = -INFINITY;
      int gi = 0x7fffffff;
      if (smp) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int n0 = half * 128 + i * 16 + 4 * lg;
          uint32_t c[4] = {(uint32_t)n0 >> 2, c1, c2, c3};
          if (tau > 0.f) philox4x32_10(c, a.smp.key0, a.smp.key1);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n0 + e >= a.N) continue;
            const float v = acc[i][j][e] * scale;
            best_merge(g, gi, tau > 0.f ? v + gumbel_of(c[e]) : v, n0 + e);
          }
        }
#pragma unroll
        for (int off = 16; off < 64; off <<= 1)
          best_merge(g, gi, shfl_xor(g, off), shfl_xor(gi, off));
      }
      if (row >= row_end) continue;
      if (lg == 0 && half < a.n_tiles) {
        a.part[(long long)row * a.n_tiles + half] = make_float4(m, s, t, __int_as_float(am));
        if (smp)
          a.smp.spart[(long long)row * a.n_tiles + half] = make_float2(g, __int_as_float(gi));
      }
      if (a.logits) {
        const int lrow = a.row_map ? a.row_map[row] : row;
        float* lp = a.logits + (long long)lrow * a.N;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int col = half * 128 + i * 16 + 4 * lg;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < a.N) lp[col + e] = acc[i][j][e];
        }
      }
    }
    return;
  }

  const bool vec = ((a.ldc | a.N) & 3) == 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = row_begin + wt * 64 + j * 16 + l16;
    if (row >= row_end) continue;
    // e4m3 tokens: the row's scale (of its source row)
    const float xs = A8 ? a.a_scale[a.a_map ? a.a_map[row] / a.a_map_div : row] : 1.f;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        // tiles i (gate) and i + 1 (up) cover the same 16 channels
        const int ch = nt * (kMmBN / 2) + ((wn * 128 + i * 16) >> 5) * 16 + 4 * lg;
        if (ch >= a.ffn) continue;  // ffn is a multiple of 64
        float g[4], u[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g[e] = acc[i][j][e];
          u[e] = acc[i + 1][j][e];
          if (W8) {
            const float* sc = a.b_scale + (long long)group * a.scale_rows;
            g[e] *= sc[ch + e];
            u[e] *= sc[a.ffn + ch + e];
          }
          if (A8) {
            g[e] *= xs;
            u[e] *= xs;
          }
        }
        *(uint2*)((uint16_t*)a.C + (long long)row * a.ldc + ch) =
            make_uint2(pack_bf2(mm_silu(g[0]) * u[0], mm_silu(g[1]) * u[1]),
                       pack_bf2(mm_silu(g[2]) * u[2], mm_silu(g[3]) * u[3]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int n = nt * kMmBN + wn * 128 + i * 16 + 4 * lg;
        if (n >= a.N) continue;
        f32x4_t v = acc[i][j];
        if (A8 && EPI != EPI_DOWN) {
          // dense W8A8 product: the weight rows' scales and the token row's
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
          const float ws = A8 ? wgt * xs : wgt;
          *(float4*)((float*)a.C + (long long)pair * a.ldc + n) =
              make_float4(v[0] * ws * sc4[0], v[1] * ws * sc4[1],
                          v[2] * ws * sc4[2], v[3] * ws * sc4[3]);
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

template <int EPI, bool W8, bool A8 = false>
hipError_t launch_mm_one(const GemmArgs& a, int grid_m, hipStream_t s) {
  int grid_n;
  if (EPI == EPI_SWIGLU) grid_n = (a.ffn + kMmBN / 2 - 1) / (kMmBN / 2);
  else grid_n = (a.N + kMmBN - 1) / kMmBN;
  if (grid_m <= 0 || grid_n <= 0) return hipSuccess;
  if (a.K % (A8 ? 2 * kMmBK : kMmBK)) return hipErrorInvalidValue;
  if (A8 && (!a.A8 || !a.a_scale || a.lda % 16)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mm_kernel<EPI, W8, A8>), dim3(grid_n, grid_m), dim3(kMmThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int mm_bm() { return kMmBM; }
int mm_bn() { return kMmBN; }

hipError_t launch_mm(int epi, bool w8, const GemmArgs& a, int grid_m, hipStream_t s) {
  if (a.splits > 1) return hipErrorInvalidValue;
  switch (epi) {
    // (dense e4m3 weights take E4M3 token rows: W8A8 on the FP8 MFMA)
    case EPI_STORE_BF16:
      if (w8) return a.A8 ? launch_mm_one<EPI_STORE_BF16, true, true>(a, grid_m, s)
                          : hipErrorInvalidValue;
      return launch_mm_one<EPI_STORE_BF16, false>(a, grid_m, s);
    case EPI_STORE_F32:
      if (w8) return a.A8 ? launch_mm_one<EPI_STORE_F32, true, true>(a, grid_m, s)
                          : hipErrorInvalidValue;
      return launch_mm_one<EPI_STORE_F32, false>(a, grid_m, s);
    case EPI_ADD_F32:
      if (w8) return a.A8 ? launch_mm_one<EPI_ADD_F32, true, true>(a, grid_m, s)
                          : hipErrorInvalidValue;
      return launch_mm_one<EPI_ADD_F32, false>(a, grid_m, s);
    case EPI_SWIGLU:
      if (a.A8) return w8 ? launch_mm_one<EPI_SWIGLU, true, true>(a, grid_m, s)
                          : hipErrorInvalidValue;
      return w8 ? launch_mm_one<EPI_SWIGLU, true>(a, grid_m, s)
                : launch_mm_one<EPI_SWIGLU, false>(a, grid_m, s);
    case EPI_DOWN:
      if (a.A8) return w8 ? launch_mm_one<EPI_DOWN, true, true>(a, grid_m, s)
                          : hipErrorInvalidValue;
      return w8 ? launch_mm_one<EPI_DOWN, true>(a, grid_m, s)
                : launch_mm_one<EPI_DOWN, false>(a, grid_m, s);
    case EPI_LMSTATS:
      // the E4M3 head takes E4M3 token rows (W8A8) only
      if (w8) return a.A8 ? launch_mm_one<EPI_LMSTATS, true, true>(a, grid_m, s)
                          : hipErrorInvalidValue;
      return launch_mm_one<EPI_LMSTATS, false>(a, grid_m, s);
    case EPI_LMSAMPLE:
      if (w8) return a.A8 && a.smp.tau ? launch_mm_one<EPI_LMSAMPLE, true, true>(a, grid_m, s)
                                       : hipErrorInvalidValue;
      if (!a.smp.tau) return hipErrorInvalidValue;
      return launch_mm_one<EPI_LMSAMPLE, false>(a, grid_m, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
