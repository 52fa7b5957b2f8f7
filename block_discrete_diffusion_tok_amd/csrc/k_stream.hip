// Weight-streaming MFMA GEMM for few token rows per weight matrix:
//   C[t][n] = sum_k X[t][k] W[n][k]
// for the tokens t of a group (the rows routed to one expert, or the
// uncommitted rows of the LM head) and every weight row n of that group's
// matrix.  At batch 1 these products move far more weight bytes than they
// compute (a weight element is used by ~16 tokens in the experts, by <= 128
// in the LM head), so the kernel is organised around HBM streaming:
//
//   * each wave owns RT x 16 weight rows and reads them straight from HBM
//     into D+1 register sets, D chunks ahead of the MFMAs (weights are used
//     once, so they never pass through LDS); a chunk's successor D chunks
//     ahead is issued before its MFMAs start.  The weights are in the packed
//     (MFMA-tiled) layout, so every wave load instruction reads one
//     contiguous kilobyte of full cache lines: with a row-major layout each
//     instruction would touch 16 lines and use half of each, and the L1's
//     outstanding-miss capacity, not HBM, would bound the stream;
//   * the group's token rows (an expert's fixed-capacity slots, whose token
//     ids the top-k kernel wrote, or the rows of a dense operand) go
//     HBM/L2 -> LDS directly (LDS-DMA loads, no registers) into a ring of
//     D+1 chunk stages shared by the workgroup's waves (4 waves per
//     workgroup).  Each chunk's token DMA and weight loads are
//     issued together D chunks ahead, so the wait for a
//     chunk covers exactly the loads issued D chunks earlier (the load
//     counter completes in issue order: a token load issued after younger
//     weight loads would force those to land first);
//   * MFMA 16x16x32 bf16 with the weights as the A operand, so a lane's
//     accumulators hold one token column and 4 consecutive weight rows: the
//     epilogues (SwiGLU of paired gate/up rows, gate-weight scaling with the
//     scatter back to (token, rank) slots, vocabulary statistics) work on
//     contiguous outputs.
//
// K-slot map: in a K chunk starting at k0, MFMA sub-step j takes from lane
// group lg (lanes 16*lg..16*lg+15) the 8 values k0 + 32*j + 8*lg + [0, 8)
// for bf16 weights, and k0 + 64*(j/2) + 16*lg + 8*(j%2) + [0, 8) for e4m3
// weights (both operands alike; the dot product is the same sum in another
// order).  This is the order of the packed layout's blocks: a lane's q-th
// 16-byte weight load of chunk kc is block kc * KC/(32 or 64) + q.
#include <math.h>

#include <type_traits>

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

// Weight loads of one K chunk into register set w.  Every address is a
// valid one: rows outside the matrix read a clamped row whose results are
// never stored, so the loads stay plain global loads with no null test (a
// select between a global and a private "zero" would turn them into flat
// loads, which the waitcnt pass can only wait for all at once).
// In the packed layout the q-th load of chunk kc is block kc * WREGS + q of
// the row tile: one contiguous kilobyte per wave load, and the 4 tiles of a
// tile group (2 waves) read one contiguous run per block column.
// The loads are non-temporal: each weight byte is read once, and leaving it
// out of the caches keeps them for the token rows that every pass re-reads.
// Measured at 256 tokens of the 128-expert layer: gate/up 144.5 -> 125.4 us,
// down 77.5 -> 69.5 us (the LM head streams faster with them too).
template <int RT, int WREGS, int ESZ, int KC>
__device__ __forceinline__ void load_w(u32x4_t (&w)[RT][WREGS],
                                       const char* const (&src)[RT], int kc) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int q = 0; q < WREGS; ++q) {
      const u32x4_t* p = (const u32x4_t*)(src[rt] + ((long long)kc * WREGS + q) * kPackKStride);
      w[rt][q] = __builtin_nontemporal_load(p);
    }
}

// LDS-DMA of 16 bytes per lane: lane l's bytes land at lds_wave_base +
// 16*l (the base is uniform over the wave).
#ifndef DG_LDS_PTR
#define DG_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
#endif
// A pointer to memory no thread writes during the kernel, in the constant
// address space: uniform loads through it are scalar loads.
#ifndef DG_CONST_PTR
#define DG_CONST_PTR(T, p) ((const __attribute__((address_space(4))) T*)(p))
#endif

__device__ __forceinline__ void dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, DG_LDS_PTR(lds_wave_base), 16, 0, 0);
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (other counters untouched).
constexpr int vm_wait(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8);
}

__device__ __forceinline__ f32x4_t mfma_v(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// One K chunk of MFMAs.  Stage layout: token row r's 16-byte unit c
// (k values 8c..8c+7 of the chunk) sits at unit r*(KC/8) + (c ^ (r & 7)),
// so the 8 rows a ds_read_b128 phase touches fall in distinct banks.
template <int RT, int NT, int KC, int WREGS, bool W8>
__device__ __forceinline__ void mfma_chunk(f32x4_t (&acc)[RT][NT],
                                           const u32x4_t (&w)[RT][WREGS],
                                           const uint16_t* stage,
                                           int l16, int lg) {
#pragma unroll
  for (int j = 0; j < KC / 32; ++j) {
    u32x4_t af[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if (W8) {
        u32x4_t lo, hi;
        widen_e4m3x16(w[rt][j >> 1], lo, hi);
        af[rt] = (j & 1) ? hi : lo;
      } else {
        af[rt] = w[rt][j];
      }
    }
    const int koff = W8 ? 64 * (j >> 1) + 16 * lg + 8 * (j & 1) : 32 * j + 8 * lg;
    const int unit = (koff >> 3) ^ (l16 & 7);
    // Every token tile is computed: tiles past the last token hold clamped
    // (valid) rows whose results the epilogues drop, and a uniform branch
    // here would serialise the LDS reads behind one wait each.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const u32x4_t bx = *(const u32x4_t*)&stage[((nt * 16 + l16) * (KC / 8) + unit) * 8];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][nt] = mfma_v(af[rt], bx, acc[rt][nt]);
    }
  }
}

// The kernel body for NT token tiles per pass.  Xs: the LDS token stages
// (at least (D+1) * NT*16 * KC elements).  dense_rows: the row count of a
// dense operand (already read), unused for groups.
template <int RT, int NT, int KC, int D, int EPI, bool W8, int WV>
__device__ __forceinline__ void stream_run(const StreamArgs& a, uint16_t* Xs, int dense_rows) {
  static_assert(RT % 2 == 0, "gate/up pairing needs an even number of row tiles");
  static_assert(epi_is_lm(EPI) || EPI == EPI_SWIGLU || EPI == EPI_DOWN, "epilogue");
  // the gate/up products read a slot's token row through row_of; the down
  // products read the slot rows of the SwiGLU output directly
  constexpr bool MAPPED = EPI == EPI_SWIGLU;
  // the expert products run over groups (experts) of slots; the LM head
  // over the rows of one dense operand
  constexpr bool GROUPED = !epi_is_lm(EPI);
  static_assert(KC == 64 || KC == 128, "K chunk");
  constexpr int WROWS = WV * RT * 16;  // weight rows per workgroup (WV waves)
  constexpr int ESZ = W8 ? 1 : 2;     // bytes per weight element
  // 16-byte weight loads per row tile per chunk (KC/4 k values per lane)
  constexpr int WREGS = (KC / 4) * ESZ / 16;
  static_assert(D >= 2, "chunks in flight");
  constexpr int S = D + 1;                     // token stages
  constexpr int STAGE = NT * 16 * KC;          // elements per stage
  constexpr int UNITS = STAGE / 8;             // 16-byte units per stage
  static_assert(UNITS % (64 * WV) == 0, "token units per thread");
  constexpr int IPW = UNITS / (64 * WV);       // token DMAs per wave per chunk
  constexpr int LOADS = IPW + RT * WREGS;      // loads per wave per chunk
  static_assert((D - 1) * LOADS <= 63, "vmcnt range");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  // Expert products: workgroups are dealt to the 8 XCDs round-robin by
  // linear id, so the natural order spreads every expert's row tiles over
  // all of them and each XCD's L2 fetches every expert's token rows.  With
  // the expert count a multiple of 8, XCD x instead runs experts x, x + 8,
  // ... (its j-th workgroup takes tile j % tiles of expert x + 8 (j / tiles)),
  // and an expert's token rows come from HBM once.
  int group = blockIdx.y, bx = blockIdx.x;
  if (GROUPED && (gridDim.y & 7) == 0) {
    const int lin = blockIdx.x + gridDim.x * blockIdx.y;
    const int j = lin >> 3;
    group = (lin & 7) + 8 * (j / gridDim.x);
    bx = j % gridDim.x;
  }

  // ---- this wave's weight row tiles (16 rows each) and the packed address
  // of this lane's piece of their first block; tiles past the matrix read
  // tile 0 (valid addresses, results never stored)
  const int n_base = bx * WROWS;
  const char* wgroup = (const char*)a.W + (long long)group * a.w_group_stride * ESZ;
  const char* wsrc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int r0;
    bool ok;
    if (EPI == EPI_SWIGLU) {
      // tiles [0, RT/2) are gate rows of channels c0 + 16*rt + [0, 16),
      // tiles [RT/2, RT) the up rows of the same channels
      const int c0 = bx * (WROWS / 2) + wave * (8 * RT) + (rt % (RT / 2)) * 16;
      ok = c0 < a.ffn;
      r0 = (rt < RT / 2) ? c0 : a.ffn + c0;
    } else {
      r0 = n_base + (wave * RT + rt) * 16;
      ok = r0 < a.N;
    }
    wsrc[rt] = wgroup + pack_block_offset(ok ? r0 >> 4 : 0, 0, a.K, ESZ) + 16 * lane;
  }
  const int nk = a.K / KC;
  // chunk k uses weight register set k % NSET and token stage k % S
  constexpr int NSET = D + 1;  // register sets: chunk k+D loads while chunk k computes

  // ---- token rows: slots [group*cap, group*cap + count) of a group (the
  // X row of a slot is row_of[slot] when given, else the slot itself), or
  // rows [0, M) (M_dev when given) in dense mode.  A group's count is a
  // uniform scalar load, counted apart from the vector loads, read after the
  // first D chunks are issued: a group's passes read slots below cap (slots
  // past the count hold stale but valid rows and ids whose results are
  // dropped), so the down products issue their first chunks at once and the
  // gate/up products wait only for the slots' token ids.  The dense operand
  // repeats its last live row (one line per pass for few rows).
  constexpr int TROWS = NT * 16;
  const long long row0 = GROUPED ? (long long)group * a.cap : 0;
  int t_end = 0;  // loaded once the first weight loads are out

  // EPI_DOWN: the pair index and gate weight of this lane's token columns,
  // loaded before the pass's first chunk (older than every chunk load, so no
  // chunk wait changes) and used by the epilogue
  int pair_of[NT];
  float wgt_of[NT];
  auto load_ids = [&](int t0) {
    if (EPI == EPI_DOWN) {
      static_for<NT>([&](auto nt) {
        const long long slot = row0 + min(t0 + nt * 16 + l16, a.cap - 1);
        pair_of[nt] = a.c_map[slot];
        wgt_of[nt] = a.row_scale[slot];
      });
    }
  };
  // token unit u = 64*(wave*IPW + i) + lane of a stage holds row
  // u / (KC/8), logical unit (u % (KC/8)) ^ (row & 7)
  auto unit_row = [&](int i) { return (64 * (wave * IPW + i) + lane) / (KC / 8); };
  int tok_id[IPW];
  auto load_tok_ids = [&](int t0) {
    if (MAPPED)
      static_for<IPW>([&](auto i) {
        tok_id[i] = a.row_of[row0 + min(t0 + unit_row(i), a.cap - 1)];
      });
  };
  const uint16_t* xsrc[IPW];
  auto set_rows = [&](int t0) {
    // (rows past a group's count repeat its last row once the count is
    // known: the same lines again, from L2, instead of stale slot rows)
    const int lim = GROUPED ? (t_end > 0 ? t_end : a.cap) : max(t_end, 1);
    static_for<IPW>([&](auto i) {
      const int u = 64 * (wave * IPW + i) + lane;
      const int row = u / (KC / 8);
      const int c = (u % (KC / 8)) ^ (row & 7);
      const long long trow = MAPPED ? (long long)min((unsigned)tok_id[i], (unsigned)(a.M - 1))
                                    : row0 + min(t0 + row, lim - 1);
      xsrc[i] = a.X + trow * a.ldx + c * 8;
    });
  };

  u32x4_t w[NSET][RT][WREGS];
  // Loads of chunk k < nk: its token DMA into stage k % S, its weights into
  // register set p = k % NSET (the chunk waits rely only on each chunk's
  // loads being contiguous in issue order, chunks in order).
  auto issue = [&](auto p, int k) {
    uint16_t* st = &Xs[(k % S) * STAGE + wave * IPW * 64 * 8];
    static_for<IPW>([&](auto i) { dma16(xsrc[i] + (long long)k * KC, st + i * 64 * 8); });
    load_w<RT, WREGS, ESZ, KC>(w[p], wsrc, k);
  };
  auto prologue = [&]() {
    static_for<D>([&](auto p) {
      issue(p, (int)p);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // the count is read-only here (an earlier kernel wrote it): a scalar load
  // through the constant address space, so its wait is not a vector-memory
  // wait for every chunk in flight.  With few tokens (one decoded position:
  // 8 of 128 experts hold a row) most groups are empty, and their first
  // chunks would be loaded for nothing: the count is then read first.
  if (GROUPED && a.count_first) {
    t_end = min(*DG_CONST_PTR(int32_t, a.group_count + group), a.cap);
    if (t_end <= 0) return;  // the whole workgroup: no load was issued
  }
  load_ids(0);
  load_tok_ids(0);
  if (!GROUPED) t_end = dense_rows;
  set_rows(0);
  prologue();
  if (GROUPED && !a.count_first)
    t_end = min(*DG_CONST_PTR(int32_t, a.group_count + group), a.cap);
  if (t_end <= 0) {  // an empty group: let the loads land before leaving
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
    return;
  }
  if (GROUPED && !MAPPED) set_rows(0);  // chunks from D on: count-bounded rows

  for (int t0 = 0; t0 < t_end; t0 += TROWS) {
    const int nt_rows = min(TROWS, t_end - t0);
    const int nt_act = (nt_rows + 15) >> 4;
    if (t0 > 0) {
      load_ids(t0);
      load_tok_ids(t0);
      set_rows(t0);
      __syncthreads();  // the previous pass is done with Xs
      prologue();
    }
    f32x4_t acc[RT][NT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Chunk k, with `younger` chunks issued after it: wait for its loads
    // (the vector-memory counter completes in issue order), barrier (every
    // wave's token DMA has landed; every wave is past chunk k-1, whose
    // stage the chunk k+D DMA reuses), issue chunk k+D if it exists (into
    // the register set no chunk in flight uses), then the MFMAs of chunk
    // k, so D chunks stay in flight while they run.  The barrier is the
    // bare instruction: a workgroup fence here would wait for every DMA in
    // flight.
    auto step = [&](auto p, int k, int younger, bool more) {
      static_for<D>([&](auto y) {
        if (younger == y) __builtin_amdgcn_s_waitcnt(vm_wait(decltype(y)::value * LOADS));
      });
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (more) issue(std::integral_constant<int, (decltype(p)::value + D) % NSET>(), k + D);
      __builtin_amdgcn_sched_barrier(0);
      mfma_chunk<RT, NT, KC, WREGS, W8>(acc, w[p], &Xs[(k % S) * STAGE], l16, lg);
      __builtin_amdgcn_sched_barrier(0);
    };

    // Groups of NSET chunks as straight-line code (register set k % NSET
    // is static) while every chunk of the group issues chunk k+D < nk; the
    // state at each group boundary is the same (at most chunks kc..kc+D-1
    // in flight), so the fixed waits stay exact.  Then the last chunks: those
    // with k+D < nk still issue, the last D drain with waits for exactly
    // the chunks still in flight (nk >= D is a launch precondition).
    int kc = 0;
    while (kc + NSET + D <= nk) {
      static_for<NSET>([&](auto p) { step(p, kc + p, D - 1, true); });
      kc += NSET;
    }
    static_for<NSET + D>([&](auto j) {
      const int k = kc + j;
      if (k < nk)
        step(std::integral_constant<int, j % NSET>(), k, min(D - 1, nk - 1 - k),
             k + D < nk);
    });
    __syncthreads();  // every wave is done with the stages before LDS is reused

    // ---- epilogues: lane holds token column t0 + 16*nt + l16 and weight
    // rows 4*lg + e of each row tile
    if (epi_is_lm(EPI)) {
      float4* red = (float4*)&Xs[0];  // [WV waves][NT*16]
      float2* red2 = (float2*)&red[WV * NT * 16];  // sampling: [WV waves][NT*16]
      static_assert(WV * NT * 16 * 24 <= S * STAGE * 2, "LDS reuse");
      constexpr bool smp = EPI == EPI_LMSAMPLE;
      // E4M3 head (token rows given as their codes' bf16 values): each logit
      // is scaled by its vocabulary row's scale and its token row's scale
      // first (every statistic below is of the scaled z)
      if (W8) {
        float wsc[RT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            wsc[rt][e] = a.w_scale[min(n_base + (wave * RT + rt) * 16 + 4 * lg + e, a.N - 1)];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float xs = a.x_scale[min(t0 + nt * 16 + l16, t_end - 1)];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[rt][nt][e] *= wsc[rt][e] * xs;
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // temperature sampling: statistics of z / tau, Gumbel-max token
        const int srow = min(t0 + nt * 16 + l16, t_end - 1);
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
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = n_base + (wave * RT + rt) * 16 + 4 * lg + e;
            const float v = smp ? acc[rt][nt][e] * scale : acc[rt][nt][e];
            if (n < a.N && v > m) { m = v; am = n; }
          }
        if (m != -INFINITY) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int n = n_base + (wave * RT + rt) * 16 + 4 * lg + e;
              if (n < a.N) {
                const float v = smp ? acc[rt][nt][e] * scale : acc[rt][nt][e];
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
          smerge(m, s, t, am, m2, s2, t2, am2);
        }
        if (lg == 0) red[wave * NT * 16 + nt * 16 + l16] = make_float4(m, s, t, __int_as_float(am));
        if (smp) {
          float g = -INFINITY;
          int gi = 0x7fffffff;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const int n0 = n_base + (wave * RT + rt) * 16 + 4 * lg;
            uint32_t c[4] = {(uint32_t)n0 >> 2, c1, c2, c3};
            if (tau > 0.f) philox4x32_10(c, a.smp.key0, a.smp.key1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (n0 + e >= a.N) continue;
              const float v = acc[rt][nt][e] * scale;
              best_merge(g, gi, tau > 0.f ? v + gumbel_of(c[e]) : v, n0 + e);
            }
          }
#pragma unroll
          for (int off = 16; off < 64; off <<= 1)
            best_merge(g, gi, shfl_xor(g, off), shfl_xor(gi, off));
          if (lg == 0) red2[wave * NT * 16 + nt * 16 + l16] = make_float2(g, __int_as_float(gi));
        }
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
        for (int w = 1; w < WV; ++w) {
          const float4 q = red[w * NT * 16 + tid];
          smerge(m, s, t, am, q.x, q.y, q.z, __float_as_int(q.w));
        }
        a.part[(long long)(t0 + tid) * a.n_tiles + bx] =
            make_float4(m, s, t, __int_as_float(am));
        if (smp) {
          float2 b = red2[tid];
          float g = b.x;
          int gi = __float_as_int(b.y);
#pragma unroll
          for (int w = 1; w < WV; ++w) {
            const float2 q = red2[w * NT * 16 + tid];
            best_merge(g, gi, q.x, __float_as_int(q.y));
          }
          a.smp.spart[(long long)(t0 + tid) * a.n_tiles + bx] = make_float2(g, __int_as_float(gi));
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int tok = t0 + nt * 16 + l16;
        if (nt >= nt_act || tok >= t_end) continue;
        // E4M3 token rows (given as their bf16 values): the row's scale
        float xs = 1.f;
        if (a.x_scale) xs = a.x_scale[MAPPED ? a.row_of[row0 + tok] : row0 + tok];
        if (EPI == EPI_SWIGLU) {
          const int c0 = bx * (WROWS / 2) + wave * (8 * RT);
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
              g[e] *= xs;
              u[e] *= xs;
            }
            *(uint2*)((uint16_t*)a.C + (row0 + tok) * a.ldc + ch) =
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
              int pair = 0;
              float wgt = 0.f;
              static_for<NT>([&](auto q) {
                if (q == nt) {
                  pair = pair_of[q];
                  wgt = wgt_of[q];
                }
              });
              float sc4[4] = {1.f, 1.f, 1.f, 1.f};
              if (W8) {
                const float* sc = a.w_scale + (long long)group * a.scale_rows + n;
                sc4[0] = sc[0]; sc4[1] = sc[1]; sc4[2] = sc[2]; sc4[3] = sc[3];
              }
              wgt *= xs;
              *(float4*)((float*)a.C + (long long)pair * a.ldc + n) =
                  make_float4(v[0] * wgt * sc4[0], v[1] * wgt * sc4[1],
                              v[2] * wgt * sc4[2], v[3] * wgt * sc4[3]);
            }
          }
        }
      }
    }
  }
}

// The LM head runs its rows in passes of 2, 4, 6 or 8 token tiles, whichever
// is the fewest that cover the live rows in one pass (the token DMA and the
// MFMAs scale with the tiles, the weight stream does not; 3, 5 and 7 tiles
// would not split into whole DMA instructions over 4 waves).
template <int RT, int NT, int KC, int D, int EPI, bool W8, int OCC, int WV>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void stream_kernel(StreamArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Xs[(D + 1) * NT * 16 * KC];
  if constexpr (epi_is_lm(EPI) && NT == 8) {
    int rows = a.M;
    if (a.M_dev) rows = min(rows, a.M_dev[0]);
    if (a.M_dev && a.rows_le > 0 && rows > a.rows_le) return;  // another kernel's rows
    if (rows <= 32)
      stream_run<RT, 2, KC, D, EPI, W8, WV>(a, Xs, rows);
    else if (rows <= 64)
      stream_run<RT, 4, KC, D, EPI, W8, WV>(a, Xs, rows);
    else if (rows <= 96)
      stream_run<RT, 6, KC, D, EPI, W8, WV>(a, Xs, rows);
    else
      stream_run<RT, 8, KC, D, EPI, W8, WV>(a, Xs, rows);
  } else if constexpr (epi_is_lm(EPI)) {
    int rows = a.M;
    if (a.M_dev) rows = min(rows, a.M_dev[0]);
    stream_run<RT, NT, KC, D, EPI, W8, WV>(a, Xs, rows);
  } else {
    stream_run<RT, NT, KC, D, EPI, W8, WV>(a, Xs, 0);
  }
}

template <int RT, int NT, int KC, int D, int EPI, bool W8, int OCC, int WV>
hipError_t launch_s(const StreamArgs& a, int groups, hipStream_t s) {
  constexpr int WROWS = WV * RT * 16;
  if ((EPI == EPI_SWIGLU || EPI == EPI_DOWN) != (a.group_count != nullptr) ||
      (EPI == EPI_SWIGLU) != (a.row_of != nullptr))
    return hipErrorInvalidValue;
  // every load reads rows below a bound known here (cap slots of a group,
  // M rows of a dense or mapped operand), so those bounds must hold rows
  if (a.group_count && a.cap <= 0) return hipErrorInvalidValue;
  if ((!a.group_count || EPI == EPI_SWIGLU) && a.M <= 0)
    return a.group_count ? hipErrorInvalidValue : hipSuccess;
  int grid_x;
  if (EPI == EPI_SWIGLU) grid_x = (a.ffn + WROWS / 2 - 1) / (WROWS / 2);
  else grid_x = (a.N + WROWS - 1) / WROWS;
  if (grid_x <= 0 || groups <= 0) return hipSuccess;
  hipLaunchKernelGGL((stream_kernel<RT, NT, KC, D, EPI, W8, OCC, WV>), dim3(grid_x, groups),
                     dim3(64 * WV), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// LM head: 2 row tiles per wave (128 vocabulary rows per workgroup), up to
// 128 token columns per pass, K chunks of 64, 3 chunks in flight (4 stages
// of 16 KB, 4 weight register sets), 2 workgroups per CU.  Experts: 2 row
// tiles per wave, K chunks of 64, 4-wave workgroups, two per CU, so that one
// fills its pipeline while the other streams; gate/up with passes of 64
// token columns and 3 chunks in flight, down with passes of 64 and 2 chunks
// in flight (it has only K / 64 = 12 chunks per row block).  Side by side in
// the 30-layer step at batch 1 (an expert has ~16 tokens), with plain weight
// loads, gate/up: one 8-wave workgroup with 128-column passes and 2 chunks in
// flight 147 us, two 4-wave workgroups with 64-column passes 142 us, with 3
// chunks in flight 140 us, with 32-column passes 151 us, 8 waves with 4
// chunks in flight 154 us.  Down: 89.0 -> 87.1 us against one 8-wave
// workgroup; 3 or 4 chunks in flight or 32-column passes within noise.  With
// non-temporal weight loads (gate/up 125 us, down 70-72 us), 4 chunks in
// flight for gate/up and 3 for down measured within noise.
constexpr int kLmRT = 2, kLmKC = 64, kLmD = 3, kLmOcc = 2, kLmWaves = 4;
constexpr int kMoeRT = 2, kMoeKC = 64, kMoeOcc = 2;
constexpr int kGuNT = 4, kGuD = 3, kGuWaves = 4;  // gate/up
constexpr int kDnNT = 4, kDnD = 2, kDnWaves = 4;  // down

int stream_rows_per_wg() { return kLmWaves * kLmRT * 16; }
bool stream_lm_ok(int hidden) {
  return hidden % kLmKC == 0 && hidden / kLmKC >= kLmD;
}
bool stream_moe_ok(int hidden, int ffn) {
  return hidden % kMoeKC == 0 && ffn % kMoeKC == 0 && hidden / kMoeKC >= kGuD &&
         ffn / kMoeKC >= kDnD;
}

hipError_t launch_stream(int epi, bool w8, const StreamArgs& a, int groups,
                         hipStream_t s) {
  switch (epi) {
    case EPI_LMSTATS:
      if (!stream_lm_ok(a.K)) return hipErrorInvalidValue;
      // the E4M3 head: E4M3 weights with per-row scales, token rows with
      // their row scales
      if (w8)
        return a.w_scale && a.x_scale
                   ? launch_s<kLmRT, 8, kLmKC, kLmD, EPI_LMSTATS, true, kLmOcc, kLmWaves>(a, groups, s)
                   : hipErrorInvalidValue;
      return launch_s<kLmRT, 8, kLmKC, kLmD, EPI_LMSTATS, false, kLmOcc, kLmWaves>(a, groups, s);
    case EPI_LMSAMPLE:
      if (!stream_lm_ok(a.K) || !a.smp.tau) return hipErrorInvalidValue;
      if (w8)
        return a.w_scale && a.x_scale
                   ? launch_s<kLmRT, 8, kLmKC, kLmD, EPI_LMSAMPLE, true, kLmOcc, kLmWaves>(a, groups, s)
                   : hipErrorInvalidValue;
      return launch_s<kLmRT, 8, kLmKC, kLmD, EPI_LMSAMPLE, false, kLmOcc, kLmWaves>(a, groups, s);
    case EPI_SWIGLU:
      if (a.K % kMoeKC || a.K / kMoeKC < kGuD) return hipErrorInvalidValue;
      return w8 ? launch_s<kMoeRT, kGuNT, kMoeKC, kGuD, EPI_SWIGLU, true, kMoeOcc, kGuWaves>(a, groups, s)
                : launch_s<kMoeRT, kGuNT, kMoeKC, kGuD, EPI_SWIGLU, false, kMoeOcc, kGuWaves>(a, groups, s);
    case EPI_DOWN:
      if (a.K % kMoeKC || a.K / kMoeKC < kDnD) return hipErrorInvalidValue;
      return w8 ? launch_s<kMoeRT, kDnNT, kMoeKC, kDnD, EPI_DOWN, true, kMoeOcc, kDnWaves>(a, groups, s)
                : launch_s<kMoeRT, kDnNT, kMoeKC, kDnD, EPI_DOWN, false, kMoeOcc, kDnWaves>(a, groups, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dg
