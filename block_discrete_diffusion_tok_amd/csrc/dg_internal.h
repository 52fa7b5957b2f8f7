// Internal declarations shared by the libdg kernels and the host runtime.
// gfx950 (CDNA4) only: wave64, bf16 MFMA 16x16x32, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "dg.h"

namespace dg {

// ------------------------------------------------------------------ types
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Native 128-bit vector: copies of it are plain register moves (a uint4
// struct copy goes through memcpy, which can pin it in private memory).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// fp32 -> bf16 bits, round to nearest even, by gfx950's packed conversion
// instruction: one instruction rounds two values, bit for bit the same as
// adding 0x7fff plus the kept lsb and truncating, for every input that is not
// a NaN (a NaN stays a NaN; its payload is the hardware's).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// 16 OCP E4M3 bytes -> 16 bf16 (exact: 3 mantissa bits and exponents
// 2^-9..2^8 all fit in bfloat16), by gfx950's packed conversion with unit
// scale: each instruction widens the two bytes of one half-word, byte 0 of
// the pair into the low half of the result.  lo takes bytes 0..7, hi 8..15.
__device__ __forceinline__ void widen_e4m3x16(const u32x4_t q, u32x4_t& lo, u32x4_t& hi) {
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, false));
    o[2 * i + 1] = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[i], 1.0f, true));
  }
  lo = u32x4_t{o[0], o[1], o[2], o[3]};
  hi = u32x4_t{o[4], o[5], o[6], o[7]};
}

// One bf16 MFMA: D(16x16) += A(16x32) * B(32x16).  Lane l supplies row
// (A) / column (B) l % 16 and the 8 k-slots 8*(l/16)..+7; the result holds
// column l % 16, rows 4*(l/16)+i in element i.  Any assignment of real k
// indices to k-slots works as long as A and B use the same one.
__device__ __forceinline__ f32x4_t mfma16x16x32(const uint4& a, const uint4& b,
                                                f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0,
      0, 0);
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
// Register arrays indexed through it get constant indices in the IR, so they
// are split into registers before any pass could place them in memory.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f,
                                                std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) {
  return __shfl_xor(v, m, kWave);
}

// ------------------------------------------------------------------ packed weights
// Every weight matrix the kernels read ([R, K] row-major per group: Q/K/V,
// output, router, gate/up, down, the tied embedding) is stored in an
// MFMA-tiled layout: 1024-byte blocks of 16 rows x kPackK values, kPackK =
// 64 / element bytes (32 bf16 or 64 e4m3 values).  Inside a block, the 16
// bytes at 16 * l (l = r + 16 q, r < 16, q < 4) hold row 16 rb + r, values
// kb * kPackK + q * kPackK/4 .. +kPackK/4 - 1: exactly what lane l feeds to
// a 16x16x32 MFMA as the A operand, so one wave load instruction reads one
// contiguous kilobyte.  Row tiles are grouped by kPackTiles (64 rows); in a
// group the blocks are ordered by kb, then tile: block (rb, kb) sits at
// ((rb / 4) * 4 * KB + kb * 4 + rb % 4) * 1024 with KB = K / kPackK.  A
// kernel streaming the row tiles of a group in K order then reads one
// contiguous run of 4 KB per block column instead of 4 separate streams
// (fewer, longer DRAM runs: ~6.1 instead of ~5.2 TB/s in a read-only probe
// of this access pattern).  Rows are zero-padded to a multiple of 64; with
// several groups (experts) the row count per group must already be one.
constexpr int kPackBlock = 1024;
constexpr int kPackTiles = 4;
constexpr int kPackRows = 16 * kPackTiles;
constexpr long long kPackKStride = (long long)kPackTiles * kPackBlock;  // kb -> kb+1
__host__ __device__ constexpr int pack_k(int esz) { return 64 / esz; }
// byte offset of block (rb, kb) in a matrix with K columns
__host__ __device__ inline long long pack_block_offset(int rb, int kb, int K, int esz) {
  const int KB = K / pack_k(esz);
  return (((long long)(rb / kPackTiles) * KB + kb) * kPackTiles + rb % kPackTiles) *
         kPackBlock;
}
hipError_t launch_pack(const void* src, int groups, int rows, int cols, int esz,
                       void* dst, hipStream_t s);

// ------------------------------------------------------------------ sampling
// Temperature sampling in the LM head's epilogue (rows are the LM head's
// token rows): the statistics are taken of z / tau (tau > 0) and the
// sampled token is argmax_v (z_v / tau + g_v), g_v = -ln(-ln u_v) with u_v
// from Philox4x32-10 (counter (v / 4, ctr[row]), key (key0, key1), output
// v % 4, top 24 bits + 1/2 times 2^-24).  tau <= 0: statistics of the raw
// logits and the argmax as the sample (the merge reports entropy 0).
struct LmSample {
  const float* tau;      // [rows] temperature of each row; nullptr: no sampling
  const int32_t* ctr;    // [rows][3] counter words 1..3 (position, step, canvas)
  uint32_t key0, key1;
  float2* spart;         // [rows][n_tiles] (best score, its vocabulary id as bits)
};

// Philox4x32-10 (Salmon et al., SC 2011): 10 rounds of two 32x32->64-bit
// products, the key advanced by the Weyl increments between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = c[0] * 0xD2511F53u, hi0 = __umulhi(c[0], 0xD2511F53u);
    const uint32_t lo1 = c[2] * 0xCD9E8D57u, hi1 = __umulhi(c[2], 0xCD9E8D57u);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}
// -ln(-ln u) of a Philox output word, u = (k + 1/2) 2^-24 with k = x >> 8.
// u = (2k + 1) 2^-25 is exact in fp32 only below 1/2; above it 1 - u =
// (2^25 - 2k - 1) 2^-25 is, and -ln u = -log1p(-(1 - u)) keeps full
// relative accuracy there, where the largest draws (u near 1) come from.
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  const uint32_t k = x >> 8;
  const float l = k < (1u << 23)
                      ? -logf((float)(2 * k + 1) * 2.98023223876953125e-8f)
                      : -log1pf(-(float)((1u << 25) - 2 * k - 1) * 2.98023223876953125e-8f);
  return -logf(l);
}
// Keep the better (score, id): larger score, lower id on ties.
__device__ __forceinline__ void best_merge(float& g, int& gi, float g2, int gi2) {
  if (g2 > g || (g2 == g && gi2 < gi)) {
    g = g2;
    gi = gi2;
  }
}

// ------------------------------------------------------------------ launches
// Every launcher returns hipSuccess or the launch error; shapes were checked
// by the caller.

enum GemmEpi : int {
  EPI_STORE_BF16 = 0,  // C bf16 [M, N]
  EPI_STORE_F32 = 1,   // C fp32 [M, N]
  EPI_ADD_F32 = 2,     // C fp32 [M, N] += acc
  EPI_SWIGLU = 3,      // act bf16 [rows, F] = silu(gate) * up
  EPI_DOWN = 4,        // y fp32 [pair, N] = w_pair * acc (scattered rows)
  EPI_LMSTATS = 5,     // per-row (max, sum exp, sum exp*(z-max), argmax)
  EPI_LMSAMPLE = 6     // EPI_LMSTATS at the rows' temperatures + sampled tokens
};
constexpr bool epi_is_lm(int epi) { return epi == EPI_LMSTATS || epi == EPI_LMSAMPLE; }

struct GemmArgs {
  const uint16_t* A;       // bf16 [rows, K]
  int lda;
  const int32_t* a_map;    // optional: A row = a_map[row] / a_map_div
  int a_map_div;
  const void* B;           // weights [N, K] (bf16 or e4m3), per group stride
  long long b_group_stride;  // elements between groups
  const float* b_scale;    // e4m3 per-row scales, [groups][scale_rows]
  int scale_rows;
  int M;                   // rows (dense)
  const int32_t* M_dev;    // optional device row count (dense)
  int N, K;
  int n_groups;                  // grouped mode when group_offsets != null
  const int32_t* group_offsets;  // [G+1] row offsets
  const int32_t* tile_offsets;   // [G+1] m-tile offsets
  void* C;                 // output
  int ldc;
  const int32_t* c_map;    // EPI_DOWN: pair index of each row
  const float* row_scale;  // EPI_DOWN: gate weight per pair
  int ffn;                 // EPI_SWIGLU: F
  float4* part;            // EPI_LMSTATS: [rows][n_tiles]
  int n_tiles;
  float* logits;           // EPI_LMSTATS: optional [rows, N] (row_map placed)
  const int32_t* row_map;  // EPI_LMSTATS: logits row of each A row
  int splits;              // EPI_STORE_F32: K splits (gridDim.z), 0/1 = none;
  long long split_stride;  //   split z writes its own slab C + z * split_stride
  int rows_gt;             // with M_dev: the launch does nothing unless
                           //   *M_dev > rows_gt (another kernel takes fewer rows)
  LmSample smp;            // EPI_LMSTATS: temperature sampling (smp.tau null: off)
  const uint8_t* A8;       // large-tile kernel: E4M3 token rows [rows, lda]
  const float* a_scale;    //   bytes instead of A, and the scale of each A row
                           //   (dense e4m3 products on the 64 x 64 tiles:
                           //   A holds the codes' bf16 values, a_scale the
                           //   row scales)
};

// Tile sizes of the grouped GEMMs (rows of one expert are tiled by this).
constexpr int kGroupBM = 64;

hipError_t launch_gemm(int epi, bool w_e4m3, const GemmArgs& a, int grid_m,
                       hipStream_t s);
int gemm_bn(int epi);   // BN of the instance used for an epilogue
int gemm_bm(int epi);   // BM of the instance used for an epilogue
// Whether launch_gemm runs a dense product on the large-tile kernel (its
// e4m3 form then takes E4M3 token rows, A8, on the FP8 MFMA).
bool gemm_dense_on_mm(int epi, const GemmArgs& a);

// Large-tile GEMM (k_mm.hip): 256 weight rows x 256 token rows per
// workgroup, for thousands of token rows (dense) or hundreds per group.
// Same arguments and epilogues as launch_gemm, no K splits; grid_m counts
// 256-row tiles (group tile offsets in units of mm_bm()).  EPI_LMSTATS
// writes two partials per workgroup, one per 128 vocabulary rows, so a
// row's partials are indexed like the streaming LM head's (n_tiles =
// ceil(N / 128)).
hipError_t launch_mm(int epi, bool w_e4m3, const GemmArgs& a, int grid_m, hipStream_t s);
int mm_bm();
int mm_bn();

// Weight-streaming GEMM (few token rows per weight matrix); see k_stream.hip.
struct StreamArgs {
  const uint16_t* X;       // bf16 token rows [rows, K]
  int ldx;
  const void* W;           // weights [N, K] per group (bf16 or e4m3), packed
  long long w_group_stride;  // elements between groups
  const float* w_scale;    // e4m3 per-row scales [groups][scale_rows]
  int scale_rows;
  int M;                   // token rows (dense)
  const int32_t* M_dev;    // optional device token count (dense)
  int N, K;                // K as stream_lm_ok / stream_moe_ok require
  // Grouped (expert) mode when group_count != null: group g owns the
  // fixed-capacity slots [g*cap, g*cap + group_count[g]).  EPI_SWIGLU reads
  // slot s's token from X row row_of[s] (clamped to [0, M); every slot read
  // is below g*cap + cap) and writes C row s; EPI_DOWN reads X row s and
  // c_map / row_scale at s.
  const int32_t* group_count;
  int cap;
  const int32_t* row_of;
  void* C;
  int ldc;
  const int32_t* c_map;    // EPI_DOWN: pair index of each slot row
  const float* row_scale;  // EPI_DOWN: gate weight per pair
  int ffn;                 // EPI_SWIGLU: F
  float4* part;            // EPI_LMSTATS: [rows][n_tiles]
  int n_tiles;
  float* logits;           // EPI_LMSTATS: optional [rows, N]
  const int32_t* row_map;  // EPI_LMSTATS: logits row of each token row
  int rows_le;             // EPI_LMSTATS with M_dev: the launch does nothing
                           //   unless *M_dev <= rows_le (0: no limit)
  LmSample smp;            // EPI_LMSTATS: temperature sampling (smp.tau null: off)
  const float* x_scale;    // SWIGLU / DOWN: X rows hold E4M3 values (as bf16);
                           //   the scale of each X row (null: none)
  int count_first;         // grouped: read a group's count before issuing any
                           //   load, so that empty groups load nothing (for
                           //   launches where most groups are empty)
};
// Epilogues EPI_LMSTATS (up to 128 token columns per pass), EPI_SWIGLU (64)
// and EPI_DOWN (64).  K must satisfy stream_lm_ok / stream_moe_ok.
hipError_t launch_stream(int epi, bool w_e4m3, const StreamArgs& a, int groups,
                         hipStream_t s);
bool stream_lm_ok(int hidden);
bool stream_moe_ok(int hidden, int ffn);
int stream_rows_per_wg();  // weight rows per workgroup

struct AttnArgs {
  const uint16_t* qkv;  // [n*C, ldqkv]
  int ldqkv;
  int C, Hq, Hkv, D;
  const uint16_t* kc;   // layer base of the K cache
  const uint16_t* vc;
  long long req_stride;   // elements between request slots
  long long head_stride;  // elements between KV heads (= max_kv_len * D)
  int req[DG_MAX_BATCH];
  int plen[DG_MAX_BATCH];
  int vis0[DG_MAX_BATCH];  // first canvas of the batch canvas b also sees
                           //   (b itself: none; canvases vis0..b-1 are the
                           //   earlier blocks of b's request)
  int n;
  int splits;
  int causal;
  uint16_t* out;        // [n*C, Hq*D]
  float* opart;         // [splits][n*Hq*C][D]
  float* lpart;         // [splits][n*Hq*C]
  // E4M3 cache (null: bf16): kc / vc then hold codes (one byte per value,
  // same strides) and ks / vs the fp32 scale of each cached row, at the
  // row's code offset / D
  const float* ks;
  const float* vs;
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// KV splits for n canvases; max_keys = longest prefix + C (0: the upper
// bound over all prefix lengths, used to size workspaces).
int attention_auto_splits(int n, int C, int Hq, int Hkv, int max_keys);

hipError_t launch_embed(const int32_t* tokens, int T, const uint16_t* embed,
                        int V, int H, float* x, hipStream_t s);
// row_map (optional) must hold `rows` readable entries; rows r >= *m_dev
// (when given) are skipped.  zero (optional): n_zero ints the first
// workgroup clears (the expert counters of the following top-k).
hipError_t launch_rmsnorm(const float* x, int rows, int H, const float* g,
                          float eps, uint16_t* out, const int32_t* row_map,
                          const int32_t* m_dev, float* copy_f32,
                          hipStream_t s, int32_t* zero = nullptr, int n_zero = 0);
// logits: `splits` fp32 slabs [T, E] (partial sums over K) added in slab
// order; with splits > 1 the sum is also written back to slab 0.
// S = 0 or 1 shared experts: idx / w are [T, k + S] with rank k the shared
// expert (id E, weight 1).
hipError_t launch_topk(float* logits, int T, int E, int k, int splits, int32_t* idx,
                       float* w, hipStream_t s, int S = 0);
// Top-k that also hands each (token, rank) pair a slot of its expert
// (slot = atomicAdd(&counts[e], 1), counts zeroed beforehand; order within
// an expert is arbitrary, cap >= T), records pair = t*k + r in
// slot_pair[e*cap + slot], its gate weight in slot_w[e*cap + slot] and the
// token t in slot_tok[e*cap + slot].
hipError_t launch_topk_slots(float* logits, int T, int E, int k, int splits,
                             int32_t* idx, float* w, int32_t* counts, int cap,
                             int32_t* slot_pair, float* slot_w, int32_t* slot_tok,
                             hipStream_t s, int S = 0);
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int n_pairs, int E, int bm,
                          int32_t* chunk_counts, int32_t* local_rank,
                          int32_t* chunk_base, int32_t* offsets,
                          int32_t* tile_offsets, int32_t* counts,
                          int32_t* perm, hipStream_t s);
int permute_chunks(int n_pairs);
// counts[e] = offsets[e + 1] - offsets[e], e < E
hipError_t launch_counts_from_offsets(const int32_t* offsets, int E, int32_t* counts,
                                      hipStream_t s);
// x = E[tok] fused with the first RMSNorm (packed table).  With committed
// given, one more workgroup meanwhile writes row_map[0..M) = the rows t with
// committed[t] == 0 in increasing order, *m_dev = M and pos_map[t] (if
// given) = t's index in row_map or -1.
hipError_t launch_embed_norm(const int32_t* tokens, int T, const uint16_t* embed,
                             int V, int H, float* x, const float* g, float eps,
                             uint16_t* xh, hipStream_t s,
                             const uint8_t* committed = nullptr,
                             int32_t* row_map = nullptr, int32_t* m_dev = nullptr,
                             int32_t* pos_map = nullptr);
// x += un-permuted expert rows, fused with the next RMSNorm into xh.
hipError_t launch_unpermute_norm(const float* y, int T, int k, int H, float* x,
                                 float* moe_out, const float* g, float eps,
                                 uint16_t* xh, float* copy_f32,
                                 const int32_t* out_row, hipStream_t s);
// Per-row E4M3 quantisation of bf16 rows x [rows, ldx] (K values each, K
// a multiple of 8, at most 4096): scale[r] = max |x_r| / 448 (1 for a zero
// row), codes e4m3(x * (448 / max |x_r|)) into q8 [rows, K] and/or their
// values as bf16 into q16
// [rows, K] (either may be null).  With count (groups of cap rows), row r
// is skipped unless r % cap < count[r / cap].
hipError_t launch_quant_rows(const uint16_t* x, int ldx, int rows, int K,
                             const int32_t* count, int cap, uint8_t* q8,
                             uint16_t* q16, float* scale, hipStream_t s);

hipError_t launch_unpermute(const float* y, int T, int k, int H, float* x,
                            float* moe_out, hipStream_t s);
// With tau / spart / sample given: the rows' sampled tokens into sample,
// entropy 0 where tau <= 0.
hipError_t launch_lm_merge(const float4* part, int n_tiles,
                           const int32_t* m_dev, int m_max,
                           const int32_t* row_map, float* entropy, float* lse,
                           int32_t* argmax, hipStream_t s,
                           const float* tau = nullptr, const float2* spart = nullptr,
                           int32_t* sample = nullptr);
// Per LM-head row r < *m_dev (m_max without m_dev): the canvas position
// t = row_map[r] (r without row_map), its canvas b = t / C and step
// st = step[b]; tau[r] = tau0 (1 - st / budget) for budget > 0, tau0
// otherwise, clamped at 0; ctr[r] = (t % C, st, b).
hipError_t launch_sample_rows(const int32_t* row_map, const int32_t* m_dev, int m_max,
                              const int32_t* step, int C, float tau0, int budget,
                              float* tau, int32_t* ctr, hipStream_t s);
// EB selection over n canvases of C <= 256 positions each.
hipError_t launch_eb_select(int n, const float* entropy, const int32_t* argmax,
                            uint8_t* committed, int32_t* tokens, int32_t* step,
                            const float* gamma, int step_cap, int refine,
                            int32_t* n_new, uint8_t* done, hipStream_t s,
                            int C = DG_CANVAS);
hipError_t launch_kv_append(const uint16_t* qkv, int ldqkv, int col0_k,
                            int col0_v, int n, int C, int Hkv, int D,
                            uint16_t* kc, uint16_t* vc, long long req_stride,
                            long long head_stride, const int* req,
                            const int* row0, hipStream_t s);
hipError_t launch_kv_install(const uint16_t* src, int Hkv, int n, int D,
                             uint16_t* dst, long long head_stride,
                             hipStream_t s);

// Rows into an E4M3 cache (per-row quantisation as launch_quant_rows).
// For canvas b < n and row j < rows, head g < Hkv: the bf16 K (V) row starts
// at src_k (src_v) + b * src_b_stride + j * src_row_stride + g *
// src_head_stride and goes to cache row row0[b] + j of slot req[b], head g:
// codes at kc / vc + ((req * Hkv + g) * S + row) * D, scale at ks / vs +
// (req * Hkv + g) * S + row.
struct KvQuantArgs {
  const uint16_t* src_k;
  const uint16_t* src_v;
  long long src_b_stride, src_row_stride, src_head_stride;
  int n, rows, Hkv, D, S;
  uint8_t* kc;
  uint8_t* vc;
  float* ks;
  float* vs;
  int req[DG_MAX_BATCH];
  int row0[DG_MAX_BATCH];
};
hipError_t launch_kv_quant(const KvQuantArgs& a, hipStream_t s);

}  // namespace dg
