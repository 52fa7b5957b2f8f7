// Latency-scale kernels of the denoising step: embedding gather, RMSNorm,
// router top-k, the stable expert permutation, un-permute + residual,
// uncommitted-row compaction, the vocabulary-statistics merge, the
// entropy-bounded selection and the KV-cache copies.
#include <math.h>

#include "dg_internal.h"

namespace dg {
namespace {

// ---------------------------------------------------------------- embedding
// x[t, :] = E[tok_t, :] (bf16 -> fp32).  One workgroup per token.  Token ids
// outside [0, V) are clamped into range so that a bad id cannot read outside
// the embedding.
// Embedding rows gathered from the packed (MFMA-tiled) table: value k of
// row id sits in block (id / 16, k / 32), piece (id % 16) + 16 * (k % 32 / 8).
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* tok,
                                                    const uint16_t* E, int V,
                                                    int H, float* x) {
  const int t = blockIdx.x;
  const int id = min(max(tok[t], 0), V - 1);
  const char* base = (const char*)E;
  float* dst = x + (long long)t * H;
  for (int i = threadIdx.x * 8; i < H; i += 256 * 8) {
    const long long off = pack_block_offset(id >> 4, i >> 5, H, 2) +
                          16 * ((id & 15) + 16 * ((i & 31) >> 3));
    const uint4 v = *(const uint4*)(base + off);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float4 lo, hi;
    lo.x = bf2f((uint16_t)(w[0] & 0xffff)); lo.y = bf2f((uint16_t)(w[0] >> 16));
    lo.z = bf2f((uint16_t)(w[1] & 0xffff)); lo.w = bf2f((uint16_t)(w[1] >> 16));
    hi.x = bf2f((uint16_t)(w[2] & 0xffff)); hi.y = bf2f((uint16_t)(w[2] >> 16));
    hi.z = bf2f((uint16_t)(w[3] & 0xffff)); hi.w = bf2f((uint16_t)(w[3] >> 16));
    *(float4*)(dst + i) = lo;
    *(float4*)(dst + i + 4) = hi;
  }
}

// Row-major [groups][rows][cols] -> packed layout, one 16-byte piece per
// thread (grid-stride); rows are padded with zeros up to a multiple of 16.
__global__ __launch_bounds__(256) void pack_kernel(const char* src, int rows,
                                                   long long pieces_per_group,
                                                   int groups, int cols, int esz,
                                                   char* dst) {
  const long long total = pieces_per_group * groups;
  const int kb_n = cols / pack_k(esz);
  const int per_piece = 16 / esz;  // values per piece
  const long long src_group = (long long)rows * cols * esz;
  for (long long p = (long long)blockIdx.x * 256 + threadIdx.x; p < total;
       p += (long long)gridDim.x * 256) {
    const long long g = p / pieces_per_group, pin = p % pieces_per_group;
    const long long block = pin >> 6;
    const int lane = (int)(pin & 63);
    // block -> (tile group, kb, tile in group), see pack_block_offset
    const long long tg = block / ((long long)kb_n * kPackTiles);
    const int rem = (int)(block % ((long long)kb_n * kPackTiles));
    const int kb = rem / kPackTiles;
    const long long rb = tg * kPackTiles + rem % kPackTiles;
    const long long row = rb * 16 + (lane & 15);
    const long long col = (long long)kb * pack_k(esz) + (lane >> 4) * per_piece;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < rows) v = *(const uint4*)(src + g * src_group + (row * cols + col) * esz);
    *(uint4*)(dst + p * 16) = v;
  }
}

// ---------------------------------------------------------------- RMSNorm
// out[r, :] = bf16(x[src, :] / sqrt(mean(x^2) + eps) * g), one wave per row;
// src = row_map[r] when given, rows beyond *m_dev skipped.
// One workgroup per row; a thread holds up to 4 float4 of the row (H up to
// 4096 in registers, longer rows are read twice).
// Loads sit outside branches, at clamped (valid) addresses with the unused
// values dropped by selects: a load inside a branch makes the compiler wait
// for every load before it, one memory latency per load.
__device__ __forceinline__ int clamp_col(int i, int H) { return i < H ? i : H - 4; }

// acc + x^2 + y^2 + z^2 + w^2 as an explicit chain of fused multiply-adds:
// every kernel that norms a row (the RMSNorm, the embedding and the
// un-permute it is fused into) sums the squares in this one order, so a
// row gets the same norm bits whichever kernel norms it (left to the
// compiler, the contraction of a*a + b*b + ... depends on the surrounding
// code).
__device__ __forceinline__ float sumsq4(float4 v, float acc) {
  acc = fmaf(v.x, v.x, acc);
  acc = fmaf(v.y, v.y, acc);
  acc = fmaf(v.z, v.z, acc);
  return fmaf(v.w, v.w, acc);
}

template <int U>
__device__ __forceinline__ void load_gains(float4 (&gg)[U], const float* g, int H) {
#pragma unroll
  for (int c = 0; c < U; ++c)
    gg[c] = *(const float4*)(g + clamp_col(1024 * c + (int)threadIdx.x * 4, H));
}

template <int U>
__device__ __forceinline__ void norm_row(float4 (&v)[U], const float4 (&g0)[U],
                                         float ss, const float* xr, int H,
                                         const float* g, float eps,
                                         uint16_t* out, float* copy_f32,
                                         float* red) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += shfl_xor(ss, off);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  ss = red[0] + red[1] + red[2] + red[3];
  const float inv = rsqrtf(ss / (float)H + eps);
  for (int base = 0; base < H; base += 1024 * U) {
    float4 gg[U];
#pragma unroll
    for (int c = 0; c < U; ++c) gg[c] = g0[c];
    if (H > 1024 * U) {  // rows longer than the registers hold: read again
#pragma unroll
      for (int c = 0; c < U; ++c) {
        const int i = clamp_col(base + 1024 * c + tid * 4, H);
        v[c] = *(const float4*)(xr + i);
        gg[c] = *(const float4*)(g + i);
      }
    }
#pragma unroll
    for (int c = 0; c < U; ++c) {
      const int i = base + 1024 * c + tid * 4;
      if (i >= H) continue;
      const uint16_t b0 = f2bf(v[c].x * inv * gg[c].x), b1 = f2bf(v[c].y * inv * gg[c].y);
      const uint16_t b2 = f2bf(v[c].z * inv * gg[c].z), b3 = f2bf(v[c].w * inv * gg[c].w);
      *(uint2*)(out + i) = make_uint2((uint32_t)b0 | ((uint32_t)b1 << 16),
                                      (uint32_t)b2 | ((uint32_t)b3 << 16));
      if (copy_f32)
        *(float4*)(copy_f32 + i) = make_float4(bf2f(b0), bf2f(b1), bf2f(b2), bf2f(b3));
    }
  }
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(
    const float* x, int rows, int H, const float* g, float eps, uint16_t* out,
    const int32_t* row_map, const int32_t* m_dev, float* copy_f32,
    int32_t* zero, int n_zero) {
  constexpr int U = 4;
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  if (r == 0)
    for (int i = tid; i < n_zero; i += 256) zero[i] = 0;
  const int n = m_dev ? *m_dev : rows;
  const int src = row_map ? row_map[r] : r;
  float4 gg[U];
  load_gains<U>(gg, g, H);
  if (r >= n) return;
  const float* xr = x + (long long)src * H;
  float4 v[U];
  float ss = 0.f;
  // the first 1024*U columns straight-line (a loop header would wait for
  // the gain loads), the rest of a longer row in a loop
#pragma unroll
  for (int c = 0; c < U; ++c)
    v[c] = *(const float4*)(xr + clamp_col(1024 * c + tid * 4, H));
  for (int base = 0;;) {
#pragma unroll
    for (int c = 0; c < U; ++c) {
      if (base + 1024 * c + tid * 4 >= H) v[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      ss = sumsq4(v[c], ss);
    }
    base += 1024 * U;
    if (base >= H) break;
#pragma unroll
    for (int c = 0; c < U; ++c)
      v[c] = *(const float4*)(xr + clamp_col(base + 1024 * c + tid * 4, H));
  }
  norm_row<U>(v, gg, ss, xr, H, g, eps, out + (long long)r * H,
              copy_f32 ? copy_f32 + (long long)r * H : nullptr, red);
}

// ---------------------------------------------------------------- router top-k
// One wave per token; lane l holds the logits of experts l, l+64, l+128 and
// l+192.  Each logit becomes a unique 64-bit key (order-preserving bits of
// the logit above, 255 - expert id below), so "larger logit first, lower id
// first among equal logits" is plain key order; k rounds of a wave-wide
// maximum pick the selection in rank order, the owner of each winner
// dropping it.  Gate weights: softmax over the selected logits, summed in
// rank order.
constexpr int kTopkMaxE = 256, kTopkMaxK = 16;
// Maximum of x over the wave, returned to every lane as a uniform value:
// within each row of 16 lanes by DPP row shifts (lane 15 of a row ends with
// the row's maximum; lanes shifted in from outside the row bring 0, the
// identity), then the four row maxima by lane reads.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false));
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
  return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  if (v == 0.f) v = 0.f;  // -0 and +0 are equal logits
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// With S shared experts (0 or 1) a token's pairs are K = k + S: ranks
// 0..k-1 the routed experts, rank k the shared expert (id E, weight 1);
// idx / w are [T, K].
template <bool SLOTS>
__global__ __launch_bounds__(256) void topk_kernel(float* logits, int T, int E,
                                                   int k, int S, int splits, int32_t* idx,
                                                   float* w, int32_t* counts, int cap,
                                                   int32_t* slot_pair, float* slot_w,
                                                   int32_t* slot_tok) {
  constexpr int PER = kTopkMaxE / kWave;
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const long long slab = (long long)T * E, row = (long long)t * E;
  // the router's K splits left `splits` partial slabs: add them in order
  float part[PER][8];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = min(lane + kWave * i, E - 1);
#pragma unroll
    for (int sp = 0; sp < 8; ++sp)
      part[i][sp] = logits[(sp < splits ? sp : 0) * slab + row + e];
  }
  unsigned long long key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    key[i] = 0;  // below every real key
    if (e < E) {
      float v = part[i][0];
#pragma unroll
      for (int sp = 1; sp < 8; ++sp)
        if (sp < splits) v += part[i][sp];
      for (int sp = 8; sp < splits; ++sp) v += logits[sp * slab + row + e];
      if (splits > 1) logits[row + e] = v;
      key[i] = ((unsigned long long)ordered_bits(v) << 32) | (uint32_t)(255 - e);
    }
  }
  float sel[kTopkMaxK];
  int sid[kTopkMaxK];
#pragma unroll
  for (int r = 0; r < kTopkMaxK; ++r) {
    sel[r] = 0.f;
    sid[r] = 0;
    if (r < k) {
      // the largest key: the largest value, then among the keys holding it
      // the largest low word (the lowest expert)
      uint32_t hl = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) hl = max(hl, (uint32_t)(key[i] >> 32));
      const uint32_t vmax = wave_max_u32(hl);
      uint32_t ll = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if ((uint32_t)(key[i] >> 32) == vmax) ll = max(ll, (uint32_t)key[i]);
      const uint32_t lmax = wave_max_u32(ll);
      const unsigned long long m = ((unsigned long long)vmax << 32) | lmax;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (key[i] == m) key[i] = 0;
      sel[r] = from_ordered_bits(vmax);
      sid[r] = 255 - (int)lmax;
    }
  }
  const float mx = sel[0];
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < kTopkMaxK; ++r)
    if (r < k) sum += __expf(sel[r] - mx);
  float my_sel = 0.f;
  int my_id = 0;
#pragma unroll
  for (int r = 0; r < kTopkMaxK; ++r)
    if (r == lane) {
      my_sel = sel[r];
      my_id = sid[r];
    }
  float my_w = __expf(my_sel - mx) / sum;
  if (S && lane == k) {  // the shared expert: every token, weight 1
    my_id = E;
    my_w = 1.f;
  }
  const int K = k + S;
  if (lane < K) {
    idx[(long long)t * K + lane] = my_id;
    w[(long long)t * K + lane] = my_w;
  }
  if (SLOTS && lane < K) {  // lane r < K takes a slot of its expert
    // (cap >= T and cleared counters leave every slot below cap; the test
    // keeps a stale counter from writing past the expert's rows)
    const int i = atomicAdd(&counts[my_id], 1);
    if (i < cap) {
      const long long sl = (long long)my_id * cap + i;
      slot_pair[sl] = t * K + lane;
      slot_w[sl] = my_w;
      slot_tok[sl] = t;
    }
  }
}

// ---------------------------------------------------------------- permute
constexpr int kChunk = 256;

__global__ __launch_bounds__(kChunk) void moe_count_kernel(
    const int32_t* idx, int n_pairs, int E, int32_t* chunk_counts,
    int32_t* local_rank) {
  __shared__ int ex[kChunk];
  __shared__ int hist[256];
  const int tid = threadIdx.x;
  const int p = blockIdx.x * kChunk + tid;
  const int e = p < n_pairs ? idx[p] : -1;
  ex[tid] = e;
  if (tid < E) hist[tid] = 0;
  __syncthreads();
  if (e >= 0) {
    int rank = 0;
    for (int q = 0; q < tid; ++q) rank += (ex[q] == e);
    local_rank[p] = rank;
    atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (tid < E) chunk_counts[(long long)blockIdx.x * E + tid] = hist[tid];
}

// Column scans of the chunk histogram [n_chunks][E]: expert offsets (the
// exclusive scan of the experts' totals), tile offsets and each chunk's
// base slot per expert.  1024 threads: thread t takes expert t % 256 (E <=
// 256) and the contiguous run of chunks of part t / 256 (4 parts), so the
// loads of a thread are independent and 4 x E of them are in flight.
constexpr int kScanParts = 4;
__global__ __launch_bounds__(1024) void moe_scan_kernel(
    int n_chunks, int E, int bm, const int32_t* chunk_counts,
    int32_t* chunk_base, int32_t* offsets, int32_t* tile_offsets,
    int32_t* counts) {
  __shared__ int s_part[kScanParts][256];
  __shared__ int s_off[256];
  __shared__ int s_tiles[256];
  const int e = threadIdx.x & 255, part = threadIdx.x >> 8;
  const int per = (n_chunks + kScanParts - 1) / kScanParts;
  const int c0 = part * per, c1 = min(n_chunks, c0 + per);
  constexpr int U = 8;
  int sum = 0;
  if (e < E)
    for (int c = c0; c < c1; c += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = c + u < c1 ? chunk_counts[(long long)(c + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) sum += v[u];
    }
  s_part[part][e] = e < E ? sum : 0;
  __syncthreads();
  if (threadIdx.x < 256) {
    int tot = 0;
#pragma unroll
    for (int q = 0; q < kScanParts; ++q) tot += s_part[q][e];
    s_off[e] = tot;
    s_tiles[e] = (tot + bm - 1) / bm;
    if (e < E && counts) counts[e] = tot;
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // exclusive scans over the (<= 256) experts
    int run = 0, runt = 0;
    for (int q = 0; q < E; ++q) {
      const int o = s_off[q];
      s_off[q] = run;
      run += o;
      const int ot = s_tiles[q];
      s_tiles[q] = runt;
      runt += ot;
    }
    offsets[E] = run;
    tile_offsets[E] = runt;
  }
  __syncthreads();
  if (threadIdx.x < E) {
    offsets[e] = s_off[e];
    tile_offsets[e] = s_tiles[e];
  }
  if (e >= E) return;
  // base of this part's first chunk: the expert's offset plus the earlier
  // parts' counts
  int base = s_off[e];
  for (int q = 0; q < part; ++q) base += s_part[q][e];
  for (int c = c0; c < c1; c += U) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = c + u < c1 ? chunk_counts[(long long)(c + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (c + u < c1) {
        chunk_base[(long long)(c + u) * E + e] = base;
        base += v[u];
      }
  }
}

__global__ __launch_bounds__(kChunk) void moe_scatter_kernel(
    const int32_t* idx, int n_pairs, int E, const int32_t* chunk_base,
    const int32_t* local_rank, int32_t* perm) {
  const int p = blockIdx.x * kChunk + threadIdx.x;
  if (p >= n_pairs) return;
  const int e = idx[p];
  perm[chunk_base[(long long)blockIdx.x * E + e] + local_rank[p]] = p;
}

// Counting sort of up to kSmallPairs pairs in one workgroup: LDS histogram,
// one scan for the expert offsets and tile offsets, then each pair takes the
// next free slot of its expert from an LDS cursor.  The order of the pairs
// inside an expert's range is arbitrary and does not matter: every pair's
// expert output is its own dot products, and the un-permute adds a token's
// pairs in rank order, so results are the same for any order.
constexpr int kSmallPairs = 4096;
__global__ __launch_bounds__(1024) void moe_permute_small_kernel(
    const int32_t* idx, int n_pairs, int E, int bm, int32_t* offsets,
    int32_t* tile_offsets, int32_t* counts, int32_t* perm) {
  __shared__ int hist[256], cursor[256], tiles[256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  int e4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int p = tid + 1024 * r;
    const int e = idx[p < n_pairs ? p : n_pairs - 1];
    e4[r] = p < n_pairs ? e : -1;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (e4[r] >= 0) atomicAdd(&hist[e4[r]], 1);
  }
  __syncthreads();
  if (tid < 256) tiles[tid] = tid < E ? (hist[tid] + bm - 1) / bm : 0;
  __syncthreads();
  if (wave == 0) {  // exclusive scans of counts and tiles, 4 experts a lane
    int c4[4], t4[4], cs = 0, ts = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      c4[c] = 4 * lane + c < E ? hist[4 * lane + c] : 0;
      t4[c] = tiles[4 * lane + c];
      cs += c4[c];
      ts += t4[c];
    }
    int ci = cs, ti = ts;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int co = __shfl_up(ci, off), to = __shfl_up(ti, off);
      if (lane >= off) { ci += co; ti += to; }
    }
    int cr = ci - cs, tr = ti - ts;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = 4 * lane + c;
      if (e < E) {
        offsets[e] = cr;
        tile_offsets[e] = tr;
        if (counts) counts[e] = c4[c];
        cursor[e] = cr;
      }
      cr += c4[c];
      tr += t4[c];
    }
    if (lane == 63) {
      offsets[E] = ci;
      tile_offsets[E] = ti;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (e4[r] >= 0) perm[atomicAdd(&cursor[e4[r]], 1)] = tid + 1024 * r;
}

// counts[e] = offsets[e + 1] - offsets[e] for e < E (the routed experts'
// token counts out of the permutation's offsets over all expert groups)
__global__ __launch_bounds__(256) void counts_kernel(const int32_t* offsets, int E,
                                                     int32_t* counts) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e < E) counts[e] = offsets[e + 1] - offsets[e];
}

// ---------------------------------------------------------------- un-permute
// x[t, :] += sum_j y[t*k + j, :] in rank order (no atomics); optionally the
// sum alone is written to moe_out.  x may be null (store only).
__global__ __launch_bounds__(256) void unpermute_kernel(const float* y, int k,
                                                        int H, float* x,
                                                        float* moe_out) {
  constexpr int KMAX = 16;
  const int t = blockIdx.x;
  for (int i = threadIdx.x * 4; i < H; i += 1024) {
    float4 v[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      v[j] = *(const float4*)(y + ((long long)t * k + (j < k ? j : 0)) * H + i);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) { s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w; }
    if (x) {  // (the x load is issued before the sums wait for y)
      float4* xp = (float4*)(x + (long long)t * H + i);
      float4 o = *xp;
      o.x += s.x; o.y += s.y; o.z += s.z; o.w += s.w;
      *xp = o;
    }
    if (moe_out) *(float4*)(moe_out + (long long)t * H + i) = s;
  }
}

// ---------------------------------------------------------------- fused row norms
// Block-wide RMSNorm of a row whose values this thread holds as v[c] at
// columns base + 1024 c + 4 tid (c < U); rows longer than 1024 U are read
// back from xr (written earlier by this same thread).  out = bf16(x * inv
// * g); copy_f32 optionally receives the bf16 values widened.

// Embedding gather (packed table, ids clamped) fused with the first layer's
// attention RMSNorm: x[t] = E[tok[t]] (fp32), xh[t] = RMSNorm(x[t]; g), one
// workgroup per row t < T.  With committed given, workgroup T compacts the
// uncommitted rows (compact_rows) meanwhile.
template <int NTH>
__device__ void compact_rows(const uint8_t* committed, int T, int32_t* row_map,
                             int32_t* m_dev, int32_t* pos_map);
__global__ __launch_bounds__(256) void embed_norm_kernel(
    const int32_t* tok, int T, const uint16_t* E, int V, int H, float* x, const float* g,
    float eps, uint16_t* xh, const uint8_t* committed, int32_t* row_map, int32_t* m_dev,
    int32_t* pos_map) {
  constexpr int U = 4;
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (t >= T) {
    compact_rows<256>(committed, T, row_map, m_dev, pos_map);
    return;
  }
  const int id = min(max(tok[t], 0), V - 1);
  float4 gg[U];
  load_gains<U>(gg, g, H);
  const char* base = (const char*)E;
  float* xr = x + (long long)t * H;
  float4 v[U];
  float ss = 0.f;
  for (int b0 = 0; b0 < H; b0 += 1024 * U) {
    uint2 w[U];
#pragma unroll
    for (int c = 0; c < U; ++c) {
      // columns i..i+3: half of one 16-byte packed piece
      const int i = clamp_col(b0 + 1024 * c + tid * 4, H);
      const long long off = pack_block_offset(id >> 4, i >> 5, H, 2) +
                            16 * ((id & 15) + 16 * ((i & 31) >> 3)) + 2 * (i & 7);
      w[c] = *(const uint2*)(base + off);
    }
#pragma unroll
    for (int c = 0; c < U; ++c) {
      const int i = b0 + 1024 * c + tid * 4;
      v[c] = make_float4(bf2f((uint16_t)(w[c].x & 0xffff)), bf2f((uint16_t)(w[c].x >> 16)),
                         bf2f((uint16_t)(w[c].y & 0xffff)), bf2f((uint16_t)(w[c].y >> 16)));
      if (i < H) {
        *(float4*)(xr + i) = v[c];
        ss = sumsq4(v[c], ss);
      }
    }
  }
  norm_row<U>(v, gg, ss, xr, H, g, eps, xh + (long long)t * H, nullptr, red);
}

// Un-permute fused with the next RMSNorm: x[t] += sum_j y[t*k + j] in rank
// order (moe_out[t] = the sum, if given), then xh[r] = RMSNorm(x[t]; g) with
// r = out_row[t] (no output when -1) or t (copy_f32[r] = widened xh[r], if
// given).
// KMAX: compile-time bound on k (8 or 16), so the y loads of every slot
// can be issued at once without loading beyond the k slots present.
template <int KMAX>
__global__ __launch_bounds__(256) void unpermute_norm_kernel(
    const float* y, int k, int H, float* x, float* moe_out, const float* g,
    float eps, uint16_t* xh, float* copy_f32, const int32_t* out_row) {
  constexpr int U = 4;
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  // the norm goes to row out_row[t] (skipped when -1), or to row t
  const int orow = out_row ? out_row[t] : t;
  float4 gg[U];
  load_gains<U>(gg, g, H);
  float* xr = x + (long long)t * H;
  float4 v[U];
  float ss = 0.f;
  for (int b0 = 0; b0 < H; b0 += 1024 * U) {
#pragma unroll
    for (int c = 0; c < U; ++c) {
      const int i = b0 + 1024 * c + tid * 4;
      const int ic = clamp_col(i, H);
      float4 yy[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
      {
        // expert outputs are read once: non-temporal loads (32 canvases:
        // 537 MB a layer, 133-143 -> 109 us)
        const f32x4_t q = __builtin_nontemporal_load(
            (const f32x4_t*)(y + ((long long)t * k + (j < k ? j : 0)) * H + ic));
        yy[j] = make_float4(q[0], q[1], q[2], q[3]);
      }
      float4 o = *(const float4*)(xr + ic);
      float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) { sum.x += yy[j].x; sum.y += yy[j].y; sum.z += yy[j].z; sum.w += yy[j].w; }
      o.x += sum.x; o.y += sum.y; o.z += sum.z; o.w += sum.w;
      if (i < H) {
        *(float4*)(xr + i) = o;
        if (moe_out) *(float4*)(moe_out + (long long)t * H + i) = sum;
        ss = sumsq4(o, ss);
      } else {
        o = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      v[c] = o;
    }
  }
  if (orow < 0) return;
  norm_row<U>(v, gg, ss, xr, H, g, eps, xh + (long long)orow * H,
              copy_f32 ? copy_f32 + (long long)orow * H : nullptr, red);
}

// ---------------------------------------------------------------- compaction
__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// row_map[0..M) = indices t with committed[t] == 0 in increasing order;
// *m_dev = M; pos_map[t] (if given) = t's index in row_map, or -1.  Run by
// one workgroup of NTH threads: chunks of NTH positions, 8 chunks' flags
// read at once; in-wave ranks from ballots, wave offsets from the wave
// counts.
template <int NTH>
__device__ void compact_rows(const uint8_t* committed, int T, int32_t* row_map,
                             int32_t* m_dev, int32_t* pos_map) {
  constexpr int G = 8, NW = NTH / 64;
  __shared__ int wcount[G][NW];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const unsigned long long below = (1ull << lane) - 1;
  int run = 0;
  for (int base = 0; base < T; base += NTH * G) {
    bool f[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int t = base + NTH * i + tid;
      const uint8_t c = committed[t < T ? t : T - 1];
      f[i] = t < T && c == 0;
    }
    int before[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const unsigned long long bal = __ballot(f[i]);
      before[i] = __popcll(bal & below);
      if (lane == 0) wcount[i][wv] = __popcll(bal);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < G; ++i) {
      int off = run, total = 0;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const int c = wcount[i][q];
        off += q < wv ? c : 0;
        total += c;
      }
      const int t = base + NTH * i + tid;
      const int r = off + before[i];
      if (f[i]) row_map[r] = t;
      if (pos_map && t < T) pos_map[t] = f[i] ? r : -1;
      run += total;
    }
    __syncthreads();  // wcount is reused
  }
  if (tid == 0) *m_dev = run;
}

// ---------------------------------------------------------------- LM merge
// Reduce the per-tile (max, sum e^(z-max), sum e^(z-max)(z-max), argmax)
// partials of a row in a fixed order: lse = max + ln s, entropy =
// ln s - t / s (clamped at 0), argmax lowest id among maxima.
__device__ __forceinline__ void merge_stats(float& m, float& s, float& t,
                                            int& am, float m2, float s2,
                                            float t2, int am2) {
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

// One workgroup per row: each thread merges 8 tiles' partials at a time
// (loads issued together), then the wave and the 4 waves are merged.
__global__ __launch_bounds__(256) void lm_merge_kernel(
    const float4* part, int n_tiles, const int32_t* m_dev, int m_max,
    const int32_t* row_map, float* entropy, float* lse, int32_t* argmax,
    const float* tau, const float2* spart, int32_t* sample) {
  constexpr int U = 8;
  __shared__ float4 red[4];
  __shared__ float2 red2[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = blockIdx.x;
  const int n = m_dev ? *m_dev : m_max;
  if (r >= n) return;
  float m = -INFINITY, s = 0.f, t = 0.f;
  int am = 0x7fffffff;
  const float4* pr = part + (long long)r * n_tiles;
  for (int base = 0; base < n_tiles; base += 256 * U) {
    float4 p[U];
#pragma unroll
    for (int c = 0; c < U; ++c) {
      const int i = base + 256 * c + tid;
      p[c] = i < n_tiles ? pr[i] : make_float4(-INFINITY, 0.f, 0.f, __int_as_float(0x7fffffff));
    }
#pragma unroll
    for (int c = 0; c < U; ++c) merge_stats(m, s, t, am, p[c].x, p[c].y, p[c].z, __float_as_int(p[c].w));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = shfl_xor(m, off), s2 = shfl_xor(s, off);
    const float t2 = shfl_xor(t, off);
    const int am2 = shfl_xor(am, off);
    merge_stats(m, s, t, am, m2, s2, t2, am2);
  }
  if (lane == 0) red[wave] = make_float4(m, s, t, __int_as_float(am));
  // sampled token: the best (score, id) over the tiles, lower id on ties
  float g = -INFINITY;
  int gi = 0x7fffffff;
  if (sample) {
    const float2* sp = spart + (long long)r * n_tiles;
    for (int i = tid; i < n_tiles; i += 256) {
      const float2 q = sp[i];
      best_merge(g, gi, q.x, __float_as_int(q.y));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
      best_merge(g, gi, shfl_xor(g, off), shfl_xor(gi, off));
    if (lane == 0) red2[wave] = make_float2(g, __int_as_float(gi));
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int w = 1; w < 4; ++w)
      merge_stats(m, s, t, am, red[w].x, red[w].y, red[w].z, __float_as_int(red[w].w));
    const int pos = row_map ? row_map[r] : r;
    const float ls = logf(s);
    lse[pos] = m + ls;
    entropy[pos] = fmaxf(ls - t / s, 0.f);
    argmax[pos] = am;
    if (sample) {
#pragma unroll
      for (int w = 1; w < 4; ++w) best_merge(g, gi, red2[w].x, __float_as_int(red2[w].y));
      // temperature 0: the point mass on the argmax
      if (!(tau[r] > 0.f)) {
        entropy[pos] = 0.f;
        gi = am;
      }
      sample[pos] = gi;
    }
  }
}

// Temperature and Philox counter words of each LM-head row (see
// launch_sample_rows).
__global__ __launch_bounds__(256) void sample_rows_kernel(
    const int32_t* row_map, const int32_t* m_dev, int m_max, const int32_t* step, int C,
    float tau0, int budget, float* tau, int32_t* ctr) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int m = m_dev ? *m_dev : m_max;
  if (r >= m) return;
  const int t = row_map ? row_map[r] : r;
  const int b = t / C;
  const int st = step[b];
  float tt = tau0;
  if (budget > 0) tt = tau0 * (1.f - (float)st / (float)budget);
  tau[r] = fmaxf(tt, 0.f);
  ctr[3 * r] = t % C;
  ctr[3 * r + 1] = st;
  ctr[3 * r + 2] = b;
}

// One workgroup of 256 threads per canvas of C <= 256 positions (thread j
// takes position j; threads j >= C hold no position).
__global__ __launch_bounds__(256) void eb_kernel(
    const float* entropy, const int32_t* argmax, uint8_t* committed,
    int32_t* tokens, int32_t* step, const float* gamma, int cap, int refine,
    int32_t* n_new, uint8_t* done, int C) {
  static_assert(DG_CANVAS == 256, "one thread per canvas position");
  __shared__ __attribute__((aligned(16))) unsigned long long keys[DG_CANVAS];
  __shared__ float sorted_h[DG_CANVAS];
  __shared__ double wave_sum[4];
  __shared__ int s_first;
  const int b = blockIdx.x, j = threadIdx.x, lane = j & 63, w = j >> 6;
  const long long base = (long long)b * C;
  const bool here = j < C;
  const int jc = here ? j : C - 1;   // (a valid address; the value is unused)
  // every global read issued at once (values at committed positions are
  // read but not used): one memory latency instead of a chain of them
  const uint8_t cm = here ? committed[base + jc] : (uint8_t)1;
  const float h_in = entropy[base + jc];
  const int32_t am_in = argmax[base + jc];
  const float lim = gamma[b];
  const int steps_done = step[b];  // read by all before thread 0 updates it
  const bool unc = cm == 0;
  float h = unc ? h_in : 0.f;
  if (h == 0.f) h = 0.f;  // -0 -> +0
  uint32_t u = __float_as_uint(h);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // order-preserving
  // (entropy, position) as one key: ties go to the lower position
  const unsigned long long key =
      unc ? (((unsigned long long)u << 32) | (unsigned)j) : ~0ull;
  keys[j] = key;
  if (j == 0) s_first = DG_CANVAS;
  const int n_unc = __syncthreads_count(unc);
  if (n_unc == 0) {
    if (j == 0) {
      n_new[b] = 0;
      done[b] = 1;
    }
    return;
  }
  // rank = number of smaller keys; committed positions hold the largest key
  int rank = 0;
  const ulonglong2* k2 = reinterpret_cast<const ulonglong2*>(keys);
#pragma unroll 8
  for (int i = 0; i < DG_CANVAS / 2; ++i) {
    const ulonglong2 kk = k2[i];
    rank += (kk.x < key) + (kk.y < key);
  }
  if (unc) sorted_h[rank] = h;
  __syncthreads();
  // inclusive prefix sums of the sorted entropies in fp64
  double c = j < n_unc ? (double)sorted_h[j] : 0.0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(c, o, 64);
    if (lane >= o) c += t;
  }
  if (lane == 63) wave_sum[w] = c;
  __syncthreads();
  for (int q = 0; q < w; ++q) c += wave_sum[q];
  // n* = length of the longest sorted prefix whose sum stays within gamma
  if (j < n_unc && c > (double)lim) atomicMin(&s_first, j);
  __syncthreads();
  int n = min(s_first, n_unc);
  if (n < 1) n = 1;
  if (steps_done + 1 >= cap) n = n_unc;
  if (unc) {
    if (rank < n) {
      committed[base + j] = 1;
      tokens[base + j] = am_in;
    } else if (refine) {
      tokens[base + j] = am_in;
    }
  }
  if (j == 0) {
    step[b] = steps_done + 1;
    n_new[b] = n;
    done[b] = (n == n_unc) ? 1 : 0;
  }
}

// ---------------------------------------------------------------- KV copies
struct KvAppendArgs {
  const uint16_t* qkv;
  int ldqkv, col0_k, col0_v, C, Hkv, D;
  uint16_t* kc;
  uint16_t* vc;
  long long req_stride, head_stride;
  int req[DG_MAX_BATCH];
  int row0[DG_MAX_BATCH];
};

__global__ __launch_bounds__(256) void kv_append_kernel(KvAppendArgs a) {
  const int b = blockIdx.y;
  const int per_row = a.Hkv * (a.D / 8);
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.C * per_row) return;
  const int j = c / per_row, rem = c % per_row;
  const int g = rem / (a.D / 8), dc = rem % (a.D / 8);
  const uint16_t* src = a.qkv + (long long)(b * a.C + j) * a.ldqkv + g * a.D + dc * 8;
  const long long dst = (long long)a.req[b] * a.req_stride +
                        (long long)g * a.head_stride +
                        (long long)(a.row0[b] + j) * a.D + dc * 8;
  *(uint4*)(a.kc + dst) = *(const uint4*)(src + a.col0_k);
  *(uint4*)(a.vc + dst) = *(const uint4*)(src + a.col0_v);
}

// src [Hkv][n][D] -> dst [Hkv][max_kv_len][D] rows [0, n)
__global__ __launch_bounds__(256) void kv_install_kernel(const uint16_t* src,
                                                         int Hkv, int n, int D,
                                                         uint16_t* dst,
                                                         long long head_stride) {
  const long long c = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long per_head = (long long)n * (D / 8);
  if (c >= Hkv * per_head) return;
  const int g = (int)(c / per_head);
  const long long rem = c % per_head;
  const long long row = rem / (D / 8);
  const int dc = (int)(rem % (D / 8));
  *(uint4*)(dst + g * head_stride + row * D + dc * 8) =
      *(const uint4*)(src + ((long long)g * n + row) * D + dc * 8);
}

}  // namespace

hipError_t launch_pack(const void* src, int groups, int rows, int cols, int esz,
                       void* dst, hipStream_t s) {
  const long long ppg =
      (long long)((rows + kPackRows - 1) / kPackRows * kPackRows) * cols * esz / 16;
  if (ppg * groups <= 0) return hipSuccess;
  const long long blocks = std::min<long long>((ppg * groups + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const char*)src, rows, ppg, groups, cols, esz, (char*)dst);
  return hipGetLastError();
}

hipError_t launch_embed(const int32_t* tokens, int T, const uint16_t* embed,
                        int V, int H, float* x, hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(T), dim3(256), 0, s, tokens, embed, V,
                     H, x);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, int rows, int H, const float* g,
                          float eps, uint16_t* out, const int32_t* row_map,
                          const int32_t* m_dev, float* copy_f32,
                          hipStream_t s, int32_t* zero, int n_zero) {
  if (rows <= 0) return launch_zero_i32(zero, zero ? n_zero : 0, s);
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(256), 0, s, x,
                     rows, H, g, eps, out, row_map, m_dev, copy_f32, zero,
                     zero ? n_zero : 0);
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_topk(float* logits, int T, int E, int k, int splits, int32_t* idx,
                       float* w, hipStream_t s, int S) {
  if (T <= 0) return hipSuccess;
  if (E > kTopkMaxE || k > kTopkMaxK || k > E || S < 0 || S > 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_kernel<false>, dim3((T + 3) / 4), dim3(256), 0, s, logits,
                     T, E, k, S, splits, idx, w, nullptr, 0, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_topk_slots(float* logits, int T, int E, int k, int splits,
                             int32_t* idx, float* w, int32_t* counts, int cap,
                             int32_t* slot_pair, float* slot_w, int32_t* slot_tok,
                             hipStream_t s, int S) {
  if (T <= 0) return hipSuccess;
  if (E > kTopkMaxE || k > kTopkMaxK || k > E || cap < T || S < 0 || S > 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_kernel<true>, dim3((T + 3) / 4), dim3(256), 0, s, logits,
                     T, E, k, S, splits, idx, w, counts, cap, slot_pair, slot_w, slot_tok);
  return hipGetLastError();
}

int permute_chunks(int n_pairs) { return (n_pairs + kChunk - 1) / kChunk; }

hipError_t launch_counts_from_offsets(const int32_t* offsets, int E, int32_t* counts,
                                      hipStream_t s) {
  if (E <= 0) return hipSuccess;
  hipLaunchKernelGGL(counts_kernel, dim3((E + 255) / 256), dim3(256), 0, s, offsets, E,
                     counts);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int n_pairs, int E, int bm,
                          int32_t* chunk_counts, int32_t* local_rank,
                          int32_t* chunk_base, int32_t* offsets,
                          int32_t* tile_offsets, int32_t* counts,
                          int32_t* perm, hipStream_t s) {
  if (n_pairs <= kSmallPairs && E <= 256) {
    hipLaunchKernelGGL(moe_permute_small_kernel, dim3(1), dim3(1024), 0, s, idx,
                       n_pairs, E, bm, offsets, tile_offsets, counts, perm);
    return hipGetLastError();
  }
  if (E > 256) return hipErrorInvalidValue;
  const int nc = permute_chunks(n_pairs);
  hipLaunchKernelGGL(moe_count_kernel, dim3(nc), dim3(kChunk), 0, s, idx,
                     n_pairs, E, chunk_counts, local_rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(1024), 0, s, nc, E, bm,
                     chunk_counts, chunk_base, offsets, tile_offsets, counts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(nc), dim3(kChunk), 0, s, idx,
                     n_pairs, E, chunk_base, local_rank, perm);
  return hipGetLastError();
}

// One wave per row (4 rows per workgroup): the row's 16-byte runs of 8
// values stay in registers (K <= 64 x 8 x kQuantRuns), the max |x| is a wave
// reduction, then each value is multiplied by r = 448 / max (fp32), clamped
// to +-448 and encoded by gfx950's packed fp32 -> E4M3 conversion (nearest,
// ties to even: checked bit for bit against the format's definition for
// every fp32 input of magnitude <= 448).
constexpr int kQuantRuns = 8;
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t* x, int ldx, int rows, int K, const int32_t* count, int cap,
    uint8_t* q8, uint16_t* q16, float* scale) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  if (count && r % cap >= count[r / cap]) return;
  const uint16_t* xr = x + (long long)r * ldx;
  const int runs = K >> 3;
  uint4 v[kQuantRuns];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kQuantRuns; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < runs ? *(const uint4*)(xr + 8 * c) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(bf2f((uint16_t)(w[j] & 0xFFFFu))));
      amax = fmaxf(amax, fabsf(bf2f((uint16_t)(w[j] >> 16))));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, shfl_xor(amax, off));
  const float sc = amax > 0.f ? amax / 448.f : 1.f;
  const float mul = amax > 0.f ? 448.f / amax : 1.f;
  if (lane == 0) scale[r] = sc;
#pragma unroll
  for (int i = 0; i < kQuantRuns; ++i) {
    const int c = lane + 64 * i;
    if (c >= runs) break;
    const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
    uint32_t pk[2];   // 8 codes, byte j = value j
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float f[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f[2 * j] = fminf(fmaxf(bf2f((uint16_t)(w[2 * h + j] & 0xFFFFu)) * mul, -448.f), 448.f);
        f[2 * j + 1] = fminf(fmaxf(bf2f((uint16_t)(w[2 * h + j] >> 16)) * mul, -448.f), 448.f);
      }
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], p, true);
      pk[h] = (uint32_t)p;
    }
    if (q8) *(uint2*)(q8 + (long long)r * K + 8 * c) = make_uint2(pk[0], pk[1]);
    if (q16) {
      u32x4_t lo, hi;
      widen_e4m3x16(u32x4_t{pk[0], pk[1], 0u, 0u}, lo, hi);
      *(uint4*)(q16 + (long long)r * K + 8 * c) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
  }
}

// One wave per (row, head) of a canvas: the K row, then the V row, each
// quantised as in quant_rows_kernel (D <= 128: at most 2 values a lane).
__global__ __launch_bounds__(256) void kv_quant_kernel(KvQuantArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (item >= a.rows * a.Hkv) return;
  const int j = item / a.Hkv, g = item % a.Hkv;
  const long long off = (long long)b * a.src_b_stride + (long long)j * a.src_row_stride +
                        (long long)g * a.src_head_stride;
  const long long crow = ((long long)a.req[b] * a.Hkv + g) * a.S + a.row0[b] + j;
  const int per = a.D >> 6;  // values per lane (1 or 2)
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const uint16_t* r = (kv ? a.src_v : a.src_k) + off;
    float v0 = 0.f, v1 = 0.f;
    if (per == 2) {
      const uint32_t w = *(const uint32_t*)(r + 2 * lane);
      v0 = bf2f((uint16_t)(w & 0xFFFFu));
      v1 = bf2f((uint16_t)(w >> 16));
    } else {
      v0 = bf2f(r[lane]);
    }
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, shfl_xor(amax, off));
    const float sc = amax > 0.f ? amax / 448.f : 1.f;
    const float mul = amax > 0.f ? 448.f / amax : 1.f;
    const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(v0 * mul, -448.f), 448.f),
                                                   fminf(fmaxf(v1 * mul, -448.f), 448.f), 0,
                                                   false);
    uint8_t* codes = (kv ? a.vc : a.kc) + crow * a.D;
    if (per == 2) *(uint16_t*)(codes + 2 * lane) = (uint16_t)(pk & 0xFFFF);
    else codes[lane] = (uint8_t)(pk & 0xFF);
    if (lane == 0) (kv ? a.vs : a.ks)[crow] = sc;
  }
}

hipError_t launch_kv_quant(const KvQuantArgs& a, hipStream_t s) {
  if (a.n <= 0 || a.rows <= 0) return hipSuccess;
  if ((a.D != 64 && a.D != 128) || a.n > DG_MAX_BATCH) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_quant_kernel, dim3((a.rows * a.Hkv + 3) / 4, a.n), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int ldx, int rows, int K,
                             const int32_t* count, int cap, uint8_t* q8,
                             uint16_t* q16, float* scale, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (K <= 0 || K % 8 || K > 64 * 8 * kQuantRuns || ldx % 8 || (count && cap <= 0))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, x, ldx,
                     rows, K, count, cap, q8, q16, scale);
  return hipGetLastError();
}

hipError_t launch_embed_norm(const int32_t* tokens, int T, const uint16_t* embed,
                             int V, int H, float* x, const float* g, float eps,
                             uint16_t* xh, hipStream_t s, const uint8_t* committed,
                             int32_t* row_map, int32_t* m_dev, int32_t* pos_map) {
  if (T <= 0) return hipSuccess;
  if (committed && (!row_map || !m_dev)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(embed_norm_kernel, dim3(T + (committed ? 1 : 0)), dim3(256), 0, s,
                     tokens, T, embed, V, H, x, g, eps, xh, committed, row_map, m_dev,
                     pos_map);
  return hipGetLastError();
}

hipError_t launch_unpermute_norm(const float* y, int T, int k, int H, float* x,
                                 float* moe_out, const float* g, float eps,
                                 uint16_t* xh, float* copy_f32,
                                 const int32_t* out_row, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (k > 16) return hipErrorInvalidValue;
  if (k <= 8)
    hipLaunchKernelGGL(unpermute_norm_kernel<8>, dim3(T), dim3(256), 0, s, y, k, H, x,
                       moe_out, g, eps, xh, copy_f32, out_row);
  else
    hipLaunchKernelGGL(unpermute_norm_kernel<16>, dim3(T), dim3(256), 0, s, y, k, H, x,
                       moe_out, g, eps, xh, copy_f32, out_row);
  return hipGetLastError();
}

hipError_t launch_unpermute(const float* y, int T, int k, int H, float* x,
                            float* moe_out, hipStream_t s) {
  hipLaunchKernelGGL(unpermute_kernel, dim3(T), dim3(256), 0, s, y, k, H, x,
                     moe_out);
  return hipGetLastError();
}


hipError_t launch_lm_merge(const float4* part, int n_tiles,
                           const int32_t* m_dev, int m_max,
                           const int32_t* row_map, float* entropy, float* lse,
                           int32_t* argmax, hipStream_t s, const float* tau,
                           const float2* spart, int32_t* sample) {
  if (m_max <= 0) return hipSuccess;
  if (sample && (!tau || !spart)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lm_merge_kernel, dim3(m_max), dim3(256), 0, s,
                     part, n_tiles, m_dev, m_max, row_map, entropy, lse,
                     argmax, tau, spart, sample);
  return hipGetLastError();
}

hipError_t launch_sample_rows(const int32_t* row_map, const int32_t* m_dev, int m_max,
                              const int32_t* step, int C, float tau0, int budget,
                              float* tau, int32_t* ctr, hipStream_t s) {
  if (m_max <= 0) return hipSuccess;
  hipLaunchKernelGGL(sample_rows_kernel, dim3((m_max + 255) / 256), dim3(256), 0, s,
                     row_map, m_dev, m_max, step, C, tau0, budget, tau, ctr);
  return hipGetLastError();
}

hipError_t launch_eb_select(int n, const float* entropy, const int32_t* argmax,
                            uint8_t* committed, int32_t* tokens, int32_t* step,
                            const float* gamma, int step_cap, int refine,
                            int32_t* n_new, uint8_t* done, hipStream_t s, int C) {
  if (C < 1 || C > DG_CANVAS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(eb_kernel, dim3(n), dim3(DG_CANVAS), 0, s, entropy, argmax,
                     committed, tokens, step, gamma, step_cap, refine, n_new,
                     done, C);
  return hipGetLastError();
}

hipError_t launch_kv_append(const uint16_t* qkv, int ldqkv, int col0_k,
                            int col0_v, int n, int C, int Hkv, int D,
                            uint16_t* kc, uint16_t* vc, long long req_stride,
                            long long head_stride, const int* req,
                            const int* row0, hipStream_t s) {
  KvAppendArgs a;
  a.qkv = qkv; a.ldqkv = ldqkv; a.col0_k = col0_k; a.col0_v = col0_v;
  a.C = C; a.Hkv = Hkv; a.D = D; a.kc = kc; a.vc = vc;
  a.req_stride = req_stride; a.head_stride = head_stride;
  for (int b = 0; b < n; ++b) { a.req[b] = req[b]; a.row0[b] = row0[b]; }
  const int total = C * Hkv * (D / 8);
  hipLaunchKernelGGL(kv_append_kernel, dim3((total + 255) / 256, n), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_kv_install(const uint16_t* src, int Hkv, int n, int D,
                             uint16_t* dst, long long head_stride,
                             hipStream_t s) {
  const long long total = (long long)Hkv * n * (D / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_install_kernel, dim3((unsigned)((total + 255) / 256)),
                     dim3(256), 0, s, src, Hkv, n, D, dst, head_stride);
  return hipGetLastError();
}

}  // namespace dg
