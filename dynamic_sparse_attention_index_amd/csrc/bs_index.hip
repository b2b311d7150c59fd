// Block-Sparse online index for gfx950.
//
// What is computed (MInference 1.0 article, "Method": mean pooling of Q and K
// over 64-token blocks and the commutativity of mean pooling with the matrix
// product estimate the block-sparse index): pooled block means, the pooled
// block score Qbar[b] . Kbar[c] for c <= b, and the top-k key blocks of every
// query block, ties to the lower block id, listed in ascending order.
//
// Layout of the work:
//  * pooling: one workgroup per (head, 64-row block); 16 threads span a row
//    with 16-byte loads, fp32 sums in a fixed order. K is pooled once per KV
//    head; both go to [d][n_b] layouts, which the score pass reads coalesced.
//  * scores: 128 x 128 tiles of the lower triangle (query blocks x key blocks)
//    on the fp32 matrix cores (the pooled product is a dense contraction), Q
//    and K pooled into [d][n_b] layouts so that the operands are coalesced;
//    each score is a fixed-order fp32 dot product, written to a score buffer
//    that holds a bounded band of rows at a time;
//  * top-k: one workgroup per (head, query block); the row's scores are held
//    in registers (up to 64 per thread) for an exact bitwise search.
//
// On a permuted sequence (a video in patch-major order: talk transcript,
// MMInference part, on permuting rows and columns so that grid attention
// becomes blocks) key block c is eligible for query block b when c's earliest
// original position is not after b's latest. The rows and columns are then
// taken in rank order (query blocks by latest position, key blocks by earliest
// position), where each row's eligible key blocks are its first columns: the
// score pass is a staircase like the causal triangle, and the selection is
// mapped back to block ids.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kMaxPoolHeads = 64;

struct PoolLaunch {
  const uint16_t* x;
  float* out_rm;  // [nh][nb][128] or null
  float* out_t;   // [nh][128][nb] or null
  const int32_t* col_map;  // block b goes to column col_map[b] (null: column b)
  int32_t n, nb, nh, b0;
  int32_t heads[kMaxPoolHeads];
  int32_t slots[kMaxPoolHeads];
};

__global__ __launch_bounds__(256) void block_pool_kernel(const PoolLaunch a) {
  __shared__ float part[16][kHeadDim];
  const int tid = threadIdx.x;
  const int b = blockIdx.x + a.b0;
  const int h = a.heads[blockIdx.y];
  const int slot = a.slots[blockIdx.y];
  const int64_t r0 = (int64_t)b * kBlock;
  const int cnt = (int)((a.n - r0) < kBlock ? (a.n - r0) : kBlock);
  const int dc = tid & 15;
  const int rg = tid >> 4;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  const uint16_t* xh = a.x + (size_t)h * a.n * kHeadDim;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = rg + 16 * i;
    if (rr < cnt) {
      const u32x4 w = *(const u32x4*)(xh + (size_t)(r0 + rr) * kHeadDim + 8 * dc);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t word = w[e >> 1];
        acc[e] += bf16_to_f32((uint16_t)((e & 1) ? (word >> 16) : (word & 0xffffu)));
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][8 * dc + e] = acc[e];
  __syncthreads();
  if (tid < kHeadDim) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) s += part[q][tid];
    const float mean = s / (float)cnt;
    const int col = a.col_map ? a.col_map[b] : b;
    if (a.out_rm) a.out_rm[((size_t)slot * a.nb + col) * kHeadDim + tid] = mean;
    if (a.out_t) a.out_t[((size_t)slot * kHeadDim + tid) * a.nb + col] = mean;
  }
}

struct BsTopkLaunch {
  const float* qbar_t;  // [nh][128][nb]
  const float* kbar_t;  // [nkv][128][nb]
  float* scores;        // [nh][rows][nb]: rows r0 .. r0 + rows - 1 of this round
  int32_t* blk_idx;     // [nh][nb][k_b]
  int32_t* blk_cnt;     // [nh][nb]
  // permuted sequences (null: causal, row b's candidates are the key blocks c <= b): rows
  // are query blocks by latest original position and columns key blocks by earliest one
  const int32_t* lrow;   // [nb] candidates of row r: columns 0 .. lrow[r] - 1 (the eligible key blocks)
  const int32_t* sigma;  // [nb] key block of column s
  const int32_t* tau;    // [nb] query block of row r
  int32_t nb, k_b, nh, r0, rows;
  int32_t kvslot[kMaxPoolHeads];
  int32_t outslot[kMaxPoolHeads];
};

static_assert(kMaxTokens / kBlock <= 256 * 64, "the top-k holds at most 64 candidates per thread");
constexpr int kTile = 128;  // query blocks x key blocks per score workgroup
constexpr int kSteps = 8;   // contraction steps per register batch (2 x 32 loads in flight)
constexpr int kBufDword3 = 0x00020000;  // buffer resource word 3 on gfx9 (32-bit data format)
constexpr int kStagePitch = 68;  // floats per staged score row (64 + 4 against bank conflicts)

// Stored position of column c of a permuted score row, and its inverse: each
// whole group of 256 columns is rotated by 4 x its group index (a last, partial
// group stays in place, so no position reaches n_b). In earliest-position
// order the key blocks of one video patch are 256 columns apart; the top-k
// reads register i of thread t from position 256 i + t, so the rotation puts
// them in different threads (and keeps 4-aligned runs of 4 columns together).
__device__ __forceinline__ int score_pos(int c, int nb) {
  return (c | 255) < nb ? (c & ~255) + ((c + 4 * (c >> 8)) & 255) : c;
}
__device__ __forceinline__ int score_col(int p, int nb) {
  return (p | 255) < nb ? (p & ~255) + ((p - 4 * (p >> 8)) & 255) : p;
}

// Pooled scores of one 128 x 128 tile (query blocks x key blocks) on the fp32
// matrix cores. Wave w computes the 64 x 64 sub-tile at query blocks
// 64 (w >> 1) and key blocks 64 (w & 1) of the tile as 2 x 2 products of
// v_mfma_f32_32x32x2_f32. Step s of the contraction takes dimension
// 2s + (lane >> 5): lane l supplies Qbar[row l & 31][2s + (l >> 5)] and
// Kbar[column l & 31][2s + (l >> 5)], read from the [d][n_b] layouts (128
// consecutive bytes per half-wave). Each score is an fp32 sum of the 128
// products in a fixed order, so repeated calls agree bitwise.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void block_score_kernel(
    const BsTopkLaunch a) {
  const int ct = blockIdx.x;
  const int bt = a.r0 / kTile + (int)blockIdx.z;
  const bool causal = a.lrow == nullptr;
  const int nb = a.nb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rb = bt * kTile + 64 * (w >> 1);  // first row (query block or rank) of the wave
  const int cb = ct * kTile + 64 * (w & 1);   // first column (key block or rank) of the wave
  const int row_end = min(nb, a.r0 + a.rows);
  if (rb >= row_end || cb >= nb) return;
  // past the last candidate of the wave's last row: above the block diagonal, or
  // past the eligible key blocks (permuted; lrow is non-decreasing over the rows)
  if (causal ? cb > rb + 63 : cb >= a.lrow[min(rb + 63, row_end - 1)]) return;
  const int hs = blockIdx.y;
  const int half = lane >> 5, col = lane & 31;
  __shared__ __attribute__((aligned(16))) float score_stage[4][32 * kStagePitch];
  // the head's pooled rows as buffer resources (2 n_b * 4 * 64 bytes <= 8 MiB):
  // per-lane 32-bit byte offsets of row `half`, column = the lane's block (rows
  // and columns past n_b read the last block; their scores are not stored), and
  // a uniform offset per contraction step
  const uint32_t bytes = (uint32_t)kHeadDim * nb * 4u;
  const __amdgpu_buffer_rsrc_t qr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.qbar_t + (size_t)hs * kHeadDim * nb), 0, bytes, kBufDword3);
  const __amdgpu_buffer_rsrc_t kr =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.kbar_t + (size_t)a.kvslot[hs] * kHeadDim * nb), 0, bytes,
                                        kBufDword3);
  const int qo[2] = {(half * nb + min(rb + col, nb - 1)) * 4, (half * nb + min(rb + 32 + col, nb - 1)) * 4};
  const int ko[2] = {(half * nb + min(cb + col, nb - 1)) * 4, (half * nb + min(cb + 32 + col, nb - 1)) * 4};
  const int c4 = cb + 4 * (lane & 15);  // first of the 4 columns this lane stores
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  // two register batches in ping-pong: batch B loads while A is multiplied, then
  // A reloads while B is multiplied (no register copies, so no early waits)
  float aq[2][kSteps], ak[2][kSteps], bq[2][kSteps], bk[2][kSteps];
  auto load = [&](int s0, float (&lq)[2][kSteps], float (&lk)[2][kSteps]) {
#pragma unroll
    for (int e = 0; e < kSteps; ++e) {
      const int so = 2 * (s0 + e) * nb * 4;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        lq[i][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(qr, qo[i], so, 0));
        lk[i][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kr, ko[i], so, 0));
      }
    }
  };
  auto mul = [&](const float (&lq)[2][kSteps], const float (&lk)[2][kSteps]) {
#pragma unroll
    for (int e = 0; e < kSteps; ++e)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(lq[i][e], lk[j][e], acc[i][j], 0, 0, 0);
  };
  // the last round is peeled so that the loop has no branch (the wait counts
  // then only cover the batch about to be multiplied); scheduling barriers keep
  // each batch's loads issued before the other batch's products
  constexpr int kLast = kHeadDim / 2 - 2 * kSteps;
  static_assert(kLast % (2 * kSteps) == 0 && kLast > 0, "whole ping-pong rounds");
  load(0, aq, ak);
#pragma unroll 1
  for (int s0 = 0; s0 < kLast; s0 += 2 * kSteps) {
    load(s0 + kSteps, bq, bk);
    __builtin_amdgcn_sched_barrier(0);
    mul(aq, ak);
    __builtin_amdgcn_sched_barrier(0);
    load(s0 + 2 * kSteps, aq, ak);
    __builtin_amdgcn_sched_barrier(0);
    mul(bq, bk);
    __builtin_amdgcn_sched_barrier(0);
  }
  load(kLast + kSteps, bq, bk);
  __builtin_amdgcn_sched_barrier(0);
  mul(aq, ak);
  mul(bq, bk);
  // accumulator v of lane l holds row 32 i + (v & 3) + 8 (v >> 2) + 4 (l >> 5)
  // and column 32 j + (l & 31) of the sub-tile. The stores go through LDS,
  // 32 rows at a time, so that each lane writes 4 consecutive scores of a row
  // (a store instruction covers 256 contiguous bytes of 4 rows); only a row's
  // candidates are stored.
  float* t = score_stage[w];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v)
#pragma unroll
      for (int j = 0; j < 2; ++j) t[((v & 3) + 8 * (v >> 2) + 4 * half) * kStagePitch + 32 * j + col] = acc[i][j][v];
    __builtin_amdgcn_wave_barrier();  // LDS accesses of a wave complete in order
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rr = (lane >> 4) + 4 * k;  // row within this half of the sub-tile
      const int b = rb + 32 * i + rr;
      if (b >= row_end) continue;
      const float4 x = *(const float4*)&t[rr * kStagePitch + 4 * (lane & 15)];
      const int clim = causal ? b : a.lrow[b] - 1;  // last column stored
      const int p4 = causal ? c4 : score_pos(c4, nb);  // where the 4 columns are stored
      float* row = a.scores + ((size_t)hs * a.rows + (b - a.r0)) * nb;
      if (c4 + 3 <= clim && (nb & 3) == 0) {  // 16-byte aligned when rows are whole float4s
        *(float4*)(row + p4) = x;
      } else {
        const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c4 + e <= clim) row[p4 + e] = xs[e];
      }
    }
    __builtin_amdgcn_wave_barrier();  // the next half overwrites the staging rows
  }
}

constexpr int kTopkCap = 1024;  // compacted candidates of the pre-filtered top-k

// Permuted rows: the top kb keys by the rule of reg_topk_threshold (keys > thr,
// then `need` of the keys == thr), where key i of this thread is column rank(i)
// and column s is key block sigma[s]. The keys at the threshold are taken in
// ascending block id, and the selected blocks are written in ascending id:
// both through a bitmap over block ids in LDS (one 64-bit word per thread).
template <int PERQ, class RankFn>
__device__ int topk_by_block_id(const uint32_t (&key)[PERQ], int n, int kb, RankFn rank, const int32_t* sigma,
                                int nb, uint64_t* gid, uint64_t* eid, int* red, int* wsum, int32_t* out) {
  const int tid = threadIdx.x;
  const int nwords = (nb + 63) >> 6;  // <= 256
  uint32_t thr;
  int need;
  const int keep = reg_topk_threshold<256, PERQ>(key, n, kb, red, thr, need);
  if (tid < nwords) {
    gid[tid] = 0ull;
    eid[tid] = 0ull;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PERQ; ++i) {
    const uint32_t x = key[i];
    if (256 * i < n && x > 0u && (x > thr || (need > 0 && x == thr))) {
      const int id = sigma[rank(i)];
      atomicOr((unsigned long long*)((x > thr ? gid : eid) + (id >> 6)), 1ull << (id & 63));
    }
  }
  __syncthreads();
  uint64_t sel = tid < nwords ? gid[tid] : 0ull;
  uint64_t eq = tid < nwords ? eid[tid] : 0ull;
  int tot;
  if (need > 0) {
    int m = need - block_excl_scan_int<256>((int)__popcll(eq), wsum, tot);  // equal keys this word may take
    while (m > 0 && eq != 0ull) {
      const uint64_t low = eq & (~eq + 1ull);
      sel |= low;
      eq ^= low;
      --m;
    }
  }
  int pos = block_excl_scan_int<256>((int)__popcll(sel), wsum, tot);
  while (sel != 0ull) {
    out[pos++] = 64 * tid + __builtin_ctzll(sel);
    sel &= sel - 1ull;
  }
  return keep;
}

// Top-k_b key blocks of every query block of the round, from the stored scores.
// Row r of the round is query block r (causal: candidates are the key blocks
// c <= r) or the query block tau[r] (permuted: candidates are the columns
// 0 .. lrow[r] - 1, the eligible key blocks in earliest-position order). One
// workgroup per row; the candidates are held as sortable keys k[i] in
// registers for the exact register top-k (ties to the lower block id).
// Long rows (PER >= 16, k_b <= 256) are first narrowed: each wave takes the
// ceil(k_b / 4)-th largest of its 64 threads' maxima (a wave-only bitwise
// search), and the smallest of the four, t0, has at least k_b keys >= it
// (each wave has ceil(k_b / 4) threads whose maximum is >= t0). The keys
// >= t0 (typically ~2 k_b) are compacted into LDS in column order and the
// register top-k runs over them; when they exceed kTopkCap the whole row is
// searched.
template <int PER, bool PERM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5))) void block_topk_kernel(const BsTopkLaunch a) {
  __shared__ uint64_t gmask[4 * PER];
  __shared__ uint64_t emask[4 * PER];
  __shared__ int red[8];
  __shared__ int wsum[4];
  __shared__ uint32_t ckey[PER >= 16 ? kTopkCap : 1];
  __shared__ int32_t cid[PER >= 16 ? kTopkCap : 1];
  __shared__ int coff[PER >= 16 ? 4 * PER : 1];
  // (gmask / emask double as the id bitmaps of a permuted row: 4 PER words hold
  // 256 PER >= n_b ids)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r_end = a.r0 + a.rows < a.nb ? a.r0 + a.rows : a.nb;
  const int r = r_end - 1 - (int)blockIdx.x;  // longest rows first
  const int b = PERM ? a.tau[r] : r;          // the query block of the row
  const int hs = blockIdx.y;
  const int slot = a.outslot[hs];
  const int kb = a.k_b;
  const int ncand = PERM ? a.lrow[r] : r + 1;
  const float* row = a.scores + ((size_t)hs * a.rows + (r - a.r0)) * a.nb;
  // all loads first, then the keys: the loads are unconditional (no branch for
  // the compiler to sink the key arithmetic into, which would wait for every
  // load in turn); a slot past the row's candidates reads a valid address near
  // the row's start, whose value the key step discards
  // (the row is uniform: 32-bit byte offsets from it, n_b * 4 < 2^32)
  // Register i of thread tid holds position 256 i + tid of the row: column
  // 256 i + tid (causal) or score_col of it (permuted: the stored rotation
  // spreads the key blocks of one video patch over the threads, so that the
  // narrowing below stays tight). A position becomes its column where it is
  // used; the empty asm keeps the compiler from holding all 64 columns live
  // between the key step and the selection.
  auto col_at = [&](int p) {
    if (!PERM) return p;
    asm volatile("" : "+v"(p));
    return score_col(p, a.nb);
  };
  float sv[PER];
  const char* rowb = (const char*)row;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = 256 * i + tid < a.nb ? 256 * i + tid : a.nb - 1;
    const uint32_t off = (uint32_t)(256 * i < ncand ? c : (tid < a.nb ? tid : a.nb - 1)) * 4u;
    sv[i] = *(const float*)(rowb + off);
  }
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t u = sortable_key(sv[i]);
    key[i] = col_at(256 * i + tid) < ncand ? (u > 0u ? u : 1u) : 0u;  // a candidate's key is never 0
  }
  int32_t* out = a.blk_idx + ((size_t)slot * a.nb + b) * kb;
  int keep = -1;
  if constexpr (PER >= 16) {
    if (kb <= 256 && ncand > kTopkCap) {
      // t0: the smallest of the waves' ceil(kb / 4)-th largest thread maxima
      uint32_t tm = 0u;
#pragma unroll
      for (int i = 0; i < PER; ++i) tm = key[i] > tm ? key[i] : tm;
      const int kq = (kb + 3) >> 2;
      uint32_t tw = 0u;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = tw | (1u << bit);
        if ((int)__popcll(__ballot(tm >= cand)) >= kq) tw = cand;
      }
      if (lane == 0) red[wave] = (int)tw;
      __syncthreads();
      uint32_t t0 = (uint32_t)red[0];
#pragma unroll
      for (int w = 1; w < 4; ++w) t0 = (uint32_t)red[w] < t0 ? (uint32_t)red[w] : t0;
      if (t0 == 0u) t0 = 1u;  // never a non-candidate
      // per (i, wave) counts of keys >= t0, then their offsets in column order
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int cnt = (int)__popcll(__ballot(key[i] >= t0));
        if (lane == 0) coff[4 * i + wave] = cnt;
      }
      __syncthreads();
      int tot;
      const int myoff = block_excl_scan_int<256>(tid < 4 * PER ? coff[tid] : 0, wsum, tot);
      if (tot <= kTopkCap) {
        if (tid < 4 * PER) coff[tid] = myoff;
        __syncthreads();
        const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const uint64_t bal = __ballot(key[i] >= t0);
          if (key[i] >= t0) {
            const int pos = coff[4 * i + wave] + (int)__popcll(bal & lt);
            ckey[pos] = key[i];
            cid[pos] = 256 * i + tid;
          }
        }
        __syncthreads();
        uint32_t k2[kTopkCap / 256];
#pragma unroll
        for (int j = 0; j < kTopkCap / 256; ++j) k2[j] = 256 * j + tid < tot ? ckey[256 * j + tid] : 0u;
        if constexpr (PERM)
          keep = topk_by_block_id<kTopkCap / 256>(k2, tot, kb, [&](int j) { return col_at(cid[256 * j + tid]); },
                                                   a.sigma, a.nb, gmask, emask, red, wsum, out);
        else
          keep = reg_topk_ordered<256, kTopkCap / 256>(k2, tot, kb, gmask, emask, red, wsum,
                                                       [&](int pos, int x) { out[pos] = cid[x]; });
      }
      __syncthreads();  // red / wsum / coff are reused below
    }
  }
  if (keep < 0) {
    if constexpr (PERM)
      keep = topk_by_block_id<PER>(key, ncand, kb, [&](int i) { return col_at(256 * i + tid); }, a.sigma, a.nb,
                                   gmask, emask, red, wsum, out);
    else
      keep = reg_topk_ordered<256, PER>(key, ncand, kb, gmask, emask, red, wsum,
                                        [&](int pos, int c) { out[pos] = c; });
  }
  for (int e = keep + tid; e < kb; e += 256) out[e] = -1;
  if (tid == 0) a.blk_cnt[(size_t)slot * a.nb + b] = keep;
}

__global__ __launch_bounds__(64) void block_minmax_kernel(const int32_t* pos, int n, int32_t* bmin, int32_t* bmax) {
  const int c = blockIdx.x;
  const int j = c * kBlock + threadIdx.x;
  int lo = 0x7fffffff, hi = -1;
  if (j < n) lo = hi = pos[j];
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off));
    hi = max(hi, __shfl_xor(hi, off));
  }
  if (threadIdx.x == 0) {
    bmin[c] = lo;
    bmax[c] = hi;
  }
}

// Orders of the blocks of a permuted sequence. The positions are distinct, so
// the blocks' earliest positions are distinct, and so are their latest ones:
// a bitmap over [0, n) of the earliest (latest) positions with a prefix count
// per 32-bit word gives each block's rank among the blocks by earliest
// (latest) position, and for a query block b the number of key blocks whose
// earliest position is <= b's latest -- its eligible key blocks, which are the
// first of them in the earliest-position order.
__global__ __launch_bounds__(256) void perm_clear_kernel(const PermRankLaunch a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < a.words) {
    a.bits_min[i] = 0u;
    a.bits_max[i] = 0u;
  }
}

__global__ __launch_bounds__(256) void perm_bits_kernel(const PermRankLaunch a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.nb) return;
  const int x = a.bmin[c], y = a.bmax[c];
  atomicOr(a.bits_min + (x >> 5), 1u << (x & 31));
  atomicOr(a.bits_max + (y >> 5), 1u << (y & 31));
}

// exclusive prefix counts of both bitmaps' set bits per word (one workgroup)
__global__ __launch_bounds__(1024) void perm_scan_kernel(const PermRankLaunch a) {
  __shared__ int wsum[16];
  const int t = threadIdx.x;
  const int per = (a.words + 1023) / 1024;
  const int w0 = t * per;
  const int w1 = min(w0 + per, a.words);
  int cmin = 0, cmax = 0;
  for (int w = w0; w < w1; ++w) {
    cmin += __popc(a.bits_min[w]);
    cmax += __popc(a.bits_max[w]);
  }
  int tot;
  int pmin = block_excl_scan_int<1024>(cmin, wsum, tot);
  int pmax = block_excl_scan_int<1024>(cmax, wsum, tot);
  for (int w = w0; w < w1; ++w) {
    a.pre_min[w] = pmin;
    a.pre_max[w] = pmax;
    pmin += __popc(a.bits_min[w]);
    pmax += __popc(a.bits_max[w]);
  }
}

__global__ __launch_bounds__(256) void perm_rank_kernel(const PermRankLaunch a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.nb) return;
  const int x = a.bmin[c], y = a.bmax[c];
  const uint32_t below_x = (1u << (x & 31)) - 1u;
  const uint32_t below_y = (1u << (y & 31)) - 1u;
  const uint32_t upto_y = (y & 31) == 31 ? 0xffffffffu : (2u << (y & 31)) - 1u;
  const int rk = a.pre_min[x >> 5] + __popc(a.bits_min[x >> 5] & below_x);
  const int rq = a.pre_max[y >> 5] + __popc(a.bits_max[y >> 5] & below_y);
  a.rank_k[c] = rk;
  a.sigma[rk] = c;
  a.rank_q[c] = rq;
  a.tau[rq] = c;
  a.lrow[rq] = a.pre_min[y >> 5] + __popc(a.bits_min[y >> 5] & upto_y);
}

// Row permutation of [heads][n] rows of row_bytes bytes (a multiple of 4):
// gather out[h][t] = x[h][src[t]], or scatter out[h][src[t]] = x[h][t].
// W is the access unit (16 bytes when the row size allows, else 4). Each
// thread moves kPermUnits units on a grid stride: the row indices are loaded
// first, then every unit, then the stores, so that several independent
// chains are in flight per thread (n * words < 2^31: 32-bit index arithmetic).
constexpr int kPermUnits = 4;
template <typename W>
__global__ __launch_bounds__(256) void permute_rows_kernel(const W* x, W* out, int n, int words,
                                                           const int32_t* src, int scatter) {
  const int total = n * words;
  const int stride = gridDim.x * 256;
  const int i0 = blockIdx.x * 256 + threadIdx.x;
  const size_t base = (size_t)blockIdx.y * total;
  int t[kPermUnits], w[kPermUnits], sr[kPermUnits];
#pragma unroll
  for (int u = 0; u < kPermUnits; ++u) {
    const int idx = i0 + u * stride;
    t[u] = idx < total ? idx / words : 0;
    w[u] = idx - t[u] * words;
    sr[u] = idx < total ? src[t[u]] : 0;
  }
  W v[kPermUnits];
#pragma unroll
  for (int u = 0; u < kPermUnits; ++u) {
    const int row = scatter ? t[u] : sr[u];
    if (i0 + u * stride < total) v[u] = x[base + (size_t)row * words + w[u]];
  }
#pragma unroll
  for (int u = 0; u < kPermUnits; ++u) {
    const int row = scatter ? sr[u] : t[u];
    if (i0 + u * stride < total) out[base + (size_t)row * words + w[u]] = v[u];
  }
}

}  // namespace

hipError_t launch_block_pool(const uint16_t* x, int n, const int32_t* heads, const int32_t* slots, int n_heads,
                             float* out_rm, float* out_t, hipStream_t stream, int first_block,
                             const int32_t* col_map) {
  const int nb = (n + kBlock - 1) / kBlock;
  if (first_block < 0 || first_block >= nb) return hipSuccess;
  for (int base = 0; base < n_heads; base += kMaxPoolHeads) {
    const int c = n_heads - base < kMaxPoolHeads ? n_heads - base : kMaxPoolHeads;
    PoolLaunch a{};
    a.x = x;
    a.out_rm = out_rm;
    a.out_t = out_t;
    a.col_map = col_map;
    a.n = n;
    a.nb = nb;
    a.nh = c;
    a.b0 = first_block;
    for (int i = 0; i < c; ++i) {
      a.heads[i] = heads[base + i];
      a.slots[i] = slots[base + i];
    }
    hipLaunchKernelGGL(block_pool_kernel, dim3(nb - first_block, c), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int block_score_rows(int nb, int n_heads) {
  // bound the score buffer to about 512 MiB; whole 64-row tiles
  const long long per_row = (long long)std::max(n_heads, 1) * nb * 4;
  long long r = (512ll << 20) / per_row / kTile * kTile;
  if (r < kTile) r = kTile;
  return (int)std::min<long long>(r, ((long long)nb + kTile - 1) / kTile * kTile);
}

hipError_t launch_block_minmax(const int32_t* pos, int n, int32_t* bmin, int32_t* bmax, hipStream_t stream) {
  const int nb = (n + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(block_minmax_kernel, dim3(nb), dim3(64), 0, stream, pos, n, bmin, bmax);
  return hipGetLastError();
}

hipError_t launch_permute_rows(const void* x, void* out, int heads, int64_t n, int row_bytes, const int32_t* src,
                               int scatter, hipStream_t stream) {
  const bool wide = row_bytes % 16 == 0 && ((uintptr_t)x | (uintptr_t)out) % 16 == 0;
  const int words = wide ? row_bytes / 16 : row_bytes / 4;
  const int64_t total = n * words;
  if (total >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((total + 256 * kPermUnits - 1) / (256 * kPermUnits)), heads);
  if (wide)
    hipLaunchKernelGGL(permute_rows_kernel<u32x4>, grid, dim3(256), 0, stream, (const u32x4*)x, (u32x4*)out, (int)n,
                       words, src, scatter);
  else
    hipLaunchKernelGGL(permute_rows_kernel<uint32_t>, grid, dim3(256), 0, stream, (const uint32_t*)x,
                       (uint32_t*)out, (int)n, words, src, scatter);
  return hipGetLastError();
}

hipError_t launch_perm_ranks(const PermRankLaunch& a, hipStream_t stream) {
  hipLaunchKernelGGL(perm_clear_kernel, dim3((a.words + 255) / 256), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(perm_bits_kernel, dim3((a.nb + 255) / 256), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
  hipLaunchKernelGGL(perm_rank_kernel, dim3((a.nb + 255) / 256), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_block_topk(const float* qbar_t, const float* kbar_t, const int32_t* kvslot, int n_heads, int nb,
                             int k_b, int32_t* blk_idx, int32_t* blk_cnt, float* scores, int rows,
                             const int32_t* lrow, const int32_t* sigma, const int32_t* tau, hipStream_t stream) {
  const int nbt = (nb + kTile - 1) / kTile;
  const bool perm = lrow != nullptr;
  for (int base = 0; base < n_heads; base += kMaxPoolHeads) {
    const int c = n_heads - base < kMaxPoolHeads ? n_heads - base : kMaxPoolHeads;
    BsTopkLaunch a{};
    a.qbar_t = qbar_t + (size_t)base * nb * kHeadDim;
    a.kbar_t = kbar_t;
    a.scores = scores;
    a.blk_idx = blk_idx;
    a.blk_cnt = blk_cnt;
    a.nb = nb;
    a.k_b = k_b;
    a.nh = c;
    a.rows = rows;
    a.lrow = lrow;
    a.sigma = sigma;
    a.tau = tau;
    for (int i = 0; i < c; ++i) {
      a.kvslot[i] = kvslot[base + i];
      a.outslot[i] = base + i;
    }
    for (int r0 = 0; r0 < nb; r0 += rows) {
      a.r0 = r0;
      const int row_tiles = (std::min(nb, r0 + rows) - r0 + kTile - 1) / kTile;
      // permuted: the band's last candidate column is known only on the device,
      // so every column tile is launched and those past it return at once
      const int col_tiles = perm ? nbt : std::min(nbt, (r0 + rows) / kTile);
      hipLaunchKernelGGL(block_score_kernel, dim3(col_tiles, c, row_tiles), dim3(256), 0, stream, a);
      const dim3 tg(std::min(rows, nb - r0), c);
      auto topk = [&](auto kern) { hipLaunchKernelGGL(kern, tg, dim3(256), 0, stream, a); };
      if (nb <= 256)
        perm ? topk(block_topk_kernel<1, true>) : topk(block_topk_kernel<1, false>);
      else if (nb <= 1024)
        perm ? topk(block_topk_kernel<4, true>) : topk(block_topk_kernel<4, false>);
      else if (nb <= 4096)
        perm ? topk(block_topk_kernel<16, true>) : topk(block_topk_kernel<16, false>);
      else
        perm ? topk(block_topk_kernel<64, true>) : topk(block_topk_kernel<64, false>);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace minf
