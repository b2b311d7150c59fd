// Shared device-side definitions for the gfx950 kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace minf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;   // token block of the sparse layout (64x64 blocks, 1x64 verticals)
constexpr int kHeadDim = 128;

// 32x32x16 bf16 MFMA with fp32 accumulation (CDNA4). Operand lane layout:
// lane l holds row/column (l & 31) and the 8 consecutive k values
// 8*(l >> 5) .. 8*(l >> 5) + 7 of the 16-wide k step. Any permutation of k
// applied identically to A and B leaves the product unchanged.
// Accumulator: lane l holds column (l & 31), rows 8*(i/4) + 4*(l >> 5) + (i & 3).
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct HBM -> LDS copies go through buffer loads (buffer_load_dwordx4 ...
// lds) over a descriptor spanning one head's K (or V): 32-bit offsets, and
// the compiler's wait-count tracking stays exact for LDS operand reads issued
// while copies are in flight (with the global form it waits for every one).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRawBufferFlags = 0x00020000;  // descriptor word 3 of a raw (unformatted) buffer
__device__ __forceinline__ rsrc_t buffer_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferFlags);
}
// 16 bytes per lane at byte voff + soff of the buffer into LDS at dst + 16 * lane
__device__ __forceinline__ void copy16(rsrc_t r, void* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, voff, soff, 0, 0);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even fp32 -> bf16 of two values packed into one word (low = a);
// one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// acc + (low bf16 of w) + (high bf16 of w), as one v_dot2_f32_bf16 against (1, 1).
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, acc, false);
}

// Value of lane l ^ 32 combined with lane l's own: v_permlane32_swap on (x, x)
// leaves lanes 0-31 of one result and lanes 32-63 of the other holding the
// partner half, so max / sum of the two results is the pair reduction.
__device__ __forceinline__ float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                            false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                            false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key); -0 is folded into +0.
__device__ __forceinline__ uint32_t sortable_key(float x) {
  x = x + 0.0f;
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__host__ __device__ __forceinline__ int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  return (a % b != 0 && ((a < 0) != (b < 0))) ? q - 1 : q;
}

// Exclusive count of set flags over the NT threads of a block, in thread
// order; `wsum`: NT / 64 ints of LDS; `total` gets the block's count.
template <int NT>
__device__ __forceinline__ int block_excl_scan_count(bool flag, int* wsum, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  constexpr int NW = NT / 64;
  uint64_t bal = __ballot(flag);
  int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(bal);
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    int c = wsum[w];
    before += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + in_wave;
}

// ---------------------------------------------------------------------------
// Block-wide exact top-k of register-held keys. Element c = NT * i + tid of
// the block's candidate list is key[i] of thread tid: 0 marks a non-candidate,
// candidates carry keys >= 1. Only i with NT * i < n are looked at. Writes
// the ids of the min(k, candidates) largest keys, ties to the lower id, in
// ascending order through out(pos, c), and returns their number.
//  * the k-th largest key t is built bit by bit from the top: t | bit is kept
//    while at least k keys are >= it, counted with wave ballots and one
//    cross-wave sum per bit; a count of exactly k ends the search early;
//  * the selected set (every key > t, then the lowest-id keys == t until k
//    are taken) is formed as 64-bit ballot words of consecutive ids and
//    written in ascending order through a popcount scan.
// No atomics, so skewed key distributions cost nothing extra.
// LDS: gmask and emask of NT / 64 * PER words each, red of 2 * NT / 64 ints,
// wsum of NT / 64 ints. Every thread of the block must call it.
// ---------------------------------------------------------------------------
template <int NT>
__device__ __forceinline__ int block_sum_waves(int v, int* red, int& half) {
  // v is uniform within each wave; `red` alternates halves, so one barrier per call suffices
  constexpr int NW = NT / 64;
  if ((threadIdx.x & 63) == 0) red[NW * half + (threadIdx.x >> 6)] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) s += red[NW * half + w];
  half ^= 1;
  return s;
}

template <int NT>
__device__ __forceinline__ int block_excl_scan_int(int v, int* wsum, int& total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = wsum[w];
    before += w < wave ? c : 0;
    tot += c;
  }
  total = tot;
  __syncthreads();
  return before + incl - v;
}

// First stage of the exact register top-k: the number of keys kept,
// min(k, number of keys > 0), and the selection rule: every key > thr, then
// `need` more among the keys == thr (need = 0 when exactly the kept keys are
// > thr). Key i of thread t is candidate NT * i + t; keys of 0 are not
// candidates; only slots NT * i < n are read.
template <int NT, int PER>
__device__ int reg_topk_threshold(const uint32_t (&key)[PER], int n, int k, int* red, uint32_t& thr, int& need) {
  int half = 0;
  int c = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (NT * i < n) c += (int)__popcll(__ballot(key[i] > 0u));
  const int ncand = block_sum_waves<NT>(c, red, half);
  const int keep = ncand < k ? ncand : k;
  thr = 0u;
  need = 0;
  if (keep < ncand) {
    uint32_t t = 0u;
    bool exact = false;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      c = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (NT * i < n) c += (int)__popcll(__ballot(key[i] >= cand));
      c = block_sum_waves<NT>(c, red, half);
      if (c >= k) {
        t = cand;
        if (c == k) {
          exact = true;
          break;
        }
      }
    }
    if (exact) {
      thr = t - 1u;  // exactly k keys are >= t
    } else {
      c = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (NT * i < n) c += (int)__popcll(__ballot(key[i] > t));
      thr = t;
      need = k - block_sum_waves<NT>(c, red, half);
    }
  }
  return keep;
}

template <int NT, int PER, class OutFn>
__device__ int reg_topk_ordered(const uint32_t (&key)[PER], int n, int k, uint64_t* gmask, uint64_t* emask,
                                int* red, int* wsum, OutFn out) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t thr;
  int need;
  const int keep = reg_topk_threshold<NT, PER>(key, n, k, red, thr, need);
  // word NW * i + wave holds ids NT * i + 64 * wave .. + 63, bit = lane
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint64_t g = __ballot(key[i] > thr);
    const uint64_t e = __ballot(need > 0 && key[i] == thr);
    if (lane == 0) {
      gmask[NW * i + wave] = g;
      emask[NW * i + wave] = e;
    }
  }
  __syncthreads();
  uint64_t sel = 0ull, eq = 0ull;
  if (tid < NW * PER) {
    sel = gmask[tid];
    eq = emask[tid];
  }
  int tot;
  if (need > 0) {
    int m = need - block_excl_scan_int<NT>((int)__popcll(eq), wsum, tot);  // equal keys this word may take
    while (m > 0 && eq != 0ull) {
      const uint64_t low = eq & (~eq + 1ull);
      sel |= low;
      eq ^= low;
      --m;
    }
  }
  int pos = block_excl_scan_int<NT>((int)__popcll(sel), wsum, tot);
  while (sel != 0ull) {
    out(pos++, 64 * tid + __builtin_ctzll(sel));
    sel &= sel - 1ull;
  }
  return keep;
}

}  // namespace minf
