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

// ---------------------------------------------------------------------------
// Block-wide radix select of the k largest keys (ties to the lower index),
// written out in ascending index order. Used by the VS top-k (keys in global
// memory) and the Block-Sparse row top-k (keys in LDS).
//   KeyFn(i) -> uint32 sortable key of element i, i in [0, n).
//   0 < k < n is assumed; callers handle k == 0 and k >= n themselves.
// NT threads (a multiple of 64, at most 1024). `hist` is LDS of 2048 ints,
// `scratch` LDS of at least 2 * (NT / 64) + 8 ints.
// ---------------------------------------------------------------------------
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

template <int NT, class KeyFn, class OutFn>
__device__ void radix_topk_ordered(KeyFn key_of, int n, int k, int* hist, int* scratch, OutFn out) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int krem = k;
  const int shifts[3] = {21, 10, 0};
  const int widths[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const int nbins = 1 << widths[pass];
    for (int i = tid; i < nbins; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      uint32_t u = key_of(i);
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & (nbins - 1)], 1);
    }
    __syncthreads();
    // wave 0 finds the digit holding the krem-th largest key (searching from the top bin)
    if (tid < 64) {
      const int per = nbins / 64;  // 32 or 16 bins per lane, lane 0 owns the top bins
      const int hi = nbins - per * tid;  // bins [hi - per, hi)
      int s = 0;
      for (int b = hi - 1; b >= hi - per; --b) s += hist[b];
      // inclusive scan over lanes (lane 0 = top chunk)
      int incl = s;
      for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off);
        if (tid >= off) incl += o;
      }
      int excl = incl - s;
      if (excl < krem && krem <= incl) {
        int cum = excl;
        for (int b = hi - 1; b >= hi - per; --b) {
          int h = hist[b];
          if (cum + h >= krem) {
            scratch[0] = b;
            scratch[1] = krem - cum;
            break;
          }
          cum += h;
        }
      }
    }
    __syncthreads();
    const int digit = scratch[0];
    krem = scratch[1];
    prefix |= (uint32_t)digit << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
    __syncthreads();
  }
  // prefix is now the exact key of the k-th largest element; krem of the keys
  // equal to it are taken, lowest indices first.
  const uint32_t thr = prefix;
  const int need_eq = krem;
  int eq_seen = 0, written = 0;
  int* wsum = scratch + 4;
  for (int base = 0; base < n && written < k; base += NT) {
    const int i = base + tid;
    uint32_t u = (i < n) ? key_of(i) : 0u;
    bool gt = (i < n) && (u > thr);
    bool eq = (i < n) && (u == thr);
    int eq_tot;
    int eq_rank = block_excl_scan_count<NT>(eq, wsum, eq_tot);
    bool sel = gt || (eq && (eq_seen + eq_rank < need_eq));
    int sel_tot;
    int pos = block_excl_scan_count<NT>(sel, wsum, sel_tot);
    if (sel) out(written + pos, i);
    eq_seen += eq_tot;
    written += sel_tot;
  }
}

}  // namespace minf
