// Top-k of long score rows on many workgroups (gfx950).
//
// The VS index keeps, per head, the k_v largest column sums and the k_s
// largest diagonal sums of rows up to 2^24 entries long (MInference 1.0
// article, "Method": top-k selection of the estimated verticals and slashes).
// One workgroup per row leaves most of the GPU idle, so every row is split
// into chunks that separate workgroups scan:
//
//  1. three radix passes over the sortable bit pattern (11, 11, 10 bits, high
//     digit first): each chunk builds a histogram of the keys that match the
//     prefix found so far in LDS and adds it to the row's histogram with
//     integer atomics; one small kernel per row then picks the digit holding
//     the k-th largest key and the rank left inside it;
//  2. after the last pass the prefix is the exact k-th largest key T and the
//     rank is the number of keys equal to T that are kept (lowest indices
//     first); each chunk counts its keys > T and == T;
//  3. each wave scans a contiguous quarter of a chunk: it adds up the counts
//     of the quarters before it, keeps its keys > T and its share of the keys
//     == T, and writes their indices in ascending order at its offset
//     (positions from wave ballots, no block-wide synchronisation).
//
// Only integer atomics are used, so the result does not depend on the order
// in which workgroups run.
#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kTopkThreads = 256;
constexpr int kRadixBins = 2048;

struct RowRef {
  const float* src;
  int32_t* dst;
  int k;
};

__device__ __forceinline__ RowRef row_ref(const TopkLaunch& a, int r) {
  const int s = r < a.seg[0].rows ? 0 : 1;
  const int rr = s == 0 ? r : r - a.seg[0].rows;
  const TopkSeg& g = a.seg[s];
  return RowRef{g.src + (size_t)rr * g.src_stride, g.dst + (size_t)rr * g.dst_stride, g.k};
}

__global__ __launch_bounds__(kTopkThreads) void topk_init_kernel(const TopkLaunch a) {
  const int r = blockIdx.x;
  int* h = a.hist + (size_t)r * kRadixBins;
  for (int i = threadIdx.x; i < kRadixBins; i += kTopkThreads) h[i] = 0;
  if (threadIdx.x == 0) {
    int* st = a.state + 4 * r;
    st[0] = 0;                    // prefix of the k-th largest key
    st[1] = 0;                    // mask of the prefix bits fixed so far
    st[2] = row_ref(a, r).k;      // rank still to place inside the prefix
    st[3] = 0;
  }
}

template <int PASS>
__global__ __launch_bounds__(kTopkThreads) void topk_hist_kernel(const TopkLaunch a) {
  constexpr int kShift = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  constexpr int kBins = PASS == 2 ? 1024 : 2048;
  __shared__ int lh[kRadixBins];
  const int r = blockIdx.y;
  const RowRef rf = row_ref(a, r);
  if (rf.k <= 0 || rf.k >= a.n) return;
  const int* st = a.state + 4 * r;
  const uint32_t prefix = (uint32_t)st[0], pmask = (uint32_t)st[1];
  for (int i = threadIdx.x; i < kBins; i += kTopkThreads) lh[i] = 0;
  __syncthreads();
  const int lo = blockIdx.x * a.chunk;
  const int hi = min(a.n, lo + a.chunk);
  // eight loads in flight per thread, then their histogram updates
  for (int base = lo + threadIdx.x; base < hi; base += 8 * kTopkThreads) {
    uint32_t u[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int i = base + x * kTopkThreads;
      u[x] = i < hi ? sortable_key(rf.src[i]) : 0u;  // slots past the chunk are skipped below
    }
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (base + x * kTopkThreads < hi && (u[x] & pmask) == prefix) atomicAdd(&lh[(u[x] >> kShift) & (kBins - 1)], 1);
  }
  __syncthreads();
  int* gh = a.hist + (size_t)r * kRadixBins;
  for (int b = threadIdx.x; b < kBins; b += kTopkThreads)
    if (lh[b]) atomicAdd(&gh[b], lh[b]);
}

// One wave per row: the digit of the k-th largest key in this pass.
template <int PASS>
__global__ __launch_bounds__(64) void topk_select_kernel(const TopkLaunch a) {
  constexpr int kShift = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
  constexpr int kBins = PASS == 2 ? 1024 : 2048;
  constexpr int kPer = kBins / 64;  // bins per lane; lane 0 owns the top ones
  const int r = blockIdx.x;
  const RowRef rf = row_ref(a, r);
  if (rf.k <= 0 || rf.k >= a.n) return;
  int* st = a.state + 4 * r;
  int* gh = a.hist + (size_t)r * kRadixBins;
  const int lane = threadIdx.x;
  const int krem = st[2];
  const int top = kBins - kPer * lane;  // this lane's bins are [top - kPer, top)
  int cnt[kPer];
  int s = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    cnt[j] = gh[top - 1 - j];
    s += cnt[j];
  }
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const int excl = incl - s;
  // every lane has read the histogram before it is cleared for the next pass
  __syncthreads();
  for (int b = lane; b < kRadixBins; b += 64) gh[b] = 0;
  if (excl < krem && krem <= incl) {
    int cum = excl;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (cum + cnt[j] >= krem && cum < krem) {
        st[0] = (int)((uint32_t)st[0] | ((uint32_t)(top - 1 - j) << kShift));
        st[1] = (int)((uint32_t)st[1] | ((uint32_t)(kBins - 1) << kShift));
        st[2] = krem - cum;
      }
      cum += cnt[j];
    }
  }
}

// Each wave scans a contiguous quarter of its chunk: [wlo, whi).
__device__ __forceinline__ void wave_range(const TopkLaunch& a, int& wlo, int& whi) {
  const int lo = blockIdx.x * a.chunk;
  const int hi = min(a.n, lo + a.chunk);
  const int sub = a.chunk / (kTopkThreads / 64);
  wlo = min(hi, lo + (int)(threadIdx.x >> 6) * sub);
  whi = min(hi, wlo + sub);
}

// Keys above and equal to the threshold in each wave's quarter of each chunk.
__global__ __launch_bounds__(kTopkThreads) void topk_count_kernel(const TopkLaunch a) {
  const int r = blockIdx.y;
  const RowRef rf = row_ref(a, r);
  if (rf.k <= 0 || rf.k >= a.n) return;
  const uint32_t thr = (uint32_t)a.state[4 * r];
  const int lane = threadIdx.x & 63;
  int wlo, whi;
  wave_range(a, wlo, whi);
  int gt = 0, eq = 0;
  for (int base = wlo + lane; base < whi; base += 8 * 64) {
    uint32_t u[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int i = base + x * 64;
      u[x] = i < whi ? sortable_key(rf.src[i]) : 0u;  // key 0 (a NaN pattern) is below every real key
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const bool in = base + x * 64 < whi;
      gt += in && u[x] > thr;
      eq += in && u[x] == thr;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  if (lane == 0) {
    constexpr int kW = kTopkThreads / 64;
    const int e = blockIdx.x * kW + (threadIdx.x >> 6);
    int* c = a.cnt + (size_t)r * 2 * kW * a.nchunks;
    c[e] = gt;
    c[kW * a.nchunks + e] = eq;
  }
}

// Ordered write-out: each wave starts after the keys kept by the quarters
// before it (all earlier chunks, then the earlier waves of its chunk) and
// places its own with ballots, 64 keys at a time.
__global__ __launch_bounds__(kTopkThreads) void topk_write_kernel(const TopkLaunch a) {
  const int r = blockIdx.y;
  const RowRef rf = row_ref(a, r);
  if (rf.k <= 0) return;
  const int lane = threadIdx.x & 63;
  int wlo, whi;
  wave_range(a, wlo, whi);
  if (rf.k >= a.n) {  // full budget: every index, in order
    for (int i = wlo + lane; i < whi; i += 64) rf.dst[i] = i;
    return;
  }
  constexpr int kW = kTopkThreads / 64;
  const uint32_t thr = (uint32_t)a.state[4 * r];
  const int need_eq = a.state[4 * r + 2];
  const int e = blockIdx.x * kW + (threadIdx.x >> 6);
  const int* c = a.cnt + (size_t)r * 2 * kW * a.nchunks;
  int gt_before = 0, eq_before = 0;
  for (int j = lane; j < e; j += 64) {
    gt_before += c[j];
    eq_before += c[kW * a.nchunks + j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    gt_before += __shfl_xor(gt_before, off);
    eq_before += __shfl_xor(eq_before, off);
  }
  int written = gt_before + min(eq_before, need_eq);
  int eq_seen = eq_before;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int base = wlo; base < whi; base += 8 * 64) {
    uint32_t u[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int i = base + x * 64 + lane;
      u[x] = i < whi ? sortable_key(rf.src[i]) : 0u;
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int i = base + x * 64 + lane;
      const bool in = i < whi;
      const bool gt = in && u[x] > thr;
      const bool eq = in && u[x] == thr;
      const uint64_t beq = __ballot(eq);
      const bool sel = gt || (eq && eq_seen + (int)__popcll(beq & below) < need_eq);
      const uint64_t bsel = __ballot(sel);
      if (sel) rf.dst[written + (int)__popcll(bsel & below)] = i;
      written += (int)__popcll(bsel);
      eq_seen += (int)__popcll(beq);
    }
  }
}

}  // namespace

int topk_chunk_len(int n) {
  int per = (n + 63) / 64;               // aim for about 64 chunks per row
  per = (per + 1023) / 1024 * 1024;      // whole 1024-element steps
  return per < 1024 ? 1024 : (per > 65536 ? 65536 : per);
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream) {
  const int rows = a.seg[0].rows + a.seg[1].rows;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)a.nchunks, (unsigned)rows);
  hipLaunchKernelGGL(topk_init_kernel, dim3(rows), dim3(kTopkThreads), 0, stream, a);
  hipLaunchKernelGGL(topk_hist_kernel<0>, grid, dim3(kTopkThreads), 0, stream, a);
  hipLaunchKernelGGL(topk_select_kernel<0>, dim3(rows), dim3(64), 0, stream, a);
  hipLaunchKernelGGL(topk_hist_kernel<1>, grid, dim3(kTopkThreads), 0, stream, a);
  hipLaunchKernelGGL(topk_select_kernel<1>, dim3(rows), dim3(64), 0, stream, a);
  hipLaunchKernelGGL(topk_hist_kernel<2>, grid, dim3(kTopkThreads), 0, stream, a);
  hipLaunchKernelGGL(topk_select_kernel<2>, dim3(rows), dim3(64), 0, stream, a);
  hipLaunchKernelGGL(topk_count_kernel, grid, dim3(kTopkThreads), 0, stream, a);
  hipLaunchKernelGGL(topk_write_kernel, grid, dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace minf
