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
//    head, into a [d][n_b] layout so that the score pass reads it coalesced.
//  * scores + top-k: one workgroup per (head, query block); the row's scores
//    live in LDS (up to 16384 blocks = 64 KiB), each a fixed-order fp32 dot
//    product, followed by the shared radix select.
#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kMaxPoolHeads = 64;

struct PoolLaunch {
  const uint16_t* x;
  float* out_rm;  // [nh][nb][128] or null
  float* out_t;   // [nh][128][nb] or null
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
    if (a.out_rm) a.out_rm[((size_t)slot * a.nb + b) * kHeadDim + tid] = mean;
    if (a.out_t) a.out_t[((size_t)slot * kHeadDim + tid) * a.nb + b] = mean;
  }
}

struct BsTopkLaunch {
  const float* qbar;    // [nh][nb][128]
  const float* kbar_t;  // [nkv][128][nb]
  int32_t* blk_idx;     // [nh][nb][k_b]
  int32_t* blk_cnt;     // [nh][nb]
  int32_t nb, k_b, nh;
  int32_t kvslot[kMaxPoolHeads];
  int32_t outslot[kMaxPoolHeads];
};

constexpr int kMaxBlocks = (int)(kMaxTokens / kBlock);

__global__ __launch_bounds__(256) void block_topk_kernel(const BsTopkLaunch a) {
  __shared__ float sc[kMaxBlocks];
  __shared__ float qb[kHeadDim];
  __shared__ int hist[2048];
  __shared__ int scratch[16];
  const int tid = threadIdx.x;
  const int b = a.nb - 1 - (int)blockIdx.x;  // longest rows first
  const int hs = blockIdx.y;
  const int slot = a.outslot[hs];
  const int kb = a.k_b;
  const int keep = (b + 1) < kb ? (b + 1) : kb;
  int32_t* out = a.blk_idx + ((size_t)slot * a.nb + b) * kb;
  if (tid == 0) a.blk_cnt[(size_t)slot * a.nb + b] = keep;
  for (int e = keep + tid; e < kb; e += 256) out[e] = -1;
  if (b + 1 <= kb) {
    for (int c = tid; c <= b; c += 256) out[c] = c;
    return;
  }
  if (tid < kHeadDim) qb[tid] = a.qbar[((size_t)hs * a.nb + b) * kHeadDim + tid];
  __syncthreads();
  const float* kt = a.kbar_t + (size_t)a.kvslot[hs] * kHeadDim * a.nb;
  for (int c = tid; c <= b; c += 256) {
    float acc = 0.f;
    for (int d = 0; d < kHeadDim; ++d) acc = fmaf(qb[d], kt[(size_t)d * a.nb + c], acc);
    sc[c] = acc;
  }
  __syncthreads();
  radix_topk_ordered<256>([&](int i) { return sortable_key(sc[i]); }, b + 1, kb, hist, scratch,
                          [&](int pos, int i) { out[pos] = i; });
}

}  // namespace

hipError_t launch_block_pool(const uint16_t* x, int n, const int32_t* heads, const int32_t* slots, int n_heads,
                             float* out_rm, float* out_t, hipStream_t stream, int first_block) {
  const int nb = (n + kBlock - 1) / kBlock;
  if (first_block < 0 || first_block >= nb) return hipSuccess;
  for (int base = 0; base < n_heads; base += kMaxPoolHeads) {
    const int c = n_heads - base < kMaxPoolHeads ? n_heads - base : kMaxPoolHeads;
    PoolLaunch a{};
    a.x = x;
    a.out_rm = out_rm;
    a.out_t = out_t;
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

hipError_t launch_block_topk(const float* qbar, const float* kbar_t, const int32_t* kvslot, int n_heads, int nb,
                             int k_b, int32_t* blk_idx, int32_t* blk_cnt, hipStream_t stream) {
  for (int base = 0; base < n_heads; base += kMaxPoolHeads) {
    const int c = n_heads - base < kMaxPoolHeads ? n_heads - base : kMaxPoolHeads;
    BsTopkLaunch a{};
    a.qbar = qbar + (size_t)base * nb * kHeadDim;
    a.kbar_t = kbar_t;
    a.blk_idx = blk_idx;
    a.blk_cnt = blk_cnt;
    a.nb = nb;
    a.k_b = k_b;
    a.nh = c;
    for (int i = 0; i < c; ++i) {
      a.kvslot[i] = kvslot[base + i];
      a.outslot[i] = base + i;
    }
    hipLaunchKernelGGL(block_topk_kernel, dim3(nb, c), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace minf
