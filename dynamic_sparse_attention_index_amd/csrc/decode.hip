// Sparse decoding with top-k block loads for gfx950.
//
// What is computed ("KV-cache-centric efficient long-context methods" talk
// transcript: in the decoding stage loading the KV cache is the bottleneck and
// can be done sparsely, and decode attention splits into a top-k selection and
// attention over the selected keys; MInference 1.0 article, "Method": the
// pooled-key block estimate): one new query row per head attends to a cache
// of n keys. Each query head scores every 64-token block c of its KV head by
// q . mean(K_c), keeps the top-k_b blocks (ties to the lower block, ascending)
// and attends exactly over their keys. k_b >= n_b is dense decoding.
//
// Layout of the work (memory bound: the point is to load few K/V rows):
//  * scores: 64 blocks per workgroup, one lane per block and one wave per
//    quarter of the dimensions, the pooled keys stored [d][n_b] so that a
//    wave reads 64 consecutive blocks per dimension; the group's queries sit
//    in LDS and are read by broadcast, so every pooled vector is read once per
//    KV head;
//  * top-k: the exact register top-k (bitwise search, ballot counts); for
//    k_b <= 256 over more than 2048 blocks, 2048-block segments are selected
//    by separate workgroups and a second kernel merges each head's segment
//    winners, else one 1024-thread workgroup per head;
//  * attention: split over the selected blocks (flash-decoding style); a wave
//    takes one 64-key block at a time, 16 lanes per key row with 16-byte
//    loads, online softmax in fp32; the four waves of a workgroup merge their
//    partials in LDS and each split writes (max, sum, o[128]); dense decoding
//    serves up to four heads of a GQA group from each loaded row;
//  * combine: per head, the splits in a fixed order (no float atomics).
#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecMaxGroup = 8;  // query heads per KV head handled by one score workgroup

__device__ __forceinline__ float dot_bf16x2(uint32_t a, uint32_t b, float c) {
  typedef __attribute__((__vector_size__(2 * sizeof(short)))) short s16x2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(s16x2, a), __builtin_bit_cast(s16x2, b), c, false);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// scores[h][c] = sum_d q_h[d] * kbar_t[g][d][c] for the heads of KV head g.
// A workgroup takes 64 blocks; wave w sums d = 32 w .. 32 w + 31 in ascending
// order and the four partials are added in wave order (a fixed order, so the
// scores are reproducible), which gives four times the loads in flight of one
// thread walking all 128 dimensions.
__global__ __launch_bounds__(kDecThreads) void decode_score_kernel(const DecodeLaunch a) {
  __shared__ float qs[kHeadDim][kDecMaxGroup];
  __shared__ float part[3][kDecMaxGroup][64];
  const int g = blockIdx.y;
  const int h0 = g * a.grp;
  for (int x = threadIdx.x; x < kHeadDim * kDecMaxGroup; x += kDecThreads) {
    const int d = x / kDecMaxGroup, t = x % kDecMaxGroup;
    qs[d][t] = t < a.grp ? __builtin_bit_cast(float, (uint32_t)a.q[(size_t)(h0 + t) * kHeadDim + d] << 16) : 0.f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wq = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float acc[kDecMaxGroup];
#pragma unroll
  for (int t = 0; t < kDecMaxGroup; ++t) acc[t] = 0.f;
  if (c < a.nb) {
    const float* kt = a.kbar_t + ((size_t)g * kHeadDim + 32 * wq) * a.nb + c;
#pragma unroll 8
    for (int d = 0; d < 32; ++d) {
      const float kv = kt[(size_t)d * a.nb];
#pragma unroll
      for (int t = 0; t < kDecMaxGroup; ++t) acc[t] = fmaf(qs[32 * wq + d][t], kv, acc[t]);
    }
  }
  if (wq > 0) {
#pragma unroll
    for (int t = 0; t < kDecMaxGroup; ++t) part[wq - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (wq == 0 && c < a.nb)
    for (int t = 0; t < a.grp; ++t)
      a.scores[(size_t)(h0 + t) * a.nb + c] = ((acc[t] + part[0][t][lane]) + part[1][t][lane]) + part[2][t][lane];
}

static_assert(kDecMaxBlocks <= 1024 * 16, "the decode top-k holds at most 16 blocks per thread");

// top-k_b blocks of one head (n_b <= kDecMaxBlocks), ascending: block
// c = 1024 i + tid is key[i] of thread tid, for the exact register top-k
template <int PER>
__global__ __launch_bounds__(1024) void decode_topk_kernel(const DecodeLaunch a) {
  __shared__ uint64_t gmask[16 * PER];
  __shared__ uint64_t emask[16 * PER];
  __shared__ int red[32];
  __shared__ int wsum[16];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const float* s = a.scores + (size_t)h * a.nb;
  float sv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) sv[i] = s[1024 * i + tid < a.nb ? 1024 * i + tid : a.nb - 1];
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t u = sortable_key(sv[i]);
    key[i] = 1024 * i + tid < a.nb ? (u > 0u ? u : 1u) : 0u;
  }
  int32_t* out = a.blk + (size_t)h * a.kb;
  reg_topk_ordered<1024, PER>(key, a.nb, a.kb, gmask, emask, red, wsum, [&](int pos, int c) { out[pos] = c; });
}

// Segmented top-k_b of one head (k_b <= kDecSegMaxK), step 1: workgroup
// (seg, h) selects the top-k_b of blocks [2048 seg, 2048 seg + 2048) with the
// register top-k and stores their keys and ids (ascending ids).
__global__ __launch_bounds__(256) void decode_topk_seg_kernel(const DecodeLaunch a) {
  constexpr int PER = kDecSeg / 256;
  __shared__ uint64_t gmask[4 * PER];
  __shared__ uint64_t emask[4 * PER];
  __shared__ int red[8];
  __shared__ int wsum[4];
  const int seg = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int c0 = seg * kDecSeg;
  const int ns = a.nb - c0 < kDecSeg ? a.nb - c0 : kDecSeg;
  const float* s = a.scores + (size_t)h * a.nb + c0;
  float sv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) sv[i] = s[256 * i + tid < ns ? 256 * i + tid : ns - 1];
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t u = sortable_key(sv[i]);
    key[i] = 256 * i + tid < ns ? (u > 0u ? u : 1u) : 0u;
  }
  const size_t so = ((size_t)h * a.nseg + seg) * a.kb;
  uint32_t* sk = a.seg_key + so;
  int32_t* si = a.seg_id + so;
  const int keep = reg_topk_ordered<256, PER>(key, ns, a.kb, gmask, emask, red, wsum, [&](int pos, int c) {
    const uint32_t u = sortable_key(s[c]);
    sk[pos] = u > 0u ? u : 1u;
    si[pos] = c0 + c;
  });
  if (tid == 0) a.seg_cnt[(size_t)h * a.nseg + seg] = keep;
}

// Step 2, one workgroup per head: the global top-k_b is contained in the union
// of the segments' top-k_b under the same order (key descending, lower id
// first). Candidate x = seg * k_b + slot lists the segments in id order, so the
// lowest candidate index is the lowest id among equal keys.
template <int PER2>
__global__ __launch_bounds__(256) void decode_topk_merge_kernel(const DecodeLaunch a) {
  __shared__ uint64_t gmask[4 * PER2];
  __shared__ uint64_t emask[4 * PER2];
  __shared__ int red[8];
  __shared__ int wsum[4];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int ncand = a.nseg * a.kb;
  const uint32_t* hk = a.seg_key + (size_t)h * a.nseg * a.kb;
  const int32_t* hid = a.seg_id + (size_t)h * a.nseg * a.kb;
  const int32_t* hcnt = a.seg_cnt + (size_t)h * a.nseg;
  uint32_t key2[PER2];
#pragma unroll
  for (int i = 0; i < PER2; ++i) {
    const int x = 256 * i + tid;
    key2[i] = 0u;
    if (x < ncand) {
      const int sg = x / a.kb;
      if (x - sg * a.kb < hcnt[sg]) key2[i] = hk[x];
    }
  }
  int32_t* out = a.blk + (size_t)h * a.kb;
  reg_topk_ordered<256, PER2>(key2, ncand, a.kb, gmask, emask, red, wsum,
                              [&](int pos, int x) { out[pos] = hid[x]; });
}

// G query heads of one KV head per workgroup: G = 1 for sparse decoding (each
// head has its own blocks), G = up to 4 heads of a GQA group for dense
// decoding (they read the same rows, so every K/V row is loaded once for all
// of them). A wave takes one 64-key block at a time, in two halves of 32 keys.
template <int G>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(const DecodeLaunch a) {
  __shared__ float wo[4][G][kHeadDim];
  __shared__ float wm[4][G], wl[4][G];
  const int sp = blockIdx.x;
  const int h0 = blockIdx.y * G;  // first query head of this workgroup
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kr = lane >> 4;  // key row within a group of four
  const int dc = lane & 15;  // 8-dim chunk
  const int g = h0 / a.grp;
  const uint16_t* kh = a.k + (size_t)g * a.n * kHeadDim;
  const uint16_t* vh = a.v + (size_t)g * a.n * kHeadDim;
  u32x4 qw[G];  // this lane's 8 dims of each head's query, bf16 pairs
#pragma unroll
  for (int t = 0; t < G; ++t) qw[t] = *(const u32x4*)(a.q + (size_t)(h0 + t) * kHeadDim + 8 * dc);
  float m[G], l[G], o[G][8];
#pragma unroll
  for (int t = 0; t < G; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[t][e] = 0.f;
  }
  const int e0 = sp * a.bps;
  const int e1 = min(a.kb, e0 + a.bps);
  for (int ent = e0 + wave; ent < e1; ent += 4) {
    const int c = a.blk ? a.blk[(size_t)h0 * a.kb + ent] : ent;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      const int64_t j0 = (int64_t)c * kBlock + 32 * half;
      u32x4 kw[8], vw[8];
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int64_t j = j0 + 4 * it + kr;
        const bool ok = j < a.n;
        kw[it] = ok ? *(const u32x4*)(kh + (size_t)j * kHeadDim + 8 * dc) : u32x4{0, 0, 0, 0};
        vw[it] = ok ? *(const u32x4*)(vh + (size_t)j * kHeadDim + 8 * dc) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int t = 0; t < G; ++t) {
        float s[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          // bf16 x bf16 products are exact in fp32; v_dot2 adds each pair in fp32
          float p = 0.f;
#pragma unroll
          for (int e = 0; e < 4; ++e) p = dot_bf16x2(qw[t][e], kw[it][e], p);
          // the 16 lanes of a key row hold its 8-dim partials: butterfly over them
          p += __shfl_xor(p, 8);
          p += __shfl_xor(p, 4);
          p += __shfl_xor(p, 2);
          p += __shfl_xor(p, 1);
          s[it] = (j0 + 4 * it + kr < a.n) ? p * a.scale_log2 : -INFINITY;
        }
        float mb = s[0];
#pragma unroll
        for (int it = 1; it < 8; ++it) mb = fmaxf(mb, s[it]);
        mb = fmaxf(mb, __shfl_xor(mb, 16));
        mb = fmaxf(mb, __shfl_xor(mb, 32));
        const float m_new = fmaxf(m[t], mb);
        if (m_new == -INFINITY) continue;  // nothing visible yet (rows past n)
        const float alpha = m[t] == -INFINITY ? 0.f : fast_exp2(m[t] - m_new);
        l[t] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[t][e] *= alpha;
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const float p = fast_exp2(s[it] - m_new);
          l[t] += p;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[t][2 * e] = fmaf(p, bf16_lo(vw[it][e]), o[t][2 * e]);
            o[t][2 * e + 1] = fmaf(p, bf16_hi(vw[it][e]), o[t][2 * e + 1]);
          }
        }
        m[t] = m_new;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < G; ++t) {
    // the four key-row groups of the wave hold disjoint keys: add them up
    l[t] += __shfl_xor(l[t], 16);
    l[t] += __shfl_xor(l[t], 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[t][e] += __shfl_xor(o[t][e], 16);
      o[t][e] += __shfl_xor(o[t][e], 32);
    }
    if (kr == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wo[wave][t][8 * dc + e] = o[t][e];
    }
    if (lane == 0) {
      wm[wave][t] = m[t];
      wl[wave][t] = l[t];
    }
  }
  __syncthreads();
  for (int x = threadIdx.x; x < G * kHeadDim; x += kDecThreads) {
    const int t = x / kHeadDim, d = x % kHeadDim;
    const float mm = fmaxf(fmaxf(wm[0][t], wm[1][t]), fmaxf(wm[2][t], wm[3][t]));
    float ls = 0.f, os = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = wm[w][t] == -INFINITY ? 0.f : fast_exp2(wm[w][t] - mm);
        ls += wl[w][t] * f;
        os += wo[w][t][d] * f;
      }
    }
    float* pp = a.part + ((size_t)(h0 + t) * a.nsplit + sp) * (kHeadDim + 2);
    pp[2 + d] = os;
    if (d == 0) {
      pp[0] = mm;
      pp[1] = ls;
    }
  }
}

// Per head: merge the splits. Thread (r, d) takes splits s = r, r + 8, ... for
// dimension d; the eight partial sums are then added in r order.
constexpr int kCombRows = 8;
__global__ __launch_bounds__(kCombRows * kHeadDim) void decode_combine_kernel(const DecodeLaunch a) {
  __shared__ float red_m[kCombRows * kHeadDim];
  __shared__ float part_l[kCombRows], part_o[kCombRows][kHeadDim];
  const int h = blockIdx.x;
  const int d = threadIdx.x % kHeadDim;
  const int r = threadIdx.x / kHeadDim;
  const int stride = kHeadDim + 2;
  const float* pp = a.part + (size_t)h * a.nsplit * stride;
  float mm = -INFINITY;
  for (int s = threadIdx.x; s < a.nsplit; s += kCombRows * kHeadDim) mm = fmaxf(mm, pp[(size_t)s * stride]);
  red_m[threadIdx.x] = mm;
  __syncthreads();
  for (int off = kCombRows * kHeadDim / 2; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red_m[threadIdx.x] = fmaxf(red_m[threadIdx.x], red_m[threadIdx.x + off]);
    __syncthreads();
  }
  mm = red_m[0];
  float ls = 0.f, os = 0.f;
  if (mm != -INFINITY) {
#pragma unroll 4
    for (int s = r; s < a.nsplit; s += kCombRows) {
      const float* x = pp + (size_t)s * stride;
      const float f = x[0] == -INFINITY ? 0.f : fast_exp2(x[0] - mm);
      ls += x[1] * f;
      os += x[2 + d] * f;
    }
  }
  part_o[r][d] = os;
  if (d == 0) part_l[r] = ls;
  __syncthreads();
  if (r != 0) return;
  float lt = 0.f, ot = 0.f;
#pragma unroll
  for (int q = 0; q < kCombRows; ++q) {
    lt += part_l[q];
    ot += part_o[q][d];
  }
  const float out = lt > 0.f ? ot / lt : 0.f;
  a.o[(size_t)h * kHeadDim + d] = (uint16_t)(pack_bf16x2(out, 0.f) & 0xffffu);
  if (d == 0 && a.lse) a.lse[h] = lt > 0.f ? (mm + log2f(lt)) * 0.69314718055994531f : -INFINITY;
}

__global__ __launch_bounds__(256) void iota_rows_kernel(int32_t* dst, int cols) {
  int32_t* row = dst + (size_t)blockIdx.y * cols;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c < cols) row[c] = c;
}

}  // namespace

hipError_t launch_iota_rows(int32_t* dst, int rows, int cols, hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  hipLaunchKernelGGL(iota_rows_kernel, dim3((cols + 255) / 256, rows), dim3(256), 0, stream, dst, cols);
  return hipGetLastError();
}

// Blocks per split for `rows` workgroup rows (query heads, or head groups for
// dense decoding): about 2048 workgroups in total, whole multiples of the 4
// waves of a workgroup.
int decode_blocks_per_split(int kb, int rows) {
  const long long want = ((long long)kb * rows + 2047) / 2048;
  int bps = (int)((want + 3) / 4 * 4);
  return bps < 4 ? 4 : bps;
}

hipError_t launch_decode(const DecodeLaunch& a, bool select, hipStream_t stream) {
  if (a.grp > kDecMaxGroup || a.nb > kDecMaxBlocks) return hipErrorInvalidValue;
  if (select) {
    hipLaunchKernelGGL(decode_score_kernel, dim3((a.nb + 63) / 64, a.hkv),
                       dim3(kDecThreads), 0, stream, a);
    if (a.seg_key && a.nseg > 1) {
      hipLaunchKernelGGL(decode_topk_seg_kernel, dim3(a.nseg, a.hq), dim3(256), 0, stream, a);
      const int per2 = (a.nseg * a.kb + 255) / 256;
      if (per2 <= 1)
        hipLaunchKernelGGL(decode_topk_merge_kernel<1>, dim3(a.hq), dim3(256), 0, stream, a);
      else if (per2 <= 2)
        hipLaunchKernelGGL(decode_topk_merge_kernel<2>, dim3(a.hq), dim3(256), 0, stream, a);
      else if (per2 <= 4)
        hipLaunchKernelGGL(decode_topk_merge_kernel<4>, dim3(a.hq), dim3(256), 0, stream, a);
      else
        hipLaunchKernelGGL(decode_topk_merge_kernel<8>, dim3(a.hq), dim3(256), 0, stream, a);
    } else if (a.nb <= 1024)
      hipLaunchKernelGGL(decode_topk_kernel<1>, dim3(a.hq), dim3(1024), 0, stream, a);
    else if (a.nb <= 4096)
      hipLaunchKernelGGL(decode_topk_kernel<4>, dim3(a.hq), dim3(1024), 0, stream, a);
    else
      hipLaunchKernelGGL(decode_topk_kernel<16>, dim3(a.hq), dim3(1024), 0, stream, a);
  }
  if (a.blk) {
    hipLaunchKernelGGL(decode_attn_kernel<1>, dim3(a.nsplit, a.hq), dim3(kDecThreads), 0, stream, a);
  } else if (a.grp % 4 == 0) {
    hipLaunchKernelGGL(decode_attn_kernel<4>, dim3(a.nsplit, a.hq / 4), dim3(kDecThreads), 0, stream, a);
  } else if (a.grp % 2 == 0) {
    hipLaunchKernelGGL(decode_attn_kernel<2>, dim3(a.nsplit, a.hq / 2), dim3(kDecThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(decode_attn_kernel<1>, dim3(a.nsplit, a.hq), dim3(kDecThreads), 0, stream, a);
  }
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.hq), dim3(kCombRows * kHeadDim), 0, stream, a);
  return hipGetLastError();
}

}  // namespace minf
