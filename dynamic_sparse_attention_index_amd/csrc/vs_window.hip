// Slash-aligned windows of the Vertical-Slash pattern for gfx950.
//
// What is computed (talk transcript, MMInference part on the permutation
// details: shifting indices, i.e. reading with skipped rows or columns,
// rearranges vertical and slash lines into dense regions; the plainest
// reading for a slash is used here): for query block b (rows 64b .. 64b + 63)
// each selected diagonal offset dl contributes the 64 keys
// [64b - dl, 64b - dl + 64) -- the keys the slash meets from the block's 64
// rows, which are one contiguous range -- as one window computed as a dense
// 64x64 tile, instead of the one or two grid blocks the slash crosses. The
// mask of row i is j <= i and (j in a window of its block or j a vertical
// column).
//
// Preparation per head, three stream-ordered launches:
//  * the bitmap of the offsets over [0, n) (cleared, then set);
//  * the cover of U = union over dl of [-dl, -dl + 64), relative to the block's
//    first row, by disjoint tiles in ascending order: every maximal interval of
//    U is cut into 64-key tiles from its start, a tile being (start, end) with
//    end - start <= 64. Block b's windows are U + 64b, so one cover serves every
//    query block. One wave per head walks the bitmap from the highest offset
//    down (window starts ascending) 64 words at a time, reading each non-empty
//    word into scalar registers.
#include "common.h"
#include "launch.h"

namespace minf {
namespace {

__global__ __launch_bounds__(256) void vsw_clear_kernel(const VswLaunch a) {
  const int h = blockIdx.y;
  const int nwords = (a.n + 31) >> 5;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < nwords) a.dbits[h][i] = 0u;
}

__global__ __launch_bounds__(256) void vsw_bits_kernel(const VswLaunch a) {
  const int h = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= a.k_s[h]) return;
  const int dl = a.s_idx[h][e];
  if (dl < 0 || dl >= a.n) return;
  atomicOr(a.dbits[h] + (dl >> 5), 1u << (dl & 31));
}

__global__ __launch_bounds__(64) void vsw_cover_kernel(const VswLaunch a) {
  const int h = blockIdx.x;
  const int lane = threadIdx.x;
  const uint32_t* bits = a.dbits[h];
  int2* out = a.tiles[h];
  const int cap = a.cap;
  const int nwords = (a.n + 31) >> 5;
  int cnt = 0;
  bool open = false;
  int cs = 0, ce = 0;  // the open interval [cs, ce)
  auto emit = [&](int s, int e) {  // the interval's tiles, 64 at a time across the lanes
    const int nt = (e - s + kBlock - 1) / kBlock;
    for (int t0 = 0; t0 < nt; t0 += 64) {
      const int t = t0 + lane;
      if (t < nt && cnt + t < cap) {
        const int ts = s + t * kBlock;
        out[cnt + t] = int2{ts, ts + kBlock < e ? ts + kBlock : e};
      }
    }
    cnt += nt;
  };
  for (int w0 = ((nwords - 1) >> 6) << 6; w0 >= 0; w0 -= 64) {
    const int wi = w0 + lane;
    const uint32_t mine = wi < nwords ? bits[wi] : 0u;
    // only the non-empty words, highest first (the offsets are sparse)
    uint64_t nz = __ballot(mine != 0u);
    while (nz != 0ull) {
      const int j = 63 - __builtin_clzll(nz);
      nz &= ~(1ull << j);
      uint32_t wd = (uint32_t)__builtin_amdgcn_readlane((int)mine, j);
      while (wd != 0u) {
        const int bit = 31 - __builtin_clz(wd);
        wd &= ~(1u << bit);
        const int s = -(((w0 + j) << 5) + bit);  // window [s, s + 64), starts ascending
        if (open && s <= ce) {
          ce = s + kBlock;
        } else {
          if (open) emit(cs, ce);
          open = true;
          cs = s;
          ce = s + kBlock;
        }
      }
    }
  }
  if (open) emit(cs, ce);
  if (lane == 0) a.count[h][0] = cnt < cap ? cnt : cap;
}

}  // namespace

int vsw_tile_capacity(int n) {
  // intervals are disjoint inside [-(n - 1), 64) and separated by gaps, so
  // sum over intervals of ceil(length / 64) <= 2 n_b + 2
  return 2 * ((n + kBlock - 1) / kBlock) + 4;
}

hipError_t launch_vsw_prepare(const VswLaunch& a, int count, int max_k_s, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int nwords = (a.n + 31) >> 5;
  hipLaunchKernelGGL(vsw_clear_kernel, dim3((nwords + 255) / 256, count), dim3(256), 0, stream, a);
  if (max_k_s > 0)
    hipLaunchKernelGGL(vsw_bits_kernel, dim3((max_k_s + 255) / 256, count), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(vsw_cover_kernel, dim3(count), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace minf
