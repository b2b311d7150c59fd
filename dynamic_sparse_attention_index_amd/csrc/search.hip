// Offline pattern search support for gfx950: the work of a head's plan in the
// sparse kernel's unit, and the attention recall of a mask from LSE rows.
//
// MInference 1.0 article, "Method": each head's pattern is chosen offline by a
// kernel-aware search, which compares candidates at their cost in the sparse
// kernel; talk transcript ("KV-cache-centric methods", MInference part):
// attention recall, the share of a row's attention that an index keeps.
//
// Work (one workgroup per head, integer counts, exact): summed over query
// blocks b, the 64-key blocks the attention kernel computes for b, plus every
// gathered vertical column as 1/64 of a block.
//  * dense: c <= b, nb (nb + 1) / 2 in all;
//  * A-shape: the sink blocks [0, ceil(sink / 64)) up to b, and the window
//    blocks from the block of key 64 b - local + 1 up to b;
//  * Block-Sparse: blk_cnt[b];
//  * Vertical-Slash: the block-offset bitmap O of the slashes (built by the
//    attention call's own offset kernel) gives key blocks b - o, o in O, o <= b,
//    so a full block b computes |O n [0, b]| blocks and the full blocks
//    together sum (nfull - o) over o in O below nfull; a partial last block
//    has its own bitmap. A vertical column j (block cb) is gathered for every
//    query block b >= cb whose offset set lacks b - cb.
// Recall (one workgroup per head, fp64): mean over the listed rows of
// exp(LSE_mask - LSE_dense), 0 where the mask row is empty (LSE = -inf).
// Both reductions run in a fixed order, so results are reproducible bitwise.
#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kThreads = 256;
constexpr int kBitWords = (kMaxTokens / kBlock) / 32 + 1;

// Sum over the block of per-thread int64 values, in a fixed order.
__device__ long long block_sum_i64(long long x, long long* red) {
  red[threadIdx.x] = x;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const long long r = red[0];
  __syncthreads();
  return r;
}

__device__ double block_sum_f64(double x, double* red) {
  red[threadIdx.x] = x;
  __syncthreads();
  for (int s = kThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kThreads) void plan_work_kernel(const WorkLaunch a) {
  __shared__ long long red[kThreads];
  __shared__ uint32_t bits[kBitWords];
  __shared__ int32_t pre[kBitWords + 1];  // set bits of the full-block bitmap before each word
  const WorkHead hd = a.heads[blockIdx.x];
  const int tid = threadIdx.x;
  const int nb = a.nb;
  long long blocks = 0, cols = 0;
  if (hd.kind == KIND_W_DENSE) {
    blocks = tid == 0 ? (long long)nb * (nb + 1) / 2 : 0;
  } else if (hd.kind == KIND_W_BLOCK) {
    for (int b = tid; b < nb; b += kThreads) blocks += hd.blk_cnt[b];
  } else if (hd.kind == KIND_W_ASHAPE) {
    const long long sb = ((long long)hd.sink + kBlock - 1) / kBlock;
    const int reach = hd.local > 0 ? (int)(((long long)hd.local + kBlock - 2) / kBlock) : 0;
    for (int b = tid; b < nb; b += kThreads) {
      const long long sink_n = sb < b + 1 ? sb : b + 1;  // blocks [0, min(sb, b + 1))
      if (hd.local <= 0) {
        blocks += sink_n;
        continue;
      }
      const long long wlo = b - reach > 0 ? b - reach : 0;  // window blocks [wlo, b]
      const long long over = sink_n - wlo > 0 ? sink_n - wlo : 0;
      blocks += sink_n + (b - wlo + 1) - over;
    }
  } else {  // Vertical-Slash
    const int nwords = (nb >> 5) + 1;
    const int partial = (a.n & (kBlock - 1)) != 0;
    const int nfull = partial ? nb - 1 : nb;
    for (int i = tid; i < nwords; i += kThreads) bits[i] = hd.obits[i];
    __syncthreads();
    if (tid == 0) {
      int run = 0;
      for (int i = 0; i < nwords; ++i) {
        pre[i] = run;
        run += __popc(bits[i]);
      }
      pre[nwords] = run;
    }
    __syncthreads();
    // |O n [0, m]| for m >= 0
    auto count_upto = [&](int m) -> int {
      const int w = m >> 5;
      const uint32_t mask = (m & 31) == 31 ? 0xffffffffu : ((1u << ((m & 31) + 1)) - 1u);
      return pre[w] + __popc(bits[w] & mask);
    };
    // full blocks: sum over o in O, o < nfull, of (nfull - o)
    for (int o = tid; o < nfull; o += kThreads)
      if ((bits[o >> 5] >> (o & 31)) & 1u) blocks += nfull - o;
    const uint32_t* last = hd.obits + nwords;  // offset bitmap of the partial last block
    if (partial && tid == 0) {
      for (int i = 0; i <= ((nb - 1) >> 5); ++i) {
        uint32_t w = last[i];
        if (i == ((nb - 1) >> 5)) w &= ((nb - 1) & 31) == 31 ? 0xffffffffu : ((1u << (((nb - 1) & 31) + 1)) - 1u);
        blocks += __popc(w);
      }
    }
    // vertical columns: unique, ascending, in [0, n)
    for (int e = tid; e < hd.k_v; e += kThreads) {
      const int j = hd.v_idx[e];
      if (j < 0 || j >= a.n || (e > 0 && hd.v_idx[e - 1] == j)) continue;
      const int cb = j / kBlock;
      if (cb < nfull) cols += (nfull - cb) - count_upto(nfull - 1 - cb);
      if (partial) {
        const int t = nb - 1 - cb;
        cols += ((last[t >> 5] >> (t & 31)) & 1u) ? 0 : 1;
      }
    }
  }
  blocks = block_sum_i64(blocks, red);
  cols = block_sum_i64(cols, red);
  if (tid == 0) a.out[blockIdx.x] = (double)blocks + (double)cols / kBlock;
}

__global__ __launch_bounds__(kThreads) void recall_kernel(const float* lse_mask, const float* lse_dense, int n,
                                                          const int32_t* rows, int n_rows, double* out) {
  __shared__ double red[kThreads];
  const int h = blockIdx.x;
  const float* lm = lse_mask + (size_t)h * n;
  const float* ld = lse_dense + (size_t)h * n;
  double acc = 0.0;
  for (int r = threadIdx.x; r < n_rows; r += kThreads) {
    const int i = rows ? rows[r] : r;
    if (i < 0 || i >= n) continue;
    const float m = lm[i];
    if (m == -INFINITY) continue;
    acc += exp((double)m - (double)ld[i]);
  }
  acc = block_sum_f64(acc, red);
  if (threadIdx.x == 0) out[h] = acc / (double)n_rows;
}

}  // namespace

hipError_t launch_plan_work(const WorkLaunch& a, int count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_work_kernel, dim3(count), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_recall(const float* lse_mask, const float* lse_dense, int n, int hq, const int32_t* rows,
                         int n_rows, double* out, hipStream_t stream) {
  hipLaunchKernelGGL(recall_kernel, dim3(hq), dim3(kThreads), 0, stream, lse_mask, lse_dense, n, rows, n_rows, out);
  return hipGetLastError();
}

}  // namespace minf
