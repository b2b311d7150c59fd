// Vertical-Slash online index for gfx950.
//
// What is computed (MInference 1.0 article, "Method": the attention between
// the last queries and all keys estimates the best vertical and slash
// indices): for each VS query head, the causally masked softmax rows of the
// last r <= 64 queries against every key, their column sums v[j] and diagonal
// sums sl[dl] (dl = i - j), then the top-k columns and top-k offsets.
//
// MI355X layout of the work:
//  * a workgroup takes up to 4 query heads that share one KV head (one wave
//    per head) and a contiguous chunk of 64-key tiles, so each K tile is read
//    from HBM once for the whole GQA group;
//  * S^T = K Q_last^T on 32x32x16 bf16 MFMA (fp32 accumulate);
//  * pass 1 keeps per-lane running (max, sum of exp2) per query row; chunk
//    partials are merged in a fixed chunk order (no float atomics);
//  * pass 2 recomputes the scores, normalises them, and reduces the 64x64
//    probability tile along columns (complete column sums) and along its 127
//    diagonals (per-tile partials; a diagonal spans at most two tiles and the
//    two partials are added in tile order by a separate kernel);
//  * top-k (topk.hip) is a radix select on the sortable bit pattern spread
//    over many workgroups per row, ties to the lower index, emitted in
//    ascending index order.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kThreads = 256;
constexpr int KSTR = 136;
constexpr int PSTR = 64;   // floats per probability-tile row in LDS (rows stored skewed)
constexpr int PROWS = 32;  // query rows of the probability tile staged at a time
// s_waitcnt immediate on gfx9: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kWaitVmem0 = 0x0F70;

struct VsSmem1 {
  uint16_t kt[kBlock * KSTR];
};
struct VsSmem2 {
  uint16_t kt[kBlock * KSTR];
  float pt[4][PROWS * PSTR];
};

template <int PASS>
__device__ __forceinline__ void vs_pass(const VsLaunch& a) {
  __shared__ typename std::conditional<PASS == 1, VsSmem1, VsSmem2>::type sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const VsGroup* grp = &a.groups[blockIdx.y];
  const int ch = blockIdx.x;
  const int n = a.n;
  const int r = a.r;
  const bool active = wave < grp->cnt;
  const int head = active ? grp->head[wave] : 0;
  const int slot = active ? grp->slot[wave] : 0;
  const uint16_t* kh = a.k + (size_t)grp->kv * n * kHeadDim;
  const float sl2 = a.scale_log2;

  // last-query rows as MFMA B operands: row slot t = 32*nt + r32 is query row n - r + t
  u32x4 qr[2][8];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int t = 32 * nt + r32;
    const bool ok = active && t < r;
    const int64_t i = (int64_t)n - r + (ok ? t : 0);
    const uint16_t* qp = a.q + ((size_t)head * n + i) * kHeadDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qr[nt][ks] = ok ? *(const u32x4*)(qp + 16 * ks) : u32x4{0, 0, 0, 0};
  }
  float run_m[2] = {-INFINITY, -INFINITY};
  float run_l[2] = {0.f, 0.f};
  float rm[2] = {0.f, 0.f}, ril[2] = {0.f, 0.f};
  if constexpr (PASS == 2) if (active) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = 32 * nt + r32;
      rm[nt] = a.row_m[slot * 64 + t];
      ril[nt] = a.row_il[slot * 64 + t];
    }
  }

  // K tiles: 16 threads per 256-byte row, rows kr + 16 i; the next tile is
  // loaded into registers while the current one is worked on
  const int dc = tid & 15;
  const int kr = tid >> 4;
  u32x4 kn[4];
  auto load_tile = [&](int T) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t j = (int64_t)T * kBlock + kr + 16 * i;
      kn[i] = j < n ? *(const u32x4*)(kh + (size_t)j * kHeadDim + 8 * dc) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(sm.kt + (kr + 16 * i) * KSTR + 8 * dc) = kn[i];
  };

  const int t0 = ch * a.tiles_per_chunk;
  const int t1 = t0 + a.tiles_per_chunk < a.ntiles ? t0 + a.tiles_per_chunk : a.ntiles;
  if (t0 < t1) {
    load_tile(t0);
    store_tile();
  }
  // the query operands (and the row statistics) have arrived on every path
  // into the loop, so that the loop's wait counts only cover the next K tile
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  __syncthreads();
  for (int T = t0; T < t1; ++T) {
    if (T + 1 < t1) load_tile(T + 1);
    // the causal mask only bites in tiles that reach past the first last-query row
    const bool edge = (int64_t)T * kBlock + kBlock - 1 > (int64_t)n - r;
    if constexpr (PASS == 1) if (active) {
      f32x16 s[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        s[mt][0] = f32x16{};
        s[mt][1] = f32x16{};
        const uint16_t* kp = sm.kt + (32 * mt + r32) * KSTR + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const u32x4 av = *(const u32x4*)(kp + 16 * ks);
          s[mt][0] = mfma32(av, qr[0][ks], s[mt][0]);
          s[mt][1] = mfma32(av, qr[1][ks], s[mt][1]);
        }
      }
      {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int t = 32 * nt + r32;
          const int64_t iq = (int64_t)n - r + t;
          const bool row_ok = t < r;
          float mx = -INFINITY;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int64_t j = (int64_t)T * kBlock + 32 * mt + 8 * (i >> 2) + 4 * g + (i & 3);
              const bool ok = row_ok && (!edge || j <= iq);
              const float x = ok ? s[mt][nt][i] * sl2 : -INFINITY;
              s[mt][nt][i] = x;
              mx = fmaxf(mx, x);
            }
          const float m_new = fmaxf(run_m[nt], mx);
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          float acc = 0.f;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc += fast_exp2(s[mt][nt][i] - m_use);
          run_l[nt] = run_l[nt] * fast_exp2(run_m[nt] - m_use) + acc;
          run_m[nt] = m_new;
        }
      }
    }
    if constexpr (PASS == 2) {
      // normalised probabilities, staged 32 query rows at a time with row t
      // rotated by t, so that every diagonal e = t - c + 63 of the tile lies in
      // one LDS column; the column sum (lane = key) and the diagonal partials
      // (lane = column s: diagonals 63 - s and 127 - s) run over t in ascending
      // order across the two halves, each a 32-step loop with no divergence
      float* pt = sm.pt[wave];
      float cs = 0.f;
      float ds[2] = {0.f, 0.f};
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if (active) {
          // scores of this half's 32 query rows (S^T = K Q^T on MFMA)
          f32x16 s[2];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            s[mt] = f32x16{};
            const uint16_t* kp = sm.kt + (32 * mt + r32) * KSTR + 8 * g;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) s[mt] = mfma32(*(const u32x4*)(kp + 16 * ks), qr[nt][ks], s[mt]);
          }
          const int t = 32 * nt + r32;
          const int64_t iq = (int64_t)n - r + t;
          const bool row_ok = t < r;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kx = 32 * mt + 8 * (i >> 2) + 4 * g + (i & 3);
              const int64_t j = (int64_t)T * kBlock + kx;
              const bool ok = row_ok && (!edge || j <= iq);
              const float pv = ok ? fast_exp2(fmaf(s[mt][i], sl2, -rm[nt])) * ril[nt] : 0.f;
              pt[r32 * PSTR + ((kx - t) & 63)] = pv;
            }
        }
        // pt is private to the wave and a wave's LDS accesses complete in order:
        // no workgroup barrier around its staging
        __builtin_amdgcn_wave_barrier();
        if (active) {
          // row t holds key c at column (c - t) mod 64: key `lane` of row t is at
          // (lane - t) mod 64, and column s holds diagonal 63 - s for t < 64 - s
          // and diagonal 127 - s after (c = s + t, resp. s + t - 64)
#pragma unroll 4
          for (int tl = 0; tl < PROWS; ++tl) {
            const int t = 32 * nt + tl;
            cs += pt[tl * PSTR + ((lane - t) & 63)];
            const float x = pt[tl * PSTR + lane];
            if (t < 64 - lane)
              ds[0] += x;
            else
              ds[1] += x;
          }
        }
        __builtin_amdgcn_wave_barrier();  // the next half overwrites pt
      }
      if (active) {
        const int64_t j = (int64_t)T * kBlock + lane;
        if (j < n) a.vcol[(size_t)slot * n + j] = cs;
        float* dp = a.dpart + ((size_t)slot * a.ntiles + T) * 128;
        dp[63 - lane] = ds[0];
        dp[127 - lane] = ds[1];
      }
    }
    __syncthreads();  // every wave is done with this K tile
    if (T + 1 < t1) {
      store_tile();
      __syncthreads();
    }
  }
  if constexpr (PASS == 1) if (active) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float om = __shfl_xor(run_m[nt], 32);
      const float ol = __shfl_xor(run_l[nt], 32);
      const float mc = fmaxf(run_m[nt], om);
      const float mu = mc == -INFINITY ? 0.f : mc;
      const float lc = run_l[nt] * fast_exp2(run_m[nt] - mu) + ol * fast_exp2(om - mu);
      if (g == 0) {
        const int t = 32 * nt + r32;
        const size_t o = ((size_t)slot * 64 + t) * a.nchunks + ch;
        a.part_m[o] = mc;
        a.part_l[o] = lc;
      }
    }
  }
}

// Pass 1 fits 3 waves per SIMD (168 VGPRs, a few spilled: 1.15 -> 0.96 ms at 1M
// tokens); pass 2 runs 2 (at 3 waves it spilled 35 VGPRs and took 3.1 instead
// of 2.0 ms).
template <int PASS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void vs_pass_kernel(
    const VsLaunch a) {
  vs_pass<PASS>(a);
}
template <>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void vs_pass_kernel<1>(
    const VsLaunch a) {
  vs_pass<1>(a);
}

// Merge the chunk partials of every row in chunk order: max and 1 / sum.
__global__ __launch_bounds__(64) void vs_row_combine_kernel(const VsLaunch a) {
  const int slot = blockIdx.x;
  const int t = threadIdx.x;
  const float* pm = a.part_m + ((size_t)slot * 64 + t) * a.nchunks;
  const float* pl = a.part_l + ((size_t)slot * 64 + t) * a.nchunks;
  float m = -INFINITY;
  for (int c = 0; c < a.nchunks; ++c) m = fmaxf(m, pm[c]);
  const float mu = m == -INFINITY ? 0.f : m;
  float l = 0.f;
  for (int c = 0; c < a.nchunks; ++c) l += pl[c] * fast_exp2(pm[c] - mu);
  a.row_m[slot * 64 + t] = mu;
  a.row_il[slot * 64 + t] = l > 0.f ? 1.f / l : 0.f;
}

// sl[dl] = sum over the (at most two) tiles whose diagonal window holds dl, in tile order.
__global__ __launch_bounds__(256) void vs_diag_reduce_kernel(const VsLaunch a) {
  const int slot = blockIdx.y;
  const int64_t dl = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n = a.n;
  if (dl >= n) return;
  // tile T holds dl at e = dl - (n - r - 64T - 63), valid for e in [0, 126]
  const int64_t base = n - a.r - 63 - dl;
  int64_t tlo = -floor_div(-base, 64);  // ceil(base / 64)
  int64_t thi = floor_div(base + 126, 64);
  if (tlo < 0) tlo = 0;
  if (thi > a.ntiles - 1) thi = a.ntiles - 1;
  float s = 0.f;
  for (int64_t T = tlo; T <= thi; ++T) {
    const int64_t e = 64 * T - base;  // = dl - (n - r - 64T - 63), in [0, 126]
    s += a.dpart[((size_t)slot * a.ntiles + T) * 128 + e];
  }
  a.slsum[(size_t)slot * n + dl] = s;
}

// Top-k of each row of a float matrix, ascending indices, ties to the lower index.
}  // namespace

hipError_t launch_vs_scores(const VsLaunch& a, hipStream_t stream) {
  dim3 grid(a.nchunks, a.ngroups);
  hipLaunchKernelGGL(vs_pass_kernel<1>, grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vs_row_combine_kernel, dim3(a.n_slots), dim3(64), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_pass_kernel<2>, grid, dim3(kThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 g2((unsigned)((a.n + 255) / 256), a.n_slots);
  hipLaunchKernelGGL(vs_diag_reduce_kernel, g2, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace minf
