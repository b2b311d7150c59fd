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
//  * pass 2 recomputes the scores as S = Q_last K^T (so a lane holds one key
//    column and 16 query rows of each 32x32 product), normalises them, sums
//    the columns in registers (complete column sums), and reduces the 64x64
//    probability tile along its 127 diagonals through LDS (per-tile partials;
//    a diagonal spans at most two tiles and the two partials are added in
//    tile order by a separate kernel);
//  * top-k (topk.hip) is a radix select on the sortable bit pattern spread
//    over many workgroups per row, ties to the lower index, emitted in
//    ascending index order.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kThreads = 256;
constexpr int kTileHalves = kBlock * kHeadDim;  // one 64 x 128 bf16 K tile, rows of 256 bytes
constexpr int kRing = 3;                        // K tiles in LDS: T (read), T + 1 (landed), T + 2 (in flight)
// Staged probability rows, 16 query rows at a time (rows t = 16 h + tl of round
// h): row tl holds key c at column q = c - tl + 16, in [1, 79]. A row writes the
// same 64 columns in every round, so the ones it never writes stay zero, and
// column q of round h holds exactly the entries of diagonal e = t - c + 63 =
// 16 h + 79 - q. A row pitch of 89 floats puts the two half-waves' writes (rows
// tl and tl + 4, the same 32 keys) on complementary halves of the 64 banks; a
// row's columns are read by consecutive lanes.
constexpr int PSTR = 89;
constexpr int PROWS = 16;
constexpr int PCOLS = 80;
// s_waitcnt immediate on gfx9: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kWaitVmem0 = 0x0F70;
constexpr int kWaitVmem4 = 0x0F74;  // vmcnt(4): the newest tile's four copies may be in flight

__device__ __forceinline__ int swz(int x) { return ((x & 3) << 2) | ((x >> 2) & 3); }

// K tiles go HBM -> LDS with buffer loads into a ring of three buffers: tile
// T + 2 streams into the buffer tile T - 1 used while tile T is worked on, so
// one barrier per tile suffices. Rows of 256 bytes, the 16-byte chunk c of row
// x at chunk position c ^ swz(x) (conflict-free operand reads of 16 rows).
struct VsSmem1 {
  uint16_t kt[kRing][kTileHalves];
};
struct VsSmem2 {
  uint16_t kt[kRing][kTileHalves];
  float pt[4][PROWS * PSTR + 64];  // + 64: lanes 16..63 read past the 80 columns of the last row
  float pacc[4][4 * PCOLS];          // per wave: column partials of the four rounds of a tile
  float crow[4][64];                 // per wave: max + log2(sum) of each last-query row
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
  // pass 2: each row's normaliser in log2 units, max + log2(sum), kept in LDS;
  // the staging rows start at zero
  if constexpr (PASS == 2) {
    sm.crow[wave][lane] = active ? a.row_m[slot * 64 + lane] : 0.f;
    for (int x = lane; x < PROWS * PSTR + 64; x += 64) sm.pt[wave][x] = 0.f;
  }

  // K tiles: wave w's copy i fills LDS chunks [256 i + 64 w, +64) = rows
  // 16 i + 4 w .. +3, 16 lanes per 256-byte row, from the swizzled source chunk;
  // rows past n read row n - 1 (they are masked)
  const rsrc_t kbuf = buffer_of(kh, (uint32_t)n * (kHeadDim * 2));
  const int crow_lo = 4 * (tid >> 6) + ((tid & 63) >> 4);
  const uint32_t cbyte = (uint32_t)(((tid & 15) ^ swz(crow_lo)) * 16);
  auto issue_tile = [&](int T, uint16_t* kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int j = T * kBlock + 16 * i + crow_lo;
      j = j < n ? j : n - 1;
      copy16(kbuf, kt + (256 * i + 64 * wave) * 8, (uint32_t)j * 256u + cbyte, 0u);
    }
  };
  // operand reads: row x = 32 m + r32, chunk 2 ks + g, at kofs + 32 m rows, XOR (ks << 5)
  const int kofs = r32 * 256 + ((g ^ swz(r32)) << 4);

  const int t0 = ch * a.tiles_per_chunk;
  const int t1 = t0 + a.tiles_per_chunk < a.ntiles ? t0 + a.tiles_per_chunk : a.ntiles;
  if (t0 < t1) issue_tile(t0, sm.kt[0]);
  if (t0 + 1 < t1) issue_tile(t0 + 1, sm.kt[1]);
  // tile t0 (and the query operands and row statistics) have arrived on every
  // path into the loop, so that the loop's wait counts only cover K tiles
  if (t0 + 1 < t1)
    __builtin_amdgcn_s_waitcnt(kWaitVmem4);
  else
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  __syncthreads();
  int cur = 0;  // ring slot of tile T
  for (int T = t0; T < t1; ++T) {
    // tile T + 2 into the slot tile T - 1 used (every wave left it at the last barrier)
    const int nxt2 = cur == 0 ? 2 : cur - 1;
    if (T + 2 < t1) issue_tile(T + 2, sm.kt[nxt2]);
    const char* ktc = (const char*)sm.kt[cur];
    // the causal mask only bites in tiles that reach past the first last-query row
    const bool edge = (int64_t)T * kBlock + kBlock - 1 > (int64_t)n - r;
    if constexpr (PASS == 1) if (active) {
      f32x16 s[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        s[mt][0] = f32x16{};
        s[mt][1] = f32x16{};
        const char* kp = ktc + 32 * mt * 256;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const u32x4 av = *(const u32x4*)(kp + (kofs ^ (ks << 5)));
          s[mt][0] = mfma32(av, qr[0][ks], s[mt][0]);
          s[mt][1] = mfma32(av, qr[1][ks], s[mt][1]);
        }
      }
      {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int t = 32 * nt + r32;
          // key slot kx = 32 mt + 8 (i >> 2) + (i & 3) of this lane (key T 64 + kx + 4 g) is visible
          // iff kx <= lim: every slot below the causal edge, none for a row past r
          const int lim = t >= r ? -1 : (edge ? (n - r + t) - T * kBlock - 4 * g : kBlock);
          float mx = -INFINITY;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kx = 32 * mt + 8 * (i >> 2) + (i & 3);
              const float x = kx <= lim ? s[mt][nt][i] * sl2 : -INFINITY;
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
      // normalised probabilities P = exp2(s sl2 - crow) of S = Q K^T: lane l holds
      // key c = 32 mk + (l & 31) and, in accumulator slot i, query row
      // t = 32 mq + 8 (i >> 2) + 4 g + (i & 3). Column sums add up in registers
      // (then across the two half-waves); for the diagonal sums every 16 rows go
      // through LDS, where lane s adds up column s (and lanes s < 16 column
      // s + 64) over the 16 rows: one partial per round and column, merged per
      // diagonal after the tile.
      float* pt = sm.pt[wave];
      // row tl (of these 16), column c - tl + 16, with c = 32 mk + r32 and
      // tl = 8 (e >> 2) + 4 g + (e & 3), is pw + 32 mk + (PSTR - 1)(8 (e >> 2) + (e & 3)):
      // one lane base and a constant offset per store, the same in every round
      float* const pw = pt + r32 + 4 * g * (PSTR - 1) + 16;
      float* const pr = pt + lane;
      float cs[2] = {0.f, 0.f};
      float acc[4][2];  // round h, column lane (0) / lane + 64 (1, lanes < 16)
      // every row present and the tile below the causal edge: nothing is masked
      const bool plain = !edge && r == 64;
#pragma unroll
      for (int mq = 0; mq < 2; ++mq) {
        f32x16 sc[2];
        if (active) {
#pragma unroll
          for (int mk = 0; mk < 2; ++mk) {
            sc[mk] = f32x16{};
            const char* kp = ktc + 32 * mk * 256;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
              sc[mk] = mfma32(qr[mq][ks], *(const u32x4*)(kp + (kofs ^ (ks << 5))), sc[mk]);
          }
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {  // round h = 2 mq + hh: rows 16 h .. + 15, slots i = 8 hh .. + 7
          const int h = 2 * mq + hh;
          if (active) {
            float cr[8];
#pragma unroll
            for (int q2 = 0; q2 < 2; ++q2) {
              const float4 v4 = *(const float4*)&sm.crow[wave][16 * h + 8 * q2 + 4 * g];
              cr[4 * q2] = v4.x;
              cr[4 * q2 + 1] = v4.y;
              cr[4 * q2 + 2] = v4.z;
              cr[4 * q2 + 3] = v4.w;
            }
#pragma unroll
            for (int mk = 0; mk < 2; ++mk) {
              const int64_t j = (int64_t)T * kBlock + 32 * mk + r32;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int t = 16 * h + 8 * (e >> 2) + 4 * g + (e & 3);
                float pv = fast_exp2(fmaf(sc[mk][8 * hh + e], sl2, -cr[e]));
                if (!plain) pv = (t < r && (!edge || j <= (int64_t)n - r + t)) ? pv : 0.f;
                cs[mk] += pv;
                pw[32 * mk + (PSTR - 1) * (8 * (e >> 2) + (e & 3))] = pv;
              }
            }
          }
          // pt is private to the wave and a wave's LDS accesses complete in order:
          // no workgroup barrier around its staging
          __builtin_amdgcn_wave_barrier();
          if (active) {
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int tl = 0; tl < PROWS; ++tl) {
              a0 += pr[tl * PSTR];
              a1 += pr[tl * PSTR + 64];  // a column of the row only for lanes < 16
            }
            acc[h][0] = a0;
            acc[h][1] = a1;
          }
          __builtin_amdgcn_wave_barrier();  // the next rows overwrite pt
        }
      }
      if (active) {
        // the other half-wave holds the same keys' other query rows
        cs[0] += __shfl_xor(cs[0], 32);
        cs[1] += __shfl_xor(cs[1], 32);
        const int64_t j = (int64_t)T * kBlock + lane;
        if (j < n) a.vcol[(size_t)slot * n + j] = g ? cs[1] : cs[0];
      }
      // diagonal e = 16 h + 79 - q: the round partials go to LDS by (h, q), then lane l
      // adds up diagonals l and l + 64 over the rounds, in round order
      float* pa = sm.pacc[wave];
      if (active) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          pa[h * PCOLS + lane] = acc[h][0];
          if (lane < 16) pa[h * PCOLS + 64 + lane] = acc[h][1];
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (active) {
        float dd[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = lane + 64 * u;  // diagonal (e = 127 has no entries)
          float x = 0.f;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const int q = 16 * h + 79 - e;
            if (q >= 0 && q < PCOLS) x += pa[h * PCOLS + q];
          }
          dd[u] = x;
        }
        float* dp = a.dpart + ((size_t)slot * a.ntiles + T) * 128;
        dp[lane] = dd[0];
        dp[64 + lane] = dd[1];
      }
      __builtin_amdgcn_wave_barrier();  // the next tile overwrites pa
    }
    // tile T + 1 landed (only tile T + 2's copies may still be in flight), then one
    // barrier: tile T + 1 visible to every wave, tile T released
    if (T + 2 < t1)
      __builtin_amdgcn_s_waitcnt(kWaitVmem4);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    __syncthreads();
    cur = cur == 2 ? 0 : cur + 1;
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
  // one wave per (head, row): lane c takes chunks c, c + 64, ..., then a
  // butterfly over the lanes (a fixed order) merges them
  const int slot = blockIdx.y;
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* pm = a.part_m + ((size_t)slot * 64 + t) * a.nchunks;
  const float* pl = a.part_l + ((size_t)slot * 64 + t) * a.nchunks;
  float m = -INFINITY;
  for (int c = lane; c < a.nchunks; c += 64) m = fmaxf(m, pm[c]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float mu = m == -INFINITY ? 0.f : m;
  float l = 0.f;
  for (int c = lane; c < a.nchunks; c += 64) l += pl[c] * fast_exp2(pm[c] - mu);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
  if (lane == 0) {
    // pass 2 normalises with exp2(x - (max + log2(sum)))
    a.row_m[slot * 64 + t] = l > 0.f ? mu + __log2f(l) : INFINITY;
    a.row_il[slot * 64 + t] = l > 0.f ? 1.f / l : 0.f;
  }
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
  hipLaunchKernelGGL(vs_row_combine_kernel, dim3(64, a.n_slots), dim3(64), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_pass_kernel<2>, grid, dim3(kThreads), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  dim3 g2((unsigned)((a.n + 255) / 256), a.n_slots);
  hipLaunchKernelGGL(vs_diag_reduce_kernel, g2, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace minf
