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
//    probability tile along its 127 diagonals: four rows at a time by DPP
//    lane shifts in registers, then through LDS; a diagonal spans at most two
//    consecutive tiles, whose partials are added in tile order by the
//    workgroup that runs both, or for the tiles at a chunk edge by a small
//    separate kernel;
//  * top-k (topk.hip) is a radix select on the sortable bit pattern spread
//    over many workgroups per row, ties to the lower index, emitted in
//    ascending index order.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kThreads = 256;   // pass 1: one wave per query head of the group
constexpr int kThreads2 = 512;  // pass 2: two waves per query head (32 query rows each)
constexpr int kTileHalves = kBlock * kHeadDim;  // one 64 x 128 bf16 K tile, rows of 256 bytes
constexpr int kRing = 3;                        // K tiles in LDS: T (read), T + 1 (landed), T + 2 (in flight)
// Diagonal sums of a 64 x 64 probability tile. In the MFMA layout a lane holds
// one key column c and, in each group of four accumulator slots, four
// consecutive query rows t0 .. t0 + 3. A chain of row shifts by one lane
// (within 16-lane rows) adds those four rows along their diagonals in
// registers: after it, lane c holds the sum over b of P[t0 + b][c - 3 + b]
// (diagonal t0 + 3 - c), and the pieces that leave a 16-lane row at its top
// lane are kept there as carries. The chain sums of 32 query rows (8 row groups
// u) then go through LDS in a skewed layout: group u writes key c at column
// c - 4u + 28 of row u, and the carries of groups u < 4 (u >= 4) go to row 8
// (9) at the column of the diagonal they belong to (no two carries share a
// cell). Column q of these ten rows then holds pieces of exactly one diagonal,
// 32 mq + 94 - q for the query rows 32 mq .. + 31, and lane s adds up column s
// (lanes < 32 also column s + 64) over the rows. Cells that are never written
// stay zero. A row pitch of 100 floats puts the two half-waves' chain stores
// on complementary halves of the 64 banks.
constexpr int PSTR = 100;
constexpr int PROWS = 10;
constexpr int PCOLS = 96;
// s_waitcnt immediate on gfx9: vmcnt(0), expcnt and lgkmcnt left at their maxima
constexpr int kWaitVmem0 = 0x0F70;
constexpr int kWaitVmem4 = 0x0F74;  // vmcnt(4): the newest tile's four copies may be in flight

__device__ __forceinline__ int swz(int x) { return ((x & 3) << 2) | ((x >> 2) & 3); }

// Four floats from 16-byte aligned LDS, read as one 128-bit integer vector. Read
// as float4, the compiler makes this load wait for every buffer-to-LDS copy in
// flight (here the next K tile, which it cannot tell apart), and the copy
// would no longer overlap the tile's work.
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 lds_f32x4(const float* p) {
  return __builtin_bit_cast(f32x4, *(const u32x4*)(const void*)p);
}

// x of the next lower lane within each 16-lane row, 0 in the row's lowest lane (DPP row_shr:1)
__device__ __forceinline__ float row_shr1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xF, 0xF, true));
}

// K tiles go HBM -> LDS with buffer loads into a ring of three buffers: tile
// T + 2 streams into the buffer tile T - 1 used while tile T is worked on, so
// one barrier per tile suffices. Rows of 256 bytes, the 16-byte chunk c of row
// x at chunk position c ^ swz(x) (conflict-free operand reads of 16 rows).
struct VsSmem1 {
  uint16_t kt[kRing][kTileHalves];
};
// Pass 2 holds two K tiles (T, and T + 1 in flight) so that two workgroups of
// eight waves fit a compute unit. Results of a tile are exchanged between the
// two waves of a head through buffers indexed by tile parity: the merge of tile
// T (after the barrier that ends it) and the writes of tile T + 2 (after the
// barrier that ends tile T + 1) never overlap.
struct alignas(16) VsSmem2 {
  uint16_t kt[2][kTileHalves];
  float pt[8][PROWS * PSTR];     // per wave: diagonal staging rows
  float pacc[2][4][2 * PCOLS];   // [parity][head]: diagonal columns of query rows 0..31, then 32..63
  float csum[2][4][2][64];       // [parity][head][half]: column sums of 32 query rows
  float crow[4][64];             // [head]: max + log2(sum) of each last-query row
  float dkeep[4][64];            // [head]: diagonals e = 0..63 of the previous tile (merging wave only)
};

// Pass 1: per-chunk (max, sum of exp2) of every last-query row.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void vs_pass1_kernel(
    const VsLaunch a) {
  __shared__ VsSmem1 sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps head, slot and pointers scalar
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
    if (active) {
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
      // masked slots become -inf in the raw scores (only in tiles that reach
      // past the first last-query row, or when fewer than 64 rows exist)
      if (edge || r < 64) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int t = 32 * nt + r32;
          // key slot kx = 32 mt + 8 (i >> 2) + (i & 3) of this lane (key T 64 + kx + 4 g) is visible
          // iff kx <= lim: every slot below the causal edge, none for a row past r
          const int lim = t >= r ? -1 : (edge ? (n - r + t) - T * kBlock - 4 * g : kBlock);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kx = 32 * mt + 8 * (i >> 2) + (i & 3);
              s[mt][nt][i] = kx <= lim ? s[mt][nt][i] : -INFINITY;
            }
        }
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        // the row max of the raw scores (scaling by sl2 > 0 keeps the order),
        // as four three-input max chains
        float mq4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float x = fmaxf(s[0][nt][4 * c], s[0][nt][4 * c + 1]);
          x = fmaxf(x, fmaxf(s[0][nt][4 * c + 2], s[0][nt][4 * c + 3]));
          x = fmaxf(x, fmaxf(s[1][nt][4 * c], s[1][nt][4 * c + 1]));
          mq4[c] = fmaxf(x, fmaxf(s[1][nt][4 * c + 2], s[1][nt][4 * c + 3]));
        }
        const float mx = fmaxf(fmaxf(mq4[0], mq4[1]), fmaxf(mq4[2], mq4[3])) * sl2;
        const float m_new = fmaxf(run_m[nt], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        // sum of exp2(s sl2 - m), one fused multiply-add per element, in two chains
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          acc0 += fast_exp2(fmaf(s[0][nt][i], sl2, -m_use));
          acc1 += fast_exp2(fmaf(s[1][nt][i], sl2, -m_use));
        }
        run_l[nt] = run_l[nt] * fast_exp2(run_m[nt] - m_use) + (acc0 + acc1);
        run_m[nt] = m_new;
      }
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
  if (active) {
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

// Pass 2: normalised probabilities P = exp2(s sl2 - crow) of S = Q K^T, their
// column sums and per-tile diagonal sums. Wave w takes query head w & 3 of the
// group and query rows 32 mq .. + 31, mq = w >> 2: lane l holds key
// c = 32 mk + (l & 31) and, in accumulator slot 4 a + b, query row
// t = 32 mq + 8 a + 4 g + b.
__global__ __launch_bounds__(kThreads2) __attribute__((amdgpu_waves_per_eu(4))) void vs_pass2_kernel(
    const VsLaunch a) {
  __shared__ VsSmem2 sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps head, slot and pointers scalar
  const int hw = wave & 3;
  const int mq = wave >> 2;
  const int g = lane >> 5;
  const int r32 = lane & 31;
  const VsGroup* grp = &a.groups[blockIdx.y];
  const int ch = blockIdx.x;
  const int n = a.n;
  const int r = a.r;
  const bool active = hw < grp->cnt;
  const int head = active ? grp->head[hw] : 0;
  const int slot = active ? grp->slot[hw] : 0;
  const uint16_t* kh = a.k + (size_t)grp->kv * n * kHeadDim;
  const float sl2 = a.scale_log2;

  // query rows t = 32 mq + r32 as MFMA A operands
  u32x4 qr[8];
  {
    const int t = 32 * mq + r32;
    const bool ok = active && t < r;
    const int64_t i = (int64_t)n - r + (ok ? t : 0);
    const uint16_t* qp = a.q + ((size_t)head * n + i) * kHeadDim + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qr[ks] = ok ? *(const u32x4*)(qp + 16 * ks) : u32x4{0, 0, 0, 0};
  }
  // each row's normaliser in log2 units, max + log2(sum); the staging rows start at zero
  if (g == 0) sm.crow[hw][32 * mq + r32] = active ? a.row_m[slot * 64 + 32 * mq + r32] : 0.f;
  for (int x = lane; x < PROWS * PSTR; x += 64) sm.pt[wave][x] = 0.f;

  // K tiles: wave w's copy i fills rows 32 i + 4 w .. + 3, 16 lanes per 256-byte
  // row, from the swizzled source chunk; rows past n read row n - 1 (they are masked)
  const rsrc_t kbuf = buffer_of(kh, (uint32_t)n * (kHeadDim * 2));
  auto issue_tile = [&](int T, uint16_t* kt, int ln) {
    const int crow_lo = 4 * wave + (ln >> 4);
    const uint32_t cbyte = (uint32_t)(((ln & 15) ^ swz(crow_lo)) * 16);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int j = T * kBlock + 32 * i + crow_lo;
      j = j < n ? j : n - 1;
      copy16(kbuf, kt + (512 * i + 64 * wave) * 8, (uint32_t)j * 256u + cbyte, 0u);
    }
  };
  float* const pt = sm.pt[wave];

  const int t0 = ch * a.tiles_per_chunk;
  const int t1 = t0 + a.tiles_per_chunk < a.ntiles ? t0 + a.tiles_per_chunk : a.ntiles;
  if (t0 < t1) issue_tile(t0, sm.kt[0], lane);
  // tile t0, the query operands and the row statistics have arrived
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  __syncthreads();
  int cur = 0;
  for (int T = t0; T < t1; ++T) {
    // Offsets derived from the lane index are recomputed in every tile (a few
    // integer operations) from an opaque copy of it, rather than held in
    // registers across the loop: at four waves per SIMD the registers are full.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lg = ln >> 5;
    const int lr = ln & 31;
    // tile T + 1 into the buffer tile T - 1 used (every wave left it at the last barrier)
    if (T + 1 < t1) issue_tile(T + 1, sm.kt[cur ^ 1], ln);
    const char* ktc = (const char*)sm.kt[cur];
    const int par = (T - t0) & 1;
    // the causal mask only bites in tiles that reach past the first last-query row
    const bool edge = (int64_t)T * kBlock + kBlock - 1 > (int64_t)n - r;
    // every row present and the tile below the causal edge: nothing is masked
    const bool plain = !edge && r == 64;
    float cs[2] = {0.f, 0.f};
    // the tile's probabilities, column sums and diagonal chain sums; PLAIN:
    // nothing of the tile is masked (a separate copy of the code, so that the
    // common case carries no per-element test)
    f32x16 sc[2];
    auto tile_probs = [&](auto plain_c) {
      constexpr bool PLAIN = decltype(plain_c)::value;
      // chain sum of block (mk, a): row u = 2 a + g, column 32 mk + r32 - 4 u + 28
      float* const pw = pt + lg * (PSTR - 4) + lr + 28;
      // carries of block (mk, a) (lanes r32 = 15, 31): row 8 + (a >> 1), columns
      // 32 mk + r32 + 29 - 4 u (chain step 2), + 1 (step 1), + 2 (step 0)
      float* const pc = pt + 8 * PSTR + lr + 29 - 4 * lg;
      const bool carry_lane = (lr & 15) == 15;
      // in edge tiles key slot c is visible to row t iff c - t <= n - r - 64 T
      const int dlim = n - r - T * kBlock;
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 cr = lds_f32x4(&sm.crow[hw][32 * mq + 8 * a4 + 4 * lg]);
        float carry[2][3];
#pragma unroll
        for (int mk = 0; mk < 2; ++mk) {
          float pv[4];
#pragma unroll
          for (int b4 = 0; b4 < 4; ++b4) {
            const int t = 32 * mq + 8 * a4 + 4 * lg + b4;
            const int c = 32 * mk + lr;
            float p = fast_exp2(fmaf(sc[mk][4 * a4 + b4], sl2, -cr[b4]));
            if (!PLAIN) p = (t < r && (!edge || c - t <= dlim)) ? p : 0.f;
            cs[mk] += p;
            pv[b4] = p;
          }
          const float x0 = pv[0];
          const float x1 = pv[1] + row_shr1(x0);
          const float x2 = pv[2] + row_shr1(x1);
          const float x3 = pv[3] + row_shr1(x2);
          pw[a4 * (2 * PSTR - 8) + 32 * mk] = x3;
          carry[mk][0] = x2;
          carry[mk][1] = x1;
          carry[mk][2] = x0;
        }
        if (carry_lane) {
#pragma unroll
          for (int mk = 0; mk < 2; ++mk)
#pragma unroll
            for (int k = 0; k < 3; ++k) pc[(a4 >> 1) * PSTR + 32 * mk - 8 * a4 + k] = carry[mk][k];
        }
        // one group of four query rows at a time (keeps the live probabilities few)
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (active) {
      // operand reads: row x = 32 mk + lr, chunk 2 ks + lg
      const int kofs = lr * 256 + ((lg ^ swz(lr)) << 4);
#pragma unroll
      for (int mk = 0; mk < 2; ++mk) {
        sc[mk] = f32x16{};
        const char* kp = ktc + 32 * mk * 256;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) sc[mk] = mfma32(qr[ks], *(const u32x4*)(kp + (kofs ^ (ks << 5))), sc[mk]);
      }
      if (plain)
        tile_probs(std::true_type{});
      else
        tile_probs(std::false_type{});
    }
    // pt is private to the wave and a wave's LDS accesses complete in order:
    // no workgroup barrier around its staging
    __builtin_amdgcn_wave_barrier();
    if (active) {
      float* pa = sm.pacc[par][hw] + mq * PCOLS;
      const float* pr = pt + ln;
      float a0 = 0.f;
#pragma unroll
      for (int row = 0; row < PROWS; ++row) a0 += pr[row * PSTR];
      pa[ln] = a0;
      if (ln < 32) {
        float a1 = 0.f;
#pragma unroll
        for (int row = 0; row < PROWS; ++row) a1 += pr[row * PSTR + 64];
        pa[64 + ln] = a1;
      }
      // the other half-wave holds the same keys' other four query rows of each group
      cs[0] += __shfl_xor(cs[0], 32);
      cs[1] += __shfl_xor(cs[1], 32);
      sm.csum[par][hw][mq][ln] = lg ? cs[1] : cs[0];
    }
    __builtin_amdgcn_wave_barrier();  // the next tile's rows overwrite pt
    // tile T + 1 landed; one barrier: it is visible to every wave, tile T released,
    // and both halves of every head have left their sums of tile T
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    __syncthreads();
    if (active && mq == 0) {
      const int64_t j = (int64_t)T * kBlock + ln;
      if (j < n) a.vcol[(size_t)slot * n + j] = sm.csum[par][hw][0][ln] + sm.csum[par][hw][1][ln];
      // diagonal e = t - c + 63 sits in column 94 - e of query rows 0..31 and in
      // column 126 - e of rows 32..63; lane l takes diagonals l and l + 64 (127 has no entries)
      const float* pa = sm.pacc[par][hw];
      float dd[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int e = ln + 64 * u;
        float x = 0.f;
        if (e <= 94) x += pa[94 - e];
        if (e >= 31 && e <= 126) x += pa[PCOLS + 126 - e];
        dd[u] = x;
      }
      // Tile T holds diagonal dl = base + e, base = n - r - 64 T - 63. Its
      // diagonals e = 64 + l (l <= 62) are the diagonals e = l of tile T - 1,
      // which are summed first; e = 63 is in no other tile. Pairs inside the
      // chunk are completed here, pairs across a chunk edge go to the edge
      // buffer (lo: the chunk's last tile, hi: its first) and are added by
      // vs_diag_edge_kernel; at the ends of the row a diagonal has one tile.
      const int64_t base = (int64_t)n - r - (int64_t)T * kBlock - 63;
      float* sl = a.slsum + (size_t)slot * n;
      float* edge = a.dedge + ((size_t)slot * a.nchunks + ch) * 128;
      if (ln == 63) {
        if (base + 63 >= 0 && base + 63 < n) sl[base + 63] = 0.f + dd[0];
      } else {
        const int64_t dh = base + 64 + ln;  // diagonal e = 64 + ln of this tile
        if (T > t0) {
          // written by this lane at the previous tile (a wave's LDS accesses complete in order)
          if (dh >= 0 && dh < n) sl[dh] = (0.f + sm.dkeep[hw][ln]) + dd[1];
        } else if (T == 0) {
          if (dh >= 0 && dh < n) sl[dh] = 0.f + dd[1];
        } else {
          edge[64 + ln] = dd[1];
        }
        if (T == t1 - 1) {
          if (T == a.ntiles - 1) {
            const int64_t dlo = base + ln;
            if (dlo >= 0 && dlo < n) sl[dlo] = 0.f + dd[0];
          } else {
            edge[ln] = dd[0];
          }
        }
        sm.dkeep[hw][ln] = dd[0];
      }
    }
    cur ^= 1;
  }
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

// Diagonals that straddle two chunks of tiles: dl = base(t0) + 64 + l is
// e = l of tile t0 - 1 (the previous chunk's last tile) and e = 64 + l of
// tile t0 (this chunk's first), added in tile order.
__global__ __launch_bounds__(64) void vs_diag_edge_kernel(const VsLaunch a) {
  const int slot = blockIdx.y;
  const int c = blockIdx.x + 1;  // chunk whose first tile closes the pair
  const int l = threadIdx.x;
  if (l > 62) return;
  const int t0 = c * a.tiles_per_chunk;
  if (t0 >= a.ntiles) return;
  const int64_t dl = (int64_t)a.n - a.r - (int64_t)t0 * kBlock - 63 + 64 + l;
  if (dl < 0 || dl >= a.n) return;
  const float* prev = a.dedge + ((size_t)slot * a.nchunks + (c - 1)) * 128;
  const float* cur = a.dedge + ((size_t)slot * a.nchunks + c) * 128;
  a.slsum[(size_t)slot * a.n + dl] = (0.f + prev[l]) + cur[64 + l];
}

// Top-k of each row of a float matrix, ascending indices, ties to the lower index.
}  // namespace

hipError_t launch_vs_scores(const VsLaunch& a, hipStream_t stream) {
  dim3 grid(a.nchunks, a.ngroups);
  hipLaunchKernelGGL(vs_pass1_kernel, grid, dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(vs_row_combine_kernel, dim3(64, a.n_slots), dim3(64), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(vs_pass2_kernel, grid, dim3(kThreads2), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.nchunks > 1) hipLaunchKernelGGL(vs_diag_edge_kernel, dim3(a.nchunks - 1, a.n_slots), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace minf
