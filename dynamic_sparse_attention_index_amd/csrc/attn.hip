// Sparse and dense causal FlashAttention for gfx950 (CDNA4).
//
// What is computed ("Latency and sparse patterns in kernels", Fig. 4 of the
// MInference 1.0 article; blockwise sparse computation on top of
// FlashAttention in the talk transcript's MInference part): for every query
// row, softmax attention restricted to the key set its head's plan selects,
// with slash lines covered by whole 64x64 key blocks and vertical lines
// computed as gathered single key columns, using the online-softmax
// recurrence across key tiles.
//
// Work decomposition (MI355X-first, not the pages' Triton/PIT layout):
//  * one workgroup = 4 wave64s = one head and a PAIR of adjacent query blocks
//    (b0 = 2p, b1 = 2p + 1), 128 query rows. Waves 0-1 own the 64 rows of b0,
//    waves 2-3 those of b1, 32 rows per wave.
//  * the workgroup walks the UNION of the two blocks' key tiles; each K/V tile
//    is staged once in LDS and used by every wave whose block selects it, so
//    one HBM/L2 read of a tile feeds up to 128 query rows.
//  * products run on 32x32x16 bf16 MFMA in transposed form: S^T = K Q^T and
//    O^T = V^T P^T, so a lane owns one query row in both the score and the
//    output accumulators and the online-softmax rescale is lane-local.
//  * V is transposed while it is staged (global row-major -> LDS [d][key])
//    with the key order inside each 16-key step permuted to match the score
//    accumulator's row order, so P goes from accumulator to MFMA operand
//    without any cross-lane movement.
//  * K/V tiles are double-buffered in LDS; the next tile's global loads are in
//    flight while the current tile is computed (one barrier per tile).
#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kThreads = 256;
constexpr int KSTR = 136;  // halves per K row in LDS (128 + 8 pad: conflict-free 16-byte reads)
constexpr int VSTR = 72;   // halves per V^T row in LDS (64 keys + 8 pad)
constexpr int kBitWords = (kMaxTokens / kBlock) / 32 + 1;  // 513 words per bitmap
constexpr int kColChunk = 1024;  // candidate vertical columns compacted per round

struct Smem {
  uint16_t kt[2][kBlock * KSTR];
  uint16_t vt[2][kHeadDim * VSTR];
  uint32_t bits[2][kBitWords];
  uint32_t clist[kColChunk];
  int scan[16];
};

enum : int { KIND_DENSE = 0, KIND_ASHAPE = 1, KIND_VS = 2, KIND_BLOCK = 3 };

__device__ __forceinline__ uint32_t bit_at(const uint32_t* w, int v) { return (w[v >> 5] >> (v & 31)) & 1u; }

// Tile sequence over the key blocks of the pair (b0, b1). Every thread runs
// the same sequence (it only reads kernel arguments and LDS).
struct BlockIter {
  int kind, b0, b1, has_b1, nb, causal;
  int c, cmax;         // dense / A-shape cursor
  int sb, wlo0, wlo1;  // A-shape
  int w, wmax, base;   // VS / BLOCK bitmap cursor
  uint32_t rem;
  // BLOCK: membership bitmaps over key blocks c of b0 and b1.
  // VS: block-offset bitmaps of b0 and b1 (they differ only for a partial last block).
  const uint32_t* bits0;
  const uint32_t* bits1;

  __device__ uint32_t union_word(int ww) const {
    if (kind == KIND_VS) {
      uint32_t bw = bits0[ww];
      uint32_t prev = ww > 0 ? bits0[ww - 1] : 0u;
      uint32_t u = (bw << 1) | (prev >> 31);  // offsets v with v - 1 in b0's set
      if (has_b1) u |= bits1[ww];             // offsets v in b1's set
      return u;
    }
    return bits0[ww] | bits1[ww];
  }

  __device__ void init_bitmap_cursor(int vmax) {
    wmax = vmax >> 5;
    w = 0;
    uint32_t u = union_word(0);
    if (wmax == 0) u &= (vmax & 31) == 31 ? 0xffffffffu : ((1u << ((vmax & 31) + 1)) - 1u);
    rem = u;
  }

  // Next tile: key block c and membership (bit 0: block b0 uses it, bit 1: b1).
  __device__ bool next(int& cout, int& mem) {
    if (kind == KIND_DENSE) {
      if (c > cmax) return false;
      cout = c;
      mem = causal ? ((c <= b0) | ((has_b1 && c <= b1) << 1)) : (1 | (has_b1 << 1));
      ++c;
      return true;
    }
    if (kind == KIND_ASHAPE) {
      while (c <= cmax) {
        int cc = c;
        int m0 = (cc <= b0) && (cc < sb || cc >= wlo0);
        int m1 = has_b1 && (cc <= b1) && (cc < sb || cc >= wlo1);
        c = (cc + 1 >= sb && cc + 1 < wlo0) ? wlo0 : cc + 1;
        if (m0 | m1) {
          cout = cc;
          mem = m0 | (m1 << 1);
          return true;
        }
      }
      return false;
    }
    // bitmap kinds: iterate set bits of the union word by word
    while (rem == 0u) {
      if (++w > wmax) return false;
      uint32_t u = union_word(w);
      if (w == wmax) {
        int top = (kind == KIND_VS ? base : cmax) & 31;
        u &= top == 31 ? 0xffffffffu : ((1u << (top + 1)) - 1u);
      }
      rem = u;
    }
    int v = (w << 5) + __builtin_ctz(rem);
    rem &= rem - 1u;
    if (kind == KIND_VS) {
      // v is a block offset measured from b0 + 1: key block c = b0 + 1 - v
      cout = base - v;
      int m1 = has_b1 && bit_at(bits1, v);
      int m0 = v >= 1 && bit_at(bits0, v - 1);
      mem = m0 | (m1 << 1);
    } else {
      cout = v;
      mem = (int)bit_at(bits0, v) | ((int)bit_at(bits1, v) << 1);
    }
    return true;
  }
};

struct TileRegs {
  u32x4 k[4];
  u32x4 v[4];
};

// Global -> registers for one K/V tile. Rows come from `rows_of(x)`, x in [0, 64):
// the key index, or -1 for a padding row (loaded as zeros).
template <class RowFn>
__device__ __forceinline__ void load_tile(TileRegs& R, const uint16_t* kh, const uint16_t* vh, RowFn rows_of) {
  const int tid = threadIdx.x;
  // K: 16 threads per row, 16 rows per pass
  const int kdc = tid & 15;
  const int krow = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int j = rows_of(krow + 16 * i);
    R.k[i] = j >= 0 ? *(const u32x4*)(kh + (size_t)j * kHeadDim + 8 * kdc) : u32x4{0, 0, 0, 0};
  }
  // V: thread owns keys 4*kq .. 4*kq+3 and dims 8*dc .. 8*dc+7
  const int kq = tid & 15;
  const int dc = tid >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int j = rows_of(4 * kq + r);
    R.v[r] = j >= 0 ? *(const u32x4*)(vh + (size_t)j * kHeadDim + 8 * dc) : u32x4{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void store_tile(const TileRegs& R, uint16_t* kt, uint16_t* vt) {
  const int tid = threadIdx.x;
  const int kdc = tid & 15;
  const int krow = tid >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) *(u32x4*)(kt + (krow + 16 * i) * KSTR + 8 * kdc) = R.k[i];
  const int kq = tid & 15;
  const int dc = tid >> 4;
  // keys 4kq..4kq+3 land at permuted positions: bits 2 and 3 of the key swapped
  const int pos = 16 * (kq >> 2) + ((kq & 1) << 3) + ((kq & 2) << 1);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int wsel = e >> 1;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint32_t lo = __builtin_amdgcn_perm(R.v[1][wsel], R.v[0][wsel], sel);
    uint32_t hi = __builtin_amdgcn_perm(R.v[3][wsel], R.v[2][wsel], sel);
    *(u32x2*)(vt + (8 * dc + e) * VSTR + pos) = u32x2{lo, hi};
  }
}

struct WaveState {
  u32x4 qr[8];     // this wave's 32 query rows as MFMA B operands (8 k-steps over d)
  f32x16 o[4];     // O^T accumulators: d = 32*mt + ..., column = query row
  float m, l;      // running max (log2 units) and this lane's partial sum
};

// One tile for one wave. mode: 0 = all visible, 1 = element predicate.
// Predicate: key j visible for row i iff j <= i (causal) or j < n (non-causal),
// plus the A-shape clause, plus (gather tiles) the column's membership flag.
template <bool GATHER>
__device__ __forceinline__ void compute_tile(WaveState& ws, const uint16_t* kt, const uint16_t* vt, int mode,
                                             int key0, const uint32_t* gcols, int qsel, int row, int n,
                                             int causal, int ashape, int sink, int local, float sl2) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int r32 = lane & 31;
  f32x16 s[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    s[mt] = f32x16{};
    const uint16_t* kp = kt + (32 * mt + r32) * KSTR + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 a = *(const u32x4*)(kp + 16 * ks);
      s[mt] = mfma32(a, ws.qr[ks], s[mt]);
    }
  }
  if (mode) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kx = 32 * mt + 8 * (i >> 2) + 4 * g + (i & 3);  // key slot in the tile
        int j;
        bool vis;
        if (GATHER) {
          uint32_t e = gcols[kx];
          j = (int)(e & 0x3fffffffu);
          vis = ((e >> (30 + qsel)) & 1u) && j <= row;
        } else {
          j = key0 + kx;
          vis = causal ? (j <= row) : (j < n);
          if (ashape) vis = vis && (j < sink || row - j < local);
        }
        if (!vis) s[mt][i] = -INFINITY;
      }
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[mt][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(ws.m, mx * sl2);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = fast_exp2(ws.m - m_use);
  float psum = 0.f;
  u32x4 pk[4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(s[mt][8 * h + e], sl2, -m_use));
        psum += p[e];
      }
      pk[2 * mt + h] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                             pack_bf16x2(p[6], p[7])};
    }
  }
  ws.l = ws.l * alpha + psum;
  ws.m = m_new;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) ws.o[mt] *= alpha;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const uint16_t* vp = vt + (32 * mt + r32) * VSTR + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4 a = *(const u32x4*)(vp + 16 * kk);
      ws.o[mt] = mfma32(a, pk[kk], ws.o[mt]);
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void attn_kernel(const AttnLaunch p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int npairs = (p.nb + 1) >> 1;
  const int item = blockIdx.x;
  if (item >= npairs * p.nh) return;
  const int hl = item % p.nh;
  const int pr = npairs - 1 - item / p.nh;  // heaviest (latest) pairs first
  const int h = p.head0 + hl;
  const int kvh = h / p.grp;
  const AttnHead hd = p.heads[hl];
  const int n = p.n;
  const int b0 = 2 * pr;
  const int b1 = b0 + 1;
  const int has_b1 = b1 < p.nb;
  const int qsel = wave >> 1;
  const int qb = qsel ? b1 : b0;
  const bool wave_on = qsel == 0 || has_b1;
  const int row = qb * kBlock + (wave & 1) * 32 + (lane & 31);
  const float sl2 = p.scale_log2;

  const uint16_t* kh = p.k + (size_t)kvh * n * kHeadDim;
  const uint16_t* vh = p.v + (size_t)kvh * n * kHeadDim;

  WaveState ws;
  {
    const int rr = row < n ? row : n - 1;
    const uint16_t* qp = p.q + ((size_t)h * n + rr) * kHeadDim + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      ws.qr[ks] = (row < n && wave_on) ? *(const u32x4*)(qp + 16 * ks) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ws.o[mt] = f32x16{};
    ws.m = -INFINITY;
    ws.l = 0.f;
  }

  // ---------------- tile sequence set-up
  BlockIter it;
  it.kind = hd.kind;
  it.b0 = b0;
  it.b1 = b1;
  it.has_b1 = has_b1;
  it.nb = p.nb;
  it.causal = p.causal;
  it.bits0 = sm.bits[0];
  it.bits1 = sm.bits[1];
  it.rem = 0;
  it.w = 0;
  it.wmax = -1;
  const int bmax = has_b1 ? b1 : b0;
  if (hd.kind == KIND_DENSE) {
    it.c = 0;
    it.cmax = p.causal ? bmax : p.nb - 1;
  } else if (hd.kind == KIND_ASHAPE) {
    it.c = 0;
    it.cmax = bmax;
    int sbk = (int)(((int64_t)hd.sink + kBlock - 1) / kBlock);
    it.sb = sbk < p.nb ? sbk : p.nb;
    auto wlo = [&](int b) -> int {
      if (hd.local <= 0) return b + 1;
      int64_t lo = (int64_t)b * kBlock - hd.local + 1;
      return lo <= 0 ? 0 : (int)(lo / kBlock);
    };
    it.wlo0 = wlo(b0);
    it.wlo1 = wlo(b1);
    if (0 >= it.sb && 0 < it.wlo0) it.c = it.wlo0;
  } else if (hd.kind == KIND_VS) {
    // offset bitmap of full blocks, and (when n % 64 != 0) of the partial last block
    const int nwords = (p.nb >> 5) + 1;
    const int last_partial = (n & (kBlock - 1)) != 0;
    const int need_last = last_partial && bmax == p.nb - 1;
    for (int i = tid; i < nwords; i += kThreads) {
      sm.bits[0][i] = hd.obits[i];
      if (need_last) sm.bits[1][i] = hd.obits[nwords + i];
    }
    __syncthreads();
    it.bits0 = (need_last && b0 == p.nb - 1) ? sm.bits[1] : sm.bits[0];
    it.bits1 = (need_last && b1 == p.nb - 1) ? sm.bits[1] : sm.bits[0];
    it.base = b0 + 1;
    it.init_bitmap_cursor(it.base);
  } else {  // KIND_BLOCK
    const int nwords = (bmax >> 5) + 1;
    for (int i = tid; i < nwords; i += kThreads) {
      sm.bits[0][i] = 0u;
      sm.bits[1][i] = 0u;
    }
    __syncthreads();
    const int kb = hd.k_b;
    for (int x = tid; x < 2 * kb; x += kThreads) {
      const int which = x >= kb;
      const int b = which ? b1 : b0;
      if (which && !has_b1) continue;
      const int cnt = hd.blk_cnt[b];
      const int e = x - which * kb;
      if (e < cnt) {
        int c = hd.blk_idx[(size_t)b * kb + e];
        if (c >= 0 && c <= b) atomicOr(&sm.bits[which][c >> 5], 1u << (c & 31));
      }
    }
    __syncthreads();
    it.cmax = bmax;
    it.init_bitmap_cursor(bmax);
  }
  const int ashape = hd.kind == KIND_ASHAPE;

  // ---------------- phase A: 64x64 key blocks
  {
    TileRegs R;
    int c_cur = 0, m_cur = 0, c_nxt = 0, m_nxt = 0;
    bool have = it.next(c_cur, m_cur);
    if (have) {
      load_tile(R, kh, vh, [&](int x) { int j = c_cur * kBlock + x; return j < n ? j : -1; });
      store_tile(R, sm.kt[0], sm.vt[0]);
    }
    __syncthreads();
    int buf = 0;
    while (have) {
      const bool hn = it.next(c_nxt, m_nxt);
      if (hn) load_tile(R, kh, vh, [&](int x) { int j = c_nxt * kBlock + x; return j < n ? j : -1; });
      if (wave_on && ((m_cur >> qsel) & 1)) {
        int full;
        if (p.causal || hd.kind != KIND_DENSE) {
          full = c_cur < qb;
          if (ashape && full)
            full = ((int64_t)c_cur * kBlock + kBlock - 1 < hd.sink) ||
                   ((int64_t)qb * kBlock + kBlock - 1 - (int64_t)c_cur * kBlock < hd.local);
        } else {
          full = (c_cur + 1) * kBlock <= n;
        }
        compute_tile<false>(ws, sm.kt[buf], sm.vt[buf], !full, c_cur * kBlock, nullptr, qsel, row, n,
                            p.causal || hd.kind != KIND_DENSE, ashape, hd.sink, hd.local, sl2);
      }
      if (hn) store_tile(R, sm.kt[buf ^ 1], sm.vt[buf ^ 1]);
      __syncthreads();
      c_cur = c_nxt;
      m_cur = m_nxt;
      have = hn;
      buf ^= 1;
    }
  }

  // ---------------- phase B: gathered vertical columns (VS heads)
  if (hd.kind == KIND_VS && hd.k_v > 0) {
    const int lim = bmax * kBlock + kBlock - 1;  // last row of the pair
    for (int base = 0; base < hd.k_v; base += kColChunk) {
      // compact this chunk's kept columns (ascending) into clist, with membership bits
      int kept_before = 0;
      bool past = false;
      for (int r = 0; r < kColChunk / kThreads; ++r) {
        const int e = base + r * kThreads + tid;
        uint32_t entry = 0;
        bool keep = false;
        if (e < hd.k_v) {
          const int j = hd.v_idx[e];
          const int prev = e > 0 ? hd.v_idx[e - 1] : -1;
          if (j > lim) past = true;
          if (j >= 0 && j < n && j <= lim && j != prev) {
            const int cb = j / kBlock;
            const int m0 = cb <= b0 && !bit_at(it.bits0, b0 - cb);
            const int m1 = has_b1 && cb <= b1 && !bit_at(it.bits1, b1 - cb);
            keep = m0 | m1;
            entry = (uint32_t)j | ((uint32_t)m0 << 30) | ((uint32_t)m1 << 31);
          }
        }
        int tot;
        const int pos = block_excl_scan_count<kThreads>(keep, sm.scan, tot);
        if (keep) sm.clist[kept_before + pos] = entry;
        kept_before += tot;
      }
      const int any_past = __syncthreads_or(past);
      const int kept = kept_before;
      const int ntile = (kept + kBlock - 1) / kBlock;
      for (int s = kept + tid; s < ntile * kBlock; s += kThreads) sm.clist[s] = 0u;  // padding: no member
      __syncthreads();
      if (ntile > 0) {
        TileRegs R;
        auto rows_of = [&](int t) {
          return [&, t](int x) -> int {
            const int s = t * kBlock + x;
            return s < kept ? (int)(sm.clist[s] & 0x3fffffffu) : -1;
          };
        };
        load_tile(R, kh, vh, rows_of(0));
        store_tile(R, sm.kt[0], sm.vt[0]);
        __syncthreads();
        int buf = 0;
        for (int t = 0; t < ntile; ++t) {
          const bool hn = t + 1 < ntile;
          if (hn) load_tile(R, kh, vh, rows_of(t + 1));
          if (wave_on) {
            // skip the tile when none of its columns belongs to this wave's query block
            // (padding slots were cleared, so they never count)
            const uint32_t* gc = sm.clist + t * kBlock;
            if (__any((gc[lane] >> (30 + qsel)) & 1u))
              compute_tile<true>(ws, sm.kt[buf], sm.vt[buf], 1, 0, gc, qsel, row, n, 1, 0, 0, 0, sl2);
          }
          if (hn) store_tile(R, sm.kt[buf ^ 1], sm.vt[buf ^ 1]);
          __syncthreads();
          buf ^= 1;
        }
      }
      if (any_past) break;
    }
  }

  // ---------------- finalize
  if (!wave_on) return;
  const float ltot = ws.l + __shfl_xor(ws.l, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (row < n) {
    const int g = lane >> 5;
    uint16_t* op = p.o + ((size_t)h * n + row) * kHeadDim + 4 * g;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 w = u32x2{pack_bf16x2(ws.o[mt][4 * q4] * inv, ws.o[mt][4 * q4 + 1] * inv),
                        pack_bf16x2(ws.o[mt][4 * q4 + 2] * inv, ws.o[mt][4 * q4 + 3] * inv)};
        *(u32x2*)(op + 32 * mt + 8 * q4) = w;
      }
    }
    if (p.lse && g == 0) {
      p.lse[(size_t)h * n + row] = ltot > 0.f ? (ws.m + __log2f(ltot)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

// Block offsets covered by a VS head's slash lines. For a full query block b,
// offset dl = 64q + rho (0 <= rho < 64) meets key block b - q (rows with
// t >= rho) and, when rho > 0, key block b - q - 1 (rows with t < rho); so
// bit o is set iff floor(dl/64) == o or ceil(dl/64) == o, and block b
// computes key blocks b - o for every set o <= b. A partial last block has
// rows t <= tmax only: there b - q is met only when rho <= tmax. The second
// bitmap (written after the first when n % 64 != 0) holds that case.
struct OffBitsLaunch {
  const int32_t* s_idx[kMaxLaunchHeads];
  int32_t k_s[kMaxLaunchHeads];
  uint32_t* bits[kMaxLaunchHeads];
  int32_t n, nb;
};

__global__ __launch_bounds__(256) void vs_offset_bits_kernel(const OffBitsLaunch a) {
  __shared__ uint32_t w[kBitWords];
  const int hsl = blockIdx.x;
  const int nwords = (a.nb >> 5) + 1;
  const int tmax = (a.n - 1) & (kBlock - 1);
  const int partial = (a.n & (kBlock - 1)) != 0;
  for (int pass = 0; pass <= partial; ++pass) {
    for (int i = threadIdx.x; i < nwords; i += 256) w[i] = 0u;
    __syncthreads();
    const int32_t* s = a.s_idx[hsl];
    for (int e = threadIdx.x; e < a.k_s[hsl]; e += 256) {
      const int dl = s[e];
      if (dl < 0 || dl >= a.n) continue;
      const int q = dl >> 6;
      const int rho = dl & (kBlock - 1);
      if (pass == 0 || rho <= tmax) atomicOr(&w[q >> 5], 1u << (q & 31));
      if (rho > 0 && q + 1 < a.nb) atomicOr(&w[(q + 1) >> 5], 1u << ((q + 1) & 31));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nwords; i += 256) a.bits[hsl][pass * nwords + i] = w[i];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_attn(const AttnLaunch& a, hipStream_t stream) {
  const int npairs = (a.nb + 1) / 2;
  const long long items = (long long)npairs * a.nh;
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(attn_kernel, dim3((unsigned)items), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_vs_offset_bits(const int32_t* const* s_idx, const int32_t* k_s, uint32_t* const* bits,
                                 int count, int n, hipStream_t stream) {
  for (int base = 0; base < count; base += kMaxLaunchHeads) {
    OffBitsLaunch a{};
    const int c = count - base < kMaxLaunchHeads ? count - base : kMaxLaunchHeads;
    for (int i = 0; i < c; ++i) {
      a.s_idx[i] = s_idx[base + i];
      a.k_s[i] = k_s[base + i];
      a.bits[i] = bits[base + i];
    }
    a.n = n;
    a.nb = (n + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(vs_offset_bits_kernel, dim3(c), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace minf
