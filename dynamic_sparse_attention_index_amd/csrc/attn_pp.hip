// Sparse and dense causal FlashAttention for gfx950 with ping-pong waves.
//
// What is computed is the same as in attn.hip ("Latency and sparse patterns in
// kernels", Fig. 4 of the MInference 1.0 article; blockwise sparse computation
// on top of FlashAttention in the talk transcript's MInference part): per query
// row, softmax attention over the key set of its head's plan, slash lines as
// whole 64x64 key blocks and verticals as gathered key columns, with the
// online-softmax recurrence across key tiles.
//
// Why a second kernel: in the pair kernel each wave alternates between MFMA
// work (S = K Q^T, O^T += V^T P^T) and VALU work (mask, row max, exp, bf16
// packing), and the two waves that share a SIMD overlap the two only by
// chance. Here the overlap is arranged:
//  * one workgroup = 8 wave64s = one head and a QUAD of query blocks
//    b_i = 4 q + i (256 rows); waves i and i + 4 hold rows 0-31 and 32-63 of
//    block b_i and run on the same SIMD (wave w runs on SIMD w mod 4);
//  * each wave's work on key tile k is QK(k) and PV(k) on the matrix cores and
//    the softmax sm(k) on the vector ALUs; a step k runs PV(k - 1) + QK(k) and
//    a softmax, and waves 0-3 run [PV(k-1), QK(k)] then [sm(k)] while waves
//    4-7 run [sm(k-1)] then [PV(k-1), QK(k)], with a workgroup barrier
//    between the two halves: on every SIMD one wave drives the matrix core
//    while the other one does its softmax;
//  * K/V tiles live in a ring of four LDS buffers, filled with direct
//    HBM -> LDS loads two tiles ahead, so a load has two steps to land;
//  * the four query blocks walk the union of their key tiles in ascending
//    key order; a wave skips the tiles its block does not select. Block b_i
//    is on SIMD i, so a tile that block selects keeps both of that SIMD's
//    waves busy.
// Supported plans: dense (causal or not), A-shape, Vertical-Slash (block
// tiles and up to kColCap gathered columns per quad) and Block-Sparse
// without positions. Other launches use the pair kernel.
#include "common.h"
#include "launch.h"

namespace minf {
namespace {

constexpr int kPPThreads = 512;
constexpr int kQuad = 4;
constexpr int kXcds = 8;
constexpr int kChunk = 32;  // workgroups one XCD runs at once (32 CUs x 1)
constexpr int kTileHalves = kBlock * kHeadDim;
constexpr int kBitWords = (kMaxTokens / kBlock) / 32 + 1;
constexpr int kColCap = 2048;  // gathered vertical columns per quad

enum : int { KIND_DENSE = 0, KIND_ASHAPE = 1, KIND_VS = 2, KIND_BLOCK = 3 };
enum : int { M_NONE = 0, M_CAUSAL = 1, M_GENERAL = 2, M_GATHER = 3 };

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef short s16x4 __attribute__((ext_vector_type(4)));

struct PPSmem {
  // BLOCK: key blocks of b0..b3; VS: [0] offsets of full blocks, [1] of a partial last
  // block (one spare word: the VS cursor starts up to three offsets past the last block)
  uint32_t bits[kQuad][kBitWords + 1];
  uint32_t clist[kColCap];          // gathered columns: key j (bits 0-19), member of block b_i (bit 28 + i)
  int scan[kPPThreads / 64];
  int ncols;
};

// 16-byte chunk c of tile row r sits at chunk position c ^ swz(r) (conflict-free
// 16-row operand reads and 4-row transpose reads).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ int uniform_i32(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ void barrier() { __builtin_amdgcn_s_barrier(); }

// Per-lane LDS byte offsets of the MFMA operands inside a tile.
struct OperandOffsets {
  int k;        // K row r32, chunk (g ^ swz): chunk 2 ks + g of the row is at k ^ (ks << 5)
  int v[4][2];  // V transpose reads: d block mt, key half h (+ 4096 per 16-key step)
};

__device__ __forceinline__ OperandOffsets operand_offsets() {
  OperandOffsets o;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int r32 = lane & 31;
  o.k = r32 * 256 + ((g ^ swz(r32)) << 4);
  // ds_read_b64_tr_b16: source lane i of 16-lane group G supplies the 4 halves
  // V[kb + i/4][dbase + 4(i%4) ..]; lane i then receives V[kb + e][dbase + i], e = 0..3
  const int G = lane >> 4;
  const int i = lane & 15;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * h + 4 * g + (i >> 2);
      const int chunk = 4 * mt + 2 * (G & 1) + ((i >> 1) & 1);
      o.v[mt][h] = row * 256 + ((chunk ^ swz(row)) << 4) + 8 * (i & 1);
    }
  return o;
}

// Tile sequence over the key blocks of the quad. Every thread runs the same
// sequence (kernel arguments and LDS only), with the cursor kept in scalar
// registers. mem: bit i set when block b_i uses the tile.
struct QuadIter {
  int kind, bq, nblk, nb, causal;  // bq = b0; nblk = blocks of the quad that exist (1..4)
  int c, cmax;                     // dense / A-shape cursor
  int sb, wlo[kQuad];              // A-shape
  int w, wmax, base;               // VS / BLOCK bitmap cursor
  uint32_t rem;
  uint32_t mw[kQuad];              // membership of each block for the bits of the current word
  const uint32_t* bitsv[kQuad];    // VS: the offset bitmap block b_i uses; BLOCK: block b_i's key blocks

  __device__ uint32_t union_word(int ww) {
    uint32_t u = 0;
    if (kind == KIND_VS) {
      // offset v (key block c = b3 - v) is used by block b_i iff v - (3 - i) is one of its offsets
#pragma unroll
      for (int i = 0; i < kQuad; ++i) {
        const int sh = kQuad - 1 - i;
        uint32_t m = 0;
        if (i < nblk) {
          const uint32_t cur = uniform_u32(bitsv[i][ww]);
          const uint32_t prev = ww > 0 ? uniform_u32(bitsv[i][ww - 1]) : 0u;
          m = sh == 0 ? cur : ((cur << sh) | (prev >> (32 - sh)));
        }
        mw[i] = m;
        u |= m;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kQuad; ++i) {
        mw[i] = i < nblk ? uniform_u32(bitsv[i][ww]) : 0u;
        u |= mw[i];
      }
    }
    return u;
  }

  // VS walks offsets v downwards from vmax (key blocks ascending); BLOCK walks key blocks upwards.
  __device__ void init_bitmap_cursor(int vmax) {
    wmax = vmax >> 5;
    w = kind == KIND_VS ? wmax : 0;
    uint32_t u = union_word(w);
    if (w == wmax) u &= (vmax & 31) == 31 ? 0xffffffffu : ((1u << ((vmax & 31) + 1)) - 1u);
    rem = u;
  }

  __device__ bool next(int& cout, int& mem) {
    if (kind == KIND_DENSE) {
      if (c > cmax) return false;
      cout = c;
      int m = 0;
#pragma unroll
      for (int i = 0; i < kQuad; ++i) m |= (i < nblk && (!causal || c <= bq + i)) << i;
      mem = m;
      ++c;
      return true;
    }
    if (kind == KIND_ASHAPE) {
      while (c <= cmax) {
        const int cc = c;
        int m = 0, lo = wlo[kQuad - 1];
#pragma unroll
        for (int i = 0; i < kQuad; ++i) {
          m |= (i < nblk && cc <= bq + i && (cc < sb || cc >= wlo[i])) << i;
          lo = min(lo, wlo[i]);
        }
        c = (cc + 1 >= sb && cc + 1 < lo) ? lo : cc + 1;
        if (m) {
          cout = cc;
          mem = m;
          return true;
        }
      }
      return false;
    }
    if (kind == KIND_VS) {
      while (rem == 0u) {
        if (--w < 0) return false;
        rem = union_word(w);
      }
      const int bit = 31 - __builtin_clz(rem);
      rem ^= 1u << bit;
      const int v = (w << 5) + bit;
      cout = base - v;
      int m = 0;
#pragma unroll
      for (int i = 0; i < kQuad; ++i) m |= (int)((mw[i] >> bit) & 1u) << i;
      mem = m;
      return true;
    }
    while (rem == 0u) {
      if (++w > wmax) return false;
      uint32_t u = union_word(w);
      if (w == wmax) {
        const int top = cmax & 31;
        u &= top == 31 ? 0xffffffffu : ((1u << (top + 1)) - 1u);
      }
      rem = u;
    }
    const int bit = __builtin_ctz(rem);
    rem &= rem - 1u;
    cout = (w << 5) + bit;
    int m = 0;
#pragma unroll
    for (int i = 0; i < kQuad; ++i) m |= (int)((mw[i] >> bit) & 1u) << i;
    mem = m;
    return true;
  }
};

struct WaveState {
  u32x4 qr[8];  // this wave's 32 query rows as MFMA B operands
  f32x16 o[4];  // O^T accumulators
  f32x16 s[2];  // scores of the current tile (S^T = K Q^T), keys 0-31 / 32-63
  u32x4 pk[4];  // bf16 probabilities of the tile waiting for its PV product
  float m, l;   // running max (log2 units) and this lane's partial row sum
};

// S^T = K Q^T for one tile: two interleaved accumulation chains.
__device__ __forceinline__ void qk(WaveState& ws, const OperandOffsets& oo, const uint16_t* kt) {
  const char* kb = (const char*)kt;
  f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int ko = oo.k ^ (ks << 5);
    const u32x4 a0 = *(const u32x4*)(kb + ko);
    const u32x4 a1 = *(const u32x4*)(kb + ko + 32 * 256);
    s0 = mfma32(a0, ws.qr[ks], s0);
    s1 = mfma32(a1, ws.qr[ks], s1);
  }
  ws.s[0] = s0;
  ws.s[1] = s1;
}

// O^T += V^T P^T for one tile from the packed probabilities.
__device__ __forceinline__ void pv(WaveState& ws, const OperandOffsets& oo, const uint16_t* vt) {
  const char* vb = (const char*)vt;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)((lds_ptr)(vb + oo.v[mt][0] + 4096 * kk)));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)((lds_ptr)(vb + oo.v[mt][1] + 4096 * kk)));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
      const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
      ws.o[mt] = mfma32(u32x4{l2[0], l2[1], h2[0], h2[1]}, ws.pk[kk], ws.o[mt]);
    }
  }
}

// Softmax of the current tile: mask, running max, rescale of O when the max
// rises (exact running max: the dominant probability stays exactly 1.0 in
// bf16), probabilities packed to bf16 for the PV product, row sum of those
// bf16 values. mask: M_*; key0 = first key of the tile; gcols: gathered
// columns' entries (M_GATHER); row = this lane's query row.
__device__ __forceinline__ void softmax(WaveState& ws, int mask, int key0, const uint32_t* gcols, int qsel,
                                        int row, int n, int causal, int ashape, int sink, int local, float sl2) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  f32x16* s = ws.s;
  if (mask == M_CAUSAL) {
    const int lim = row - key0 - 4 * g;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kx0 = 32 * mt + 8 * (i >> 2) + (i & 3);
        s[mt][i] = kx0 <= lim ? s[mt][i] : -INFINITY;
      }
  } else if (mask == M_GENERAL) {
    const int base = key0 + 4 * g;
    const int hi = causal ? row - base : n - 1 - base;
    const int lo_sink = ashape ? sink - base : 1 << 30;
    const int lo_win = ashape ? row - local - base : -(1 << 30);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kx0 = 32 * mt + 8 * (i >> 2) + (i & 3);
        const bool vis = kx0 <= hi && (kx0 < lo_sink || kx0 > lo_win);
        s[mt][i] = vis ? s[mt][i] : -INFINITY;
      }
  } else if (mask == M_GATHER) {
    const uint32_t sh = 28 + qsel;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x4 e4 = *(const u32x4*)(gcols + 32 * mt + 8 * q4 + 4 * g);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t e = e4[t];
          const bool vis = ((e >> sh) & 1u) && (int)(e & 0xfffffu) <= row;
          s[mt][4 * q4 + t] = vis ? s[mt][4 * q4 + t] : -INFINITY;
        }
      }
  }
  float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[0][i], s[1][i]));
  const float m_tile = pair_max32(mx) * sl2;
  if (__any(m_tile > ws.m)) {
    const float m_new = fmaxf(ws.m, m_tile);
    float alpha = fast_exp2(ws.m - (m_new == -INFINITY ? 0.f : m_new));
    asm volatile("" : "+v"(alpha));  // keeps the rescale a real branch
    ws.l *= alpha;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) ws.o[mt] *= alpha;
    ws.m = m_new;
  }
  const float m_use = ws.m == -INFINITY ? 0.f : ws.m;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(s[mt][8 * h + e], sl2, -m_use));
      ws.pk[2 * mt + h] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                pack_bf16x2(p[6], p[7])};
    }
  }
  float psum = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int w = 0; w < 4; ++w) psum = sum_bf16x2(ws.pk[kk][w], psum);
  ws.l += psum;
}

// One tile of the sequence: key block c (or, for gathered tiles, the index of
// the 64-column group in clist), the blocks using it, and whether it is gathered.
struct TileRef {
  int c, mem, gath;
};

// The key row of tile row x (always a valid row).
__device__ __forceinline__ int tile_key_row(const TileRef& t, int x, int n, const uint32_t* clist, int ncols) {
  if (t.gath) {
    const int s = 64 * t.c + x;
    return s < ncols ? (int)(clist[s] & 0xfffffu) : 0;
  }
  const int j = t.c * kBlock + x;
  return j < n ? j : n - 1;
}

// Direct HBM -> LDS copy of one K/V tile: wave w's instruction i fills LDS
// chunks [512 i + 64 w, +64) = rows 32 i + 4 w .. +3, 16 lanes per row.
__device__ __forceinline__ void issue_tile(const TileRef& t, const uint16_t* kh, const uint16_t* vh, uint16_t* kt,
                                           uint16_t* vt, int n, const uint32_t* clist, int ncols) {
  const int wave = wave_index();
  const int lane = threadIdx.x & 63;
  const int rlo = 4 * (threadIdx.x >> 6) + (lane >> 4);
  const uint32_t cb = (uint32_t)((((lane & 15) ^ swz(rlo)) * 16));
  if (!t.gath && (t.c + 1) * kBlock <= n) {
    const size_t base = (size_t)t.c * kBlock * (kHeadDim * 2);
    const char* kb = (const char*)kh + base;
    const char* vb = (const char*)vh + base;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off = (uint32_t)(32 * i + rlo) * 256u + cb;
      __builtin_amdgcn_global_load_lds(kb + off, (lds_ptr)(kt + (512 * i + 64 * wave) * 8), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(vb + off, (lds_ptr)(vt + (512 * i + 64 * wave) * 8), 16, 0, 0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t off = (uint32_t)tile_key_row(t, 32 * i + rlo, n, clist, ncols) * 256u + cb;
      __builtin_amdgcn_global_load_lds((const char*)kh + off, (lds_ptr)(kt + (512 * i + 64 * wave) * 8), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const char*)vh + off, (lds_ptr)(vt + (512 * i + 64 * wave) * 8), 16, 0, 0);
    }
  }
}

// vmcnt(N) with expcnt and lgkmcnt at their maxima (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

struct ItemCtx {
  const uint16_t* kh;
  const uint16_t* vh;
  int n, causal, ashape, sink, local, qsel, row, rmin, qb;
  float sl2;
};

// Mask of tile t for the wave's block qb.
__device__ __forceinline__ int tile_mask(const TileRef& t, const ItemCtx& cx) {
  if (t.gath) return M_GATHER;
  if (cx.causal) {
    bool full = t.c < cx.qb;
    if (cx.ashape && full)
      full = ((int64_t)t.c * kBlock + kBlock - 1 < cx.sink) ||
             ((int64_t)cx.qb * kBlock + kBlock - 1 - (int64_t)t.c * kBlock < cx.local);
    return full ? M_NONE : (cx.ashape ? M_GENERAL : M_CAUSAL);
  }
  return (t.c + 1) * kBlock <= cx.n ? M_NONE : M_GENERAL;
}

// The work item: head h, quad q.
__device__ __forceinline__ void pp_item(const AttnLaunch& p, int item, PPSmem& sm, uint16_t* k0, uint16_t* k1, uint16_t* k2,
                        uint16_t* k3, uint16_t* v0, uint16_t* v1, uint16_t* v2, uint16_t* v3) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int nq = (p.nb + kQuad - 1) / kQuad;
  const int hg = p.hgroup;
  const int qpc = kChunk / hg;                 // quads per chunk
  const int nqb = (nq + qpc - 1) / qpc;        // quad blocks
  const int nhg = p.nh / hg;
  const int chunk = item / kChunk;
  if (chunk >= nqb * nhg) return;
  const int within = item % kChunk;
  const int qd = (nqb - 1 - chunk / nhg) * qpc + within / hg;  // heaviest quads first
  if (qd >= nq) return;
  const int hl = (chunk % nhg) * hg + within % hg;
  const int h = p.head0 + hl;
  const int kvh = h / p.grp;
  const AttnHead hd = p.heads[hl];
  const int n = p.n;
  const int bq = kQuad * qd;
  const int nblk = min(kQuad, p.nb - bq);
  const int qsel = wave & 3;                  // block b_qsel, on SIMD qsel
  const int qb = bq + qsel;
  const bool wave_on = qsel < nblk;
  const int row = qb * kBlock + 32 * (wave >> 2) + (lane & 31);
  const bool group_a = wave < 4;

  ItemCtx cx;
  cx.kh = p.k + (size_t)kvh * n * kHeadDim;
  cx.vh = p.v + (size_t)kvh * n * kHeadDim;
  cx.n = n;
  cx.causal = p.causal || hd.kind != KIND_DENSE;
  cx.ashape = hd.kind == KIND_ASHAPE;
  cx.sink = hd.sink;
  cx.local = hd.local;
  cx.qsel = qsel;
  cx.row = row;
  cx.qb = qb;
  cx.sl2 = p.scale_log2;

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
  QuadIter it;
  it.kind = hd.kind;
  it.bq = bq;
  it.nblk = nblk;
  it.nb = p.nb;
  it.causal = p.causal;
  it.rem = 0;
  it.w = 0;
  it.wmax = -1;
  const int bmax = bq + nblk - 1;
  if (hd.kind == KIND_DENSE) {
    it.c = 0;
    it.cmax = p.causal ? bmax : p.nb - 1;
  } else if (hd.kind == KIND_ASHAPE) {
    it.c = 0;
    it.cmax = bmax;
    const int sbk = (int)(((int64_t)hd.sink + kBlock - 1) / kBlock);
    it.sb = sbk < p.nb ? sbk : p.nb;
#pragma unroll
    for (int i = 0; i < kQuad; ++i) {
      const int b = bq + i;
      int lo = b + 1;
      if (hd.local > 0) {
        const int64_t l0 = (int64_t)b * kBlock - hd.local + 1;
        lo = l0 <= 0 ? 0 : (int)(l0 / kBlock);
      }
      it.wlo[i] = lo;
    }
    int lo = it.wlo[0];
    if (0 >= it.sb && 0 < lo) it.c = lo;
  } else if (hd.kind == KIND_VS) {
    const int nwords = (p.nb >> 5) + 1;
    const int last_partial = (n & (kBlock - 1)) != 0;
    const int need_last = last_partial && bmax == p.nb - 1;
    for (int i = tid; i <= nwords; i += kPPThreads) {
      sm.bits[0][i] = i < nwords ? hd.obits[i] : 0u;
      if (need_last) sm.bits[1][i] = i < nwords ? hd.obits[nwords + i] : 0u;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQuad; ++i) it.bitsv[i] = (need_last && bq + i == p.nb - 1) ? sm.bits[1] : sm.bits[0];
    // offsets v relative to b3 = bq + 3 (key block c = b3 - v), whether or not b3 exists
    it.base = bq + kQuad - 1;
    it.init_bitmap_cursor(bq + kQuad - 1);
  } else {  // KIND_BLOCK
    const int nwords = (bmax >> 5) + 1;
    for (int i = tid; i < kQuad * nwords; i += kPPThreads) sm.bits[i / nwords][i % nwords] = 0u;
    __syncthreads();
    const int kb = hd.k_b;
    for (int x = tid; x < kQuad * kb; x += kPPThreads) {
      const int i = x / kb;
      const int e = x - i * kb;
      if (i >= nblk) continue;
      const int b = bq + i;
      if (e < hd.blk_cnt[b]) {
        const int c = hd.blk_idx[(size_t)b * kb + e];
        if (c >= 0 && c <= b) atomicOr(&sm.bits[i][c >> 5], 1u << (c & 31));
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kQuad; ++i) it.bitsv[i] = sm.bits[i];
    it.cmax = bmax;
    it.init_bitmap_cursor(bmax);
  }

  // ---------------- gathered vertical columns of VS heads: compacted up front
  int ncols = 0;
  if (hd.kind == KIND_VS && hd.k_v > 0) {
    const int lim = bmax * kBlock + kBlock - 1;  // last row of the quad
    int kept = 0;
    for (int base = 0; base < hd.k_v && kept < kColCap; base += kPPThreads) {
      const int e = base + tid;
      uint32_t entry = 0;
      bool keep = false;
      if (e < hd.k_v) {
        const int j = hd.v_idx[e];
        const int prev = e > 0 ? hd.v_idx[e - 1] : -1;
        if (j >= 0 && j < n && j <= lim && j != prev) {
          const int cb = j / kBlock;
          uint32_t m = 0;
#pragma unroll
          for (int i = 0; i < kQuad; ++i) {
            const int b = bq + i;
            if (i < nblk && cb <= b) {
              const uint32_t* bw = it.bitsv[i];
              const int o = b - cb;
              if (!((bw[o >> 5] >> (o & 31)) & 1u)) m |= 1u << i;
            }
          }
          keep = m != 0;
          entry = (uint32_t)j | (m << 28);
        }
      }
      int tot;
      const int pos = block_excl_scan_count<kPPThreads>(keep, sm.scan, tot);
      if (keep && kept + pos < kColCap) sm.clist[kept + pos] = entry;
      kept += tot;
    }
    ncols = kept < kColCap ? kept : kColCap;
    const int ntile = (ncols + kBlock - 1) / kBlock;
    for (int s = ncols + tid; s < ntile * kBlock; s += kPPThreads) sm.clist[s] = 0u;  // padding: no member
    __syncthreads();
  }
  const int ngath = (ncols + kBlock - 1) / kBlock;
  int gnext = 0;

  // the next tile of the sequence: block tiles, then gathered tiles
  bool blocks_done = false;
  auto next_tile = [&](TileRef& t) -> bool {
    if (!blocks_done) {
      int c, mem;
      if (it.next(c, mem)) {
        t.c = c;
        t.mem = mem;
        t.gath = 0;
        return true;
      }
      blocks_done = true;
    }
    if (gnext < ngath) {
      int m = 0;
      // members: blocks with a column in this group
      const uint32_t ew = sm.clist[64 * gnext + lane];
#pragma unroll
      for (int i = 0; i < kQuad; ++i) m |= (__ballot((ew >> (28 + i)) & 1u) != 0ull) << i;
      t.c = gnext;
      t.mem = uniform_i32(m);
      t.gath = 1;
      ++gnext;
      return true;
    }
    return false;
  };

  const OperandOffsets oo = operand_offsets();

  // ring of the tiles in flight: tile k in buffer k % 4
  TileRef tr[4];
  int have[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    tr[i] = TileRef{0, 0, 0};
    have[i] = 0;
  }
  have[0] = next_tile(tr[0]);
  if (have[0]) issue_tile(tr[0], cx.kh, cx.vh, k0, v0, n, sm.clist, ncols);
  have[1] = have[0] && next_tile(tr[1]);
  if (have[1]) issue_tile(tr[1], cx.kh, cx.vh, k1, v1, n, sm.clist, ncols);
  // both first tiles in LDS before step 0
  wait_vmem_le<0>();
  barrier();

  // step k: tile k in buffer k % 4 (its QK and, for waves 4-7 one step later,
  // its softmax), tile k - 1 in buffer (k - 1) % 4 (its PV), tile k + 2 loaded
  // into buffer (k + 2) % 4.
  auto step = [&](const int k, uint16_t* kc, uint16_t* vprev, const TileRef& tc, const int hc, const TileRef& tp,
                  const int hp, uint16_t* kn, uint16_t* vn, TileRef& tn, int& hn) -> bool {
    if (!hc && !hp) return false;
    // tile k + 2: its buffer last held tile k - 2, whose PV ended in step k - 1
    hn = hc && next_tile(tn);
    if (hn) issue_tile(tn, cx.kh, cx.vh, kn, vn, n, sm.clist, ncols);
    const bool use_c = hc && wave_on && ((tc.mem >> qsel) & 1);
    const bool use_p = hp && wave_on && ((tp.mem >> qsel) & 1);
    const int mask_c = use_c ? tile_mask(tc, cx) : 0;
    const int mask_p = use_p ? tile_mask(tp, cx) : 0;
    const uint32_t* gc_c = sm.clist + 64 * tc.c;
    const uint32_t* gc_p = sm.clist + 64 * tp.c;
    if (group_a) {
      if (use_p) pv(ws, oo, vprev);
      if (use_c) qk(ws, oo, kc);
      barrier();
      if (use_c)
        softmax(ws, mask_c, tc.gath ? 0 : tc.c * kBlock, gc_c, qsel, row, n, cx.causal, cx.ashape, cx.sink, cx.local,
                cx.sl2);
    } else {
      // the softmax of tile k - 1 (its scores are still in ws.s), then its PV and tile k's QK
      if (use_p)
        softmax(ws, mask_p, tp.gath ? 0 : tp.c * kBlock, gc_p, qsel, row, n, cx.causal, cx.ashape, cx.sink, cx.local,
                cx.sl2);
      barrier();
      if (use_p) pv(ws, oo, vprev);
      if (use_c) qk(ws, oo, kc);
    }
    // tile k + 1 must have landed for step k + 1 (only tile k + 2's loads may be in flight)
    if (hn)
      wait_vmem_le<4>();
    else
      wait_vmem_le<0>();
    barrier();
    return true;
  };

  // steps k = 0, 1, 2, ...: tile k's buffer is k % 4, the previous tile's (k + 3) % 4
  for (int k = 0;; k += 4) {
    if (!step(k, k0, v3, tr[0], have[0], tr[3], k > 0 ? have[3] : 0, k2, v2, tr[2], have[2])) break;
    if (!step(k + 1, k1, v0, tr[1], have[1], tr[0], have[0], k3, v3, tr[3], have[3])) break;
    if (!step(k + 2, k2, v1, tr[2], have[2], tr[1], have[1], k0, v0, tr[0], have[0])) break;
    if (!step(k + 3, k3, v2, tr[3], have[3], tr[2], have[2], k1, v1, tr[1], have[1])) break;
  }

  // ---------------- finalize
  if (!wave_on) return;
  const float ltot = pair_sum32(ws.l);
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
    if (p.lse && g == 0)
      p.lse[(size_t)h * n + row] = ltot > 0.f ? (ws.m + __log2f(ltot)) * 0.6931471805599453f : -INFINITY;
  }
}

// XCD-aware work order: workgroup L runs on XCD L % 8; that XCD's k-th
// workgroup takes item (k / C * 8 + L % 8) * C + k % C (C = 32 resident per XCD).
__global__ __launch_bounds__(kPPThreads, 1) void attn_pp_kernel(const AttnLaunch p) {
  __shared__ PPSmem sm;
  __shared__ __attribute__((aligned(16))) uint16_t k0[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t k1[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t k2[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t k3[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t v0[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t v1[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t v2[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t v3[kTileHalves];
  // when a rounds launch of the same work was queued beside this one, only one of them works
  if (p.rounds_flag != nullptr && *p.rounds_flag != 0) return;
  const int slot = blockIdx.x >> 3;
  const int xcd = (int)(blockIdx.x & (kXcds - 1));
  pp_item(p, ((slot / kChunk) * kXcds + xcd) * kChunk + slot % kChunk, sm, k0, k1, k2, k3, v0, v1, v2, v3);
}

// The 32 workgroups of one XCD wait for each other between rounds: a counter
// per XCD, raised once per workgroup and round. The wait is bounded, so the
// kernel ends even if the group were not resident together (only the L2
// sharing would suffer).
constexpr int kSpinLimit = 1 << 22;
__device__ __forceinline__ void xcd_barrier(int32_t* ctr, int target) {
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(ctr, 1);
    int spins = 0;
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target && spins < kSpinLimit) {
      __builtin_amdgcn_s_sleep(4);
      ++spins;
    }
  }
  __syncthreads();
}

// Rounds variant: exactly 8 x 32 workgroups, one per CU. In round r workgroup L
// takes item (r * 8 + L % 8) * C + L / 8, and the 32 workgroups of an XCD start
// every round together, so long items stay near the same key position and keep
// sharing K/V tiles in that XCD's L2. It works only when *p.rounds_flag is set.
__global__ __launch_bounds__(kPPThreads, 1) void attn_pp_rounds_kernel(const AttnLaunch p) {
  __shared__ PPSmem sm;
  __shared__ __attribute__((aligned(16))) uint16_t k0[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t k1[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t k2[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t k3[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t v0[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t v1[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t v2[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t v3[kTileHalves];
  if (*p.rounds_flag == 0) return;
  const int slot = blockIdx.x >> 3;
  const int xcd = (int)(blockIdx.x & (kXcds - 1));
  for (int r = 0; r < p.rounds; ++r) {
    pp_item(p, (r * kXcds + xcd) * kChunk + slot, sm, k0, k1, k2, k3, v0, v1, v2, v3);
    xcd_barrier(p.xcd_sync + xcd, kChunk * (r + 1));
  }
}

__global__ void pp_zero_counters_kernel(int32_t* c, int n) {
  if ((int)threadIdx.x < n) c[threadIdx.x] = 0;
}

}  // namespace

bool attn_pp_supported(const AttnLaunch& a) {
  for (int i = 0; i < a.nh; ++i) {
    const AttnHead& h = a.heads[i];
    if (h.pos != nullptr) return false;
    if (h.kind != KIND_DENSE && h.kind != KIND_ASHAPE && h.kind != KIND_VS && h.kind != KIND_BLOCK) return false;
    if (h.kind == KIND_VS && h.k_v > kColCap) return false;
  }
  return true;
}

// Whether this device holds all 8 x 32 workgroups of a rounds launch at once
// (one per CU on at least 256 CUs). Asked once per device.
static bool pp_rounds_supported() {
  static int cache[64] = {};  // 0 unknown, 1 yes, 2 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  int& c = cache[dev];
  if (c == 0) {
    int cus = 0, per_cu = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)attn_pp_rounds_kernel, kPPThreads, 0);
    c = (e == hipSuccess && (long long)cus * per_cu >= kXcds * kChunk) ? 1 : 2;
  }
  return c == 1;
}

hipError_t launch_attn_pp(const AttnLaunch& a, hipStream_t stream) {
  const int nq = (a.nb + kQuad - 1) / kQuad;
  if (nq <= 0 || a.nh <= 0 || a.hgroup <= 0 || a.nh % a.hgroup != 0 || kChunk % a.hgroup != 0)
    return hipErrorInvalidValue;
  const int qpc = kChunk / a.hgroup;
  const long long chunks = (long long)((nq + qpc - 1) / qpc) * (a.nh / a.hgroup);
  const long long grid = (chunks + kXcds - 1) / kXcds * kXcds * kChunk;
  AttnLaunch c = a;
  c.xcd_sync = nullptr;
  c.rounds_flag = nullptr;
  if (a.xcd_sync != nullptr && a.rounds_flag != nullptr && pp_rounds_supported()) {
    // the rounds launch, then the ordinary one; the device-side flag lets exactly one of them work
    AttnLaunch b = a;
    b.rounds = (int)((chunks + kXcds - 1) / kXcds);
    hipLaunchKernelGGL(pp_zero_counters_kernel, dim3(1), dim3(64), 0, stream, b.xcd_sync, kXcds);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_pp_rounds_kernel, dim3(kXcds * kChunk), dim3(kPPThreads), 0, stream, b);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    c.rounds_flag = a.rounds_flag;
  }
  hipLaunchKernelGGL(attn_pp_kernel, dim3((unsigned)grid), dim3(kPPThreads), 0, stream, c);
  return hipGetLastError();
}

}  // namespace minf
