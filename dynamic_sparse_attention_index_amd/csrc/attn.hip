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
//  * K and V tiles go from HBM straight into LDS with 16-byte direct loads
//    (buffer_load_dwordx4 ... lds: no staging registers, no VALU), row-major with
//    the 16-byte chunk index of each row XOR-swizzled so that both operand
//    reads below are free of bank conflicts.
//  * V is read with the CDNA4 LDS transpose load (ds_read_b64_tr_b16): each
//    16-lane group turns 4 key rows x 16 d into 16 lanes x 4 keys, which is
//    the A-operand layout of O^T = V^T P^T; the key order inside each 16-key
//    step matches the score accumulator's row order, so P goes from
//    accumulator to MFMA operand without any cross-lane movement.
//  * K and V have rings of two LDS buffers each, one barrier per tile. Key
//    blocks and windows of every kind (Block-Sparse also on permuted
//    sequences) run a software pipeline per wave (tile.h): the scores of tile
//    t + 1 are formed on the matrix cores while the vector ALUs compute tile
//    t's probabilities, then tile t's PV product runs; K of tile t + 2 and V
//    of tile t + 1 stream in meanwhile. Gathered columns (and launches that
//    would mix permuted and window heads) compute one tile per step with the
//    next tile's K and V in flight.
//  * every kind walks its key tiles in ascending key order, and the work map
//    gives each XCD whole chunks of 64 workgroups (one head x 64 pairs for
//    sparse plans, one GQA group x 16 pairs for dense) that move through the
//    keys together and share the tiles in that XCD's L2.
//  * Block-Sparse plans on a permuted sequence (the grid pattern) carry the
//    original position of every row; a tile that is not entirely earlier than
//    the wave's earliest query is masked by comparing positions, which the
//    instantiations with the kXkPos bit handle.
//  * VS and Block-Sparse items keep a summary bit per 32-bit word of their
//    bitmaps in LDS, so the tile cursor skips runs of empty words.
#include "common.h"
#include "launch.h"
#include "tile.h"

namespace minf {
namespace {

constexpr int kThreads = 256;
constexpr int kXcds = kRoundXcds;  // MI355X: workgroups are dealt round-robin to 8 XCDs, each with its own L2
constexpr int kChunk = 64;   // workgroups one XCD runs at once (32 CUs x 2)
constexpr int kTileHalves = kBlock * kHeadDim;  // one 64 x 128 bf16 tile, 16 KiB, rows of 256 bytes
constexpr int kBitWords = (kMaxTokens / kBlock) / 32 + 1;  // 513 words per bitmap
constexpr int kColChunk = 1024;  // candidate vertical columns compacted per round
constexpr int kBitRounds = (kBitWords + kThreads - 1) / kThreads;  // bitmap words per thread (3)
constexpr int kNzWords = kBitRounds * (kThreads / 32);               // summary words (24)

// K/V tile buffers are four distinct LDS objects (not one array): the
// compiler then knows that the direct loads filling one buffer cannot alias
// the reads of the other, and does not wait for the loads in flight before
// computing on the current tile.
struct Smem {
  uint32_t bits[2][kBitWords];
  uint32_t nz[kNzWords];  // VS / BLOCK: bit w set when word w of either bitmap is non-zero
  uint32_t clist[kColChunk];
  int scan[16];
};



__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

enum : int { KIND_DENSE = 0, KIND_ASHAPE = 1, KIND_VS = 2, KIND_BLOCK = 3, KIND_VSW = 4 };

__device__ __forceinline__ uint32_t bit_at(const uint32_t* w, int v) { return (w[v >> 5] >> (v & 31)) & 1u; }

// Whether the offset bitmap w over [0, n) has a set bit in [x, x + 63].
__device__ __forceinline__ bool any_offset(const uint32_t* w, int x, int n) {
  const int lo = x > 0 ? x : 0;
  const int hi = x + 63 < n - 1 ? x + 63 : n - 1;
  if (lo > hi) return false;
  for (int ww = lo >> 5; ww <= (hi >> 5); ++ww) {
    uint32_t m = w[ww];
    if (ww == (lo >> 5)) m &= 0xffffffffu << (lo & 31);
    if (ww == (hi >> 5)) m &= 0xffffffffu >> (31 - (hi & 31));
    if (m != 0u) return true;
  }
  return false;
}

// A value that is the same in every lane of the wave, as a scalar.
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Tile sequence over the key blocks of the pair (b0, b1). Every thread runs
// the same sequence (it only reads kernel arguments and LDS).
struct BlockIter {
  int kind, b0, b1, has_b1, nb, causal;
  int c, cmax;         // dense / A-shape cursor
  int sb, wlo0, wlo1;  // A-shape
  int w, wmax, base;   // VS / BLOCK bitmap cursor
  uint32_t rem;
  uint32_t mw0, mw1;   // membership of b0 / b1 for the bits of the current word
  // VS windows: the head's tile cover (relative to a block's first row), the
  // next tile of b0 and of b1, and the blocks' first rows
  const int2* wt;
  int nwt, i0, i1, wb0, wb1;
  int2 w0, w1;  // entries i0 and i1 of wt, loaded one call ahead (the same in every lane)
  // BLOCK: membership bitmaps over key blocks c of b0 and b1.
  // VS: block-offset bitmaps of b0 and b1 (they differ only for a partial last block).
  const uint32_t* bits0;
  const uint32_t* bits1;
  const uint32_t* nzw;  // VS / BLOCK: non-empty words of the bitmaps

  // VS: the highest word <= ww whose union can be non-zero, or -1. The union
  // of word x reads bit 31 of word x - 1, so a non-empty word z makes words z
  // and z + 1 candidates.
  __device__ int prev_nonempty(int ww) {
    int sw = ww >> 5;
    uint32_t m = uniform_u32(nzw[sw]) & (0xffffffffu >> (31 - (ww & 31)));
    while (m == 0u) {
      if (--sw < 0) return -1;
      m = uniform_u32(nzw[sw]);
    }
    const int z = (sw << 5) + 31 - __builtin_clz(m);
    return z + 1 <= ww ? z + 1 : ww;
  }

  // BLOCK: the lowest word >= ww with a set bit, or wmax + 1.
  __device__ int next_nonempty(int ww) {
    int sw = ww >> 5;
    const int swmax = wmax >> 5;
    uint32_t m = uniform_u32(nzw[sw]) & (0xffffffffu << (ww & 31));
    while (m == 0u) {
      if (++sw > swmax) return wmax + 1;
      m = uniform_u32(nzw[sw]);
    }
    return (sw << 5) + __builtin_ctz(m);
  }

  // Reads word ww of both memberships from LDS (kept in registers until the
  // cursor leaves the word) and returns their union. The words are the same
  // in every lane; taking them as wave-uniform keeps the tile index and the
  // copy addresses derived from it in scalar registers.
  __device__ uint32_t union_word(int ww) {
    if (kind == KIND_VS) {
      const uint32_t bw = uniform_u32(bits0[ww]);
      const uint32_t prev = ww > 0 ? uniform_u32(bits0[ww - 1]) : 0u;
      mw0 = (bw << 1) | (prev >> 31);                  // offsets v with v - 1 in b0's set
      mw1 = has_b1 ? uniform_u32(bits1[ww]) : 0u;     // offsets v in b1's set
    } else {
      mw0 = uniform_u32(bits0[ww]);
      mw1 = uniform_u32(bits1[ww]);
    }
    return mw0 | mw1;
  }

  // Bitmap cursor over offsets/blocks [0, vmax]. VS walks its offsets
  // downwards (key blocks in ascending order, like every other kind), BLOCK
  // walks its key blocks upwards.
  __device__ void init_bitmap_cursor(int vmax) {
    wmax = vmax >> 5;
    w = kind == KIND_VS ? wmax : 0;
    uint32_t u = union_word(w);
    if (w == wmax) u &= (vmax & 31) == 31 ? 0xffffffffu : ((1u << ((vmax & 31) + 1)) - 1u);
    rem = u;
  }

  // VS windows: the next tile of the pair in key order. b1's tiles are b0's
  // shifted by 64 keys; a tile both blocks have is visited once. t is the
  // tile's first key (may be negative near the start), e0 / e1 the end of the
  // tile's interval for b0 / b1.
  __device__ bool next_window(int& t, int& mem, int& e0, int& e1) {
    const int s0 = i0 < nwt ? wb0 + (int)uniform_u32((uint32_t)w0.x) : 0x7fffffff;
    const int s1 = i1 < nwt ? wb1 + (int)uniform_u32((uint32_t)w1.x) : 0x7fffffff;
    if (s0 == 0x7fffffff && s1 == 0x7fffffff) return false;
    t = s0 < s1 ? s0 : s1;
    const int m0 = s0 == t, m1 = s1 == t;
    e0 = m0 ? wb0 + (int)uniform_u32((uint32_t)w0.y) : 0;
    e1 = m1 ? wb1 + (int)uniform_u32((uint32_t)w1.y) : 0;
    i0 += m0;
    i1 += m1;
    mem = m0 | (m1 << 1);
    // the entries the next call reads: loaded now, so their latency overlaps
    // the step (the step's closing wait for its copies covers them)
    if (m0 && i0 < nwt) w0 = wt[i0];
    if (m1 && i1 < nwt) w1 = wt[i1];
    return true;
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
    if (kind == KIND_VS) {
      // highest remaining offset v first: key block c = b0 + 1 - v ascending;
      // below an empty word, the run of empty words is skipped through the summary
      while (rem == 0u) {
        if (--w < 0) return false;
        rem = union_word(w);
        if (rem == 0u && w > 0) {
          w = prev_nonempty(w - 1);
          if (w < 0) return false;
          rem = union_word(w);
        }
      }
      const int bit = 31 - __builtin_clz(rem);
      rem ^= 1u << bit;
      const int v = (w << 5) + bit;
      cout = base - v;
      mem = (int)((mw0 >> bit) & 1u) | ((int)((mw1 >> bit) & 1u) << 1);
      return true;
    }
    // bitmap kinds: iterate set bits of the union word by word; above an
    // empty word, the run of empty words is skipped through the summary
    while (rem == 0u) {
      if (++w > wmax) return false;
      uint32_t u = union_word(w);
      if (u == 0u && w < wmax) {
        w = next_nonempty(w + 1);
        if (w > wmax) return false;
        u = union_word(w);
      }
      if (w == wmax) {
        const int top = cmax & 31;
        u &= top == 31 ? 0xffffffffu : ((1u << (top + 1)) - 1u);
      }
      rem = u;
    }
    const int bit = __builtin_ctz(rem);
    rem &= rem - 1u;
    cout = (w << 5) + bit;
    mem = (int)((mw0 >> bit) & 1u) | ((int)((mw1 >> bit) & 1u) << 1);
    return true;
  }
};

// Issue the direct HBM -> LDS copies of one K/V tile. Wave w's instruction i
// fills LDS chunks [256 i + 64 w, +64): rows 16 i + 4 w .. +3, the 16 lanes of
// a row covering its 16 chunks (one 256-byte row per 16 lanes, coalesced).
__device__ __forceinline__ int tile_row_lo() { return 4 * (threadIdx.x >> 6) + ((threadIdx.x & 63) >> 4); }
__device__ __forceinline__ uint32_t tile_chunk_byte() {
  return (uint32_t)((((threadIdx.x & 63) & 15) ^ swz(tile_row_lo())) * 16);
}

// Tile of 64 consecutive key rows starting at byte tile_byte of the head (a
// valid row with 64 rows left): a uniform offset and per-lane 32-bit offsets.
__device__ __forceinline__ void issue_contig(rsrc_t kr, rsrc_t vr, uint32_t tile_byte, uint16_t* kt, uint16_t* vt,
                                             uint32_t lane_off) {
  const int wave = wave_index();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t off = lane_off + (uint32_t)i * 16 * 256;
    copy16(kr, kt + (256 * i + 64 * wave) * 8, off, tile_byte);
    copy16(vr, vt + (256 * i + 64 * wave) * 8, off, tile_byte);
  }
}

// General tile: rows_of(x) gives the key index of tile row x (always a valid
// row; rows past the mask are masked later).
template <class RowFn>
__device__ __forceinline__ void issue_rows(rsrc_t kr, rsrc_t vr, uint16_t* kt, uint16_t* vt, RowFn rows_of) {
  const int wave = threadIdx.x >> 6;
  const int rlo = tile_row_lo();
  const uint32_t cb = tile_chunk_byte();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t off = (uint32_t)rows_of(16 * i + rlo) * 256u + cb;
    copy16(kr, kt + (256 * i + 64 * wave) * 8, off, 0u);
    copy16(vr, vt + (256 * i + 64 * wave) * 8, off, 0u);
  }
}

// One of the two (K or V) of a tile: contiguous rows, then general rows.
__device__ __forceinline__ void issue_contig1(rsrc_t r, uint32_t tile_byte, uint16_t* t, uint32_t lane_off) {
  const int wave = wave_index();
#pragma unroll
  for (int i = 0; i < 4; ++i) copy16(r, t + (256 * i + 64 * wave) * 8, lane_off + (uint32_t)i * 16 * 256, tile_byte);
}
template <class RowFn>
__device__ __forceinline__ void issue_rows1(rsrc_t r, uint16_t* t, RowFn rows_of) {
  const int wave = threadIdx.x >> 6;
  const int rlo = tile_row_lo();
  const uint32_t cb = tile_chunk_byte();
#pragma unroll
  for (int i = 0; i < 4; ++i) copy16(r, t + (256 * i + 64 * wave) * 8, (uint32_t)rows_of(16 * i + rlo) * 256u + cb, 0u);
}

// One tile for one wave. MASK: 0 = every key visible; 1 = causal (j <= i);
// 2 = general predicate (causal or j < n, plus the A-shape clause);
// 3 = gathered columns (per-column membership flag and j <= i).
// 4 = original positions (permuted sequences): key visible iff its position <= the row's.
enum : int { MASK_NONE = 0, MASK_CAUSAL = 1, MASK_GENERAL = 2, MASK_GATHER = 3, MASK_POS = 4, MASK_WIN = 5 };
constexpr int kXkPos = 1, kXkWin = 2;  // extended plan kinds of an attention instantiation

// The mask touches only the score registers; MASK is uniform across the wave.
template <int XK>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[2], int MASK, int key0, const uint32_t* gcols, int qsel,
                                            int row, int n, int causal, int ashape, int sink, int local) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  if (MASK == MASK_CAUSAL) {
    const int lim = row - key0 - 4 * g;  // key slot kx = kx0 + 4g is visible iff kx0 <= lim
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kx0 = 32 * mt + 8 * (i >> 2) + (i & 3);
        s[mt][i] = kx0 <= lim ? s[mt][i] : -INFINITY;
      }
  } else if (MASK == MASK_GENERAL) {
    // with j = key0 + 4g + kx0: visible iff kx0 <= hi and (kx0 < lo_sink or kx0 > lo_win)
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
  } else if ((XK & kXkWin) && MASK == MASK_WIN) {
    // VS window tile from key key0: visible iff 0 <= j < local (the end of the
    // block's window interval) and j <= row, with j = key0 + 4g + kx0
    const int base = key0 + 4 * g;
    const int hi = min(row - base, local - 1 - base);
    const int lo = -base;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kx0 = 32 * mt + 8 * (i >> 2) + (i & 3);
        s[mt][i] = (kx0 <= hi && kx0 >= lo) ? s[mt][i] : -INFINITY;
      }
  } else if ((XK & kXkPos) && MASK == MASK_POS) {
    // gcols holds the tile's key positions; `row` is this lane's query position
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x4 e4 = *(const u32x4*)(gcols + 32 * mt + 8 * q4 + 4 * g);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool vis = (int)(e4[t] & 0x3fffffffu) <= row;
          s[mt][4 * q4 + t] = vis ? s[mt][4 * q4 + t] : -INFINITY;
        }
      }
  } else if (MASK == MASK_GATHER) {
    const uint32_t sh = 30 + qsel;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x4 e4 = *(const u32x4*)(gcols + 32 * mt + 8 * q4 + 4 * g);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t e = e4[t];
          const bool vis = ((e >> sh) & 1u) && (int)(e & 0x3fffffffu) <= row;
          s[mt][4 * q4 + t] = vis ? s[mt][4 * q4 + t] : -INFINITY;
        }
      }
  }
}

// One tile for one wave, MASK as above.
template <int XK>
__device__ __forceinline__ void compute_tile(WaveState& ws, const OperandOffsets& oo, const uint16_t* kt,
                                             const uint16_t* vt, int MASK, int key0, const uint32_t* gcols,
                                             int qsel, int row, int n, int causal, int ashape, int sink,
                                             int local, float sl2) {
  f32x16 s[2];
  qk_tile(ws, oo, kt, s);
  mask_scores<XK>(s, MASK, key0, gcols, qsel, row, n, causal, ashape, sink, local);
  softmax_pv(ws, oo, s, vt, sl2);
}

// XK: the extended plan kinds the launch holds (kXkPos: Block-Sparse heads on
// permuted sequences; kXkWin: VS window heads). Each combination is its own
// instantiation, so every kernel carries only the code its launch needs.
// One work item: a head and a pair of query blocks. Item i is the (i % C)-th
// member of chunk i / C; a chunk is one group of hg heads sharing a KV head
// times C / hg consecutive query-block pairs (C = 64), and chunks go heaviest
// pair block first.
template <int XK>
__device__ __forceinline__ void attn_item(const AttnLaunch& p, const int item, Smem& sm, uint16_t* kt0,
                                          uint16_t* kt1, uint16_t* vt0, uint16_t* vt1) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int npairs = (p.nb + 1) >> 1;
  const int hg = p.hgroup;
  const int ppc = kChunk / hg;                  // pairs per chunk
  const int npb = (npairs + ppc - 1) / ppc;     // pair blocks
  const int nhg = p.nh / hg;                    // head groups in this launch
  const int chunk = item / kChunk;
  if (chunk >= npb * nhg) return;
  const int within = item % kChunk;
  const int pr = (npb - 1 - chunk / nhg) * ppc + within / hg;
  if (pr >= npairs) return;
  const int hl = (chunk % nhg) * hg + within % hg;
  const AttnHead hd = p.heads[hl];
  const int h = hd.head;
  const int kvh = h / p.grp;
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
  const rsrc_t kr = buffer_of(kh, (uint32_t)n * (kHeadDim * 2));
  const rsrc_t vr = buffer_of(vh, (uint32_t)n * (kHeadDim * 2));

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
    // offset bitmap of full blocks, and (when n % 64 != 0) of the partial
    // last block, up to the pair's largest offset b0 + 1, with one summary bit
    // per word (either bitmap non-zero); all loads are issued before any use
    const int nwords = (p.nb >> 5) + 1;
    const int ncopy = ((b0 + 1) >> 5) + 1;
    const int last_partial = (n & (kBlock - 1)) != 0;
    const int need_last = last_partial && bmax == p.nb - 1;
    uint32_t wa[kBitRounds], wb[kBitRounds];
#pragma unroll
    for (int r = 0; r < kBitRounds; ++r) {
      const int i = r * kThreads + tid;
      wa[r] = i < ncopy ? hd.obits[i] : 0u;
      wb[r] = i < ncopy && need_last ? hd.obits[nwords + i] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kBitRounds; ++r) {
      const int i = r * kThreads + tid;
      if (r * kThreads < ncopy) {  // uniform: every wave takes the ballot
        if (i < ncopy) {
          sm.bits[0][i] = wa[r];
          if (need_last) sm.bits[1][i] = wb[r];
        }
        const uint64_t bal = __ballot((wa[r] | wb[r]) != 0u);
        if (lane == 0) {
          const int sw = (r * kThreads + 64 * wave) >> 5;
          sm.nz[sw] = (uint32_t)bal;
          sm.nz[sw + 1] = (uint32_t)(bal >> 32);
        }
      }
    }
    __syncthreads();
    it.nzw = sm.nz;
    it.bits0 = (need_last && b0 == p.nb - 1) ? sm.bits[1] : sm.bits[0];
    it.bits1 = (need_last && b1 == p.nb - 1) ? sm.bits[1] : sm.bits[0];
    it.base = b0 + 1;
    it.init_bitmap_cursor(it.base);
  } else if ((XK & kXkWin) && hd.kind == KIND_VSW) {
    // first tile of each block's window list that ends after key 0
    it.wt = hd.wtiles;
    it.nwt = (int)uniform_u32((uint32_t)*hd.wcount);
    it.wb0 = b0 * kBlock;
    it.wb1 = b1 * kBlock;
    // 64-way search: each round the 64 lanes test 64 evenly spaced entries
    // (tile ends ascend) with one load each, so a few rounds of loads replace a
    // chain of dependent ones
    auto first_tile = [&](int wb) -> int {
      int lo = 0, hi = it.nwt;  // entries below lo end at or before key 0, entries from hi on after it
      while (lo < hi) {
        const int step = (hi - lo + 63) >> 6;
        const int idx = lo + lane * step;
        const bool after = idx >= hi || wb + it.wt[idx].y > 0;
        const uint64_t bal = __ballot(after);
        if (bal == 0ull) {
          lo += 63 * step + 1;
        } else {
          const int f = __builtin_ctzll(bal);
          const int nhi = min(hi, lo + f * step);
          if (f > 0) lo += (f - 1) * step + 1;
          hi = nhi;
        }
        lo = (int)uniform_u32((uint32_t)lo);
        hi = (int)uniform_u32((uint32_t)hi);
      }
      return lo;
    };
    it.i0 = first_tile(it.wb0);
    it.i1 = has_b1 ? first_tile(it.wb1) : it.nwt;
    it.w0 = it.i0 < it.nwt ? it.wt[it.i0] : int2{0, 0};
    it.w1 = it.i1 < it.nwt ? it.wt[it.i1] : int2{0, 0};
  } else {  // KIND_BLOCK (on a permuted sequence: every key block can be selected)
    const int cmax_blk = hd.pos ? p.nb - 1 : bmax;
    const int nwords = (cmax_blk >> 5) + 1;
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
        if (c >= 0 && c <= (hd.pos ? cmax_blk : b)) atomicOr(&sm.bits[which][c >> 5], 1u << (c & 31));
      }
    }
    __syncthreads();
    // summary of the non-empty words (every wave takes the ballots)
#pragma unroll
    for (int r = 0; r < kBitRounds; ++r) {
      if (r * kThreads < nwords) {
        const int i = r * kThreads + tid;
        const uint64_t bal = __ballot(i < nwords && (sm.bits[0][i] | sm.bits[1][i]) != 0u);
        if (lane == 0) {
          const int sw = (r * kThreads + 64 * wave) >> 5;
          sm.nz[sw] = (uint32_t)bal;
          sm.nz[sw + 1] = (uint32_t)(bal >> 32);
        }
      }
    }
    __syncthreads();
    it.nzw = sm.nz;
    it.cmax = cmax_blk;
    it.init_bitmap_cursor(cmax_blk);
  }
  // permuted sequences: each lane's query position and the wave's earliest one
  const bool posm = (XK & kXkPos) && hd.kind == KIND_BLOCK && hd.pos != nullptr;
  const rsrc_t posr = buffer_of(posm ? (const void*)hd.pos : (const void*)kh, posm ? (uint32_t)n * 4u : 0u);
  int rpos = row, wminpos = 0;
  if (posm) {
    rpos = row < n ? hd.pos[row] : -1;
    int mn = row < n ? rpos : 0x3fffffff;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mn = min(mn, __shfl_xor(mn, off));
    wminpos = mn;
  }
  const int ashape = hd.kind == KIND_ASHAPE;

  const OperandOffsets oo = operand_offsets();

  // ---------------- phase A: 64x64 key blocks
  {
    int c_cur = 0, m_cur = 0, c_nxt = 0, m_nxt = 0;
    const uint32_t lane_off = (uint32_t)tile_row_lo() * 256u + tile_chunk_byte();
    const int causal_eff = p.causal || hd.kind != KIND_DENSE;
    auto issue_block = [&](int cblk, uint16_t* ktn, uint16_t* vtn, uint32_t* psn) {
      if ((cblk + 1) * kBlock <= n) {
        issue_contig(kr, vr, (uint32_t)cblk * kBlock * (kHeadDim * 2), ktn, vtn, lane_off);
        // permuted sequences: the tile's 64 key positions go to LDS with it
        if (posm && wave == 0)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(posr, (lds_ptr)psn, 4, (uint32_t)lane * 4u,
                                                   (uint32_t)cblk * kBlock * 4u, 0, 0);
      } else {
        // partial last block: rows past n repeat row n - 1 and are always masked
        issue_rows(kr, vr, ktn, vtn, [&](int x) { int j = cblk * kBlock + x; return j < n ? j : n - 1; });
        if (posm && wave == 0) {
          const int j = cblk * kBlock + lane;
          psn[lane] = j < n ? (uint32_t)hd.pos[j] : 0x3fffffffu;
        }
      }
    };
    // VS windows: tiles start at any key; e0 / e1 end the tile's interval for b0 / b1
    const bool vsw = (XK & kXkWin) && hd.kind == KIND_VSW;
    int e0_cur = 0, e1_cur = 0, e0_nxt = 0, e1_nxt = 0;
    // permuted sequences: the latest original position of the tile's key block,
    // loaded with the tile so that the visibility test does not wait for it
    int bm_cur = 0, bm_nxt = 0;
    auto next_tile = [&](int& c, int& m, int& e0, int& e1) -> bool {
      if ((XK & kXkWin) && vsw) return it.next_window(c, m, e0, e1);
      return it.next(c, m);
    };
    auto issue_tile = [&](int c, uint16_t* ktn, uint16_t* vtn, uint32_t* psn) {
      if ((XK & kXkWin) && vsw) {
        // 64 keys from key c; rows outside [0, n) load a valid row and are masked
        if (c >= 0 && c + kBlock <= n) {
          issue_contig(kr, vr, (uint32_t)c * (kHeadDim * 2), ktn, vtn, lane_off);
        } else {
          issue_rows(kr, vr, ktn, vtn, [&](int x) {
            const int j = c + x;
            return j < 0 ? 0 : (j < n ? j : n - 1);
          });
        }
      } else {
        issue_block(c, ktn, vtn, psn);
      }
    };
    // one pipelined step: issue the next tile into (ktn, vtn), compute the current one from (ktc, vtc)
    auto step = [&](uint16_t* ktc, uint16_t* vtc, uint32_t* psc, uint16_t* ktn, uint16_t* vtn,
                    uint32_t* psn) -> bool {
      const bool hn = next_tile(c_nxt, m_nxt, e0_nxt, e1_nxt);
      if (hn) issue_tile(c_nxt, ktn, vtn, psn);
      if ((XK & kXkPos) && posm && hn) bm_nxt = hd.blkmax[c_nxt];
      if (wave_on && ((m_cur >> qsel) & 1)) {
        int full, mask;
        int key0 = c_cur * kBlock, wend = hd.local;
        if ((XK & kXkPos) && posm) {
          full = bm_cur <= wminpos;
          mask = full ? MASK_NONE : MASK_POS;
        } else if ((XK & kXkWin) && vsw) {
          key0 = c_cur;
          wend = qsel ? e1_cur : e0_cur;
          const int rmin = qb * kBlock + (wave & 1) * 32;  // the wave's first row
          full = key0 >= 0 && key0 + kBlock <= wend && key0 + kBlock - 1 <= rmin;
          mask = full ? MASK_NONE : MASK_WIN;
        } else {
          if (causal_eff) {
            full = c_cur < qb;
            if (ashape && full)
              full = ((int64_t)c_cur * kBlock + kBlock - 1 < hd.sink) ||
                     ((int64_t)qb * kBlock + kBlock - 1 - (int64_t)c_cur * kBlock < hd.local);
          } else {
            full = (c_cur + 1) * kBlock <= n;
          }
          mask = full ? MASK_NONE : ((causal_eff && !ashape) ? MASK_CAUSAL : MASK_GENERAL);
        }
        // rpos is the query row itself unless the sequence is permuted
        compute_tile<XK>(ws, oo, ktc, vtc, mask, key0, (XK & kXkPos) ? psc : nullptr, qsel, rpos, n, causal_eff, ashape,
                           hd.sink, wend, sl2);
      }
      wait_vmem();
      __syncthreads();
      c_cur = c_nxt;
      m_cur = m_nxt;
      e0_cur = e0_nxt;
      e1_cur = e1_nxt;
      bm_cur = bm_nxt;
      return hn;
    };
    if constexpr (XK == 0 || XK == kXkWin || XK == kXkPos) {
      // Software-pipelined walk (dense, A-shape, VS, VS window and Block-Sparse
      // heads, Block-Sparse also on permuted sequences). Tile t's K sits in K buffer t % 2 and
      // its V in V buffer t % 2. Step t forms the scores of tile t + 1 (K buffer
      // (t + 1) % 2) while the softmax of tile t runs, then tile t's PV product
      // (V buffer t % 2); meanwhile K of tile t + 2 streams into K buffer t % 2
      // (tile t's K was last read in step t - 1) and V of tile t + 1 into V
      // buffer (t + 1) % 2 (last read in step t - 1). Both land before the
      // step's closing barrier. A tile is key block c (keys 64 c ..), or for a
      // VS window head the 64 keys from key c.
      auto kstart = [&](int c) -> int { return ((XK & kXkWin) && vsw) ? c : c * kBlock; };
      auto issue_k = [&](int c, uint16_t* dst) {
        const int j0 = kstart(c);
        if (j0 >= 0 && j0 + kBlock <= n)
          issue_contig1(kr, (uint32_t)j0 * (kHeadDim * 2), dst, lane_off);
        else
          issue_rows1(kr, dst, [&](int x) { const int j = j0 + x; return j < 0 ? 0 : (j < n ? j : n - 1); });
      };
      auto issue_v = [&](int c, uint16_t* dst) {
        const int j0 = kstart(c);
        if (j0 >= 0 && j0 + kBlock <= n)
          issue_contig1(vr, (uint32_t)j0 * (kHeadDim * 2), dst, lane_off);
        else
          issue_rows1(vr, dst, [&](int x) { const int j = j0 + x; return j < 0 ? 0 : (j < n ? j : n - 1); });
      };
      // permuted sequences: a tile's key positions go to LDS with its V rows (slot
      // t % 2, read when tile t is masked) and its key block's latest position to
      // a register, both one step ahead
      uint32_t* ps0 = sm.clist;
      uint32_t* ps1 = sm.clist + kBlock;
      auto issue_pos = [&](int cblk, uint32_t* psn) {
        if (wave != 0) return;
        if ((cblk + 1) * kBlock <= n) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(posr, (lds_ptr)psn, 4, (uint32_t)lane * 4u,
                                                   (uint32_t)cblk * kBlock * 4u, 0, 0);
        } else {
          const int j = cblk * kBlock + lane;
          psn[lane] = j < n ? (uint32_t)hd.pos[j] : 0x3fffffffu;
        }
      };
      const int rmin = qb * kBlock + (wave & 1) * 32;  // the wave's first row
      // mask of tile c for this wave's block; wend: the A-shape window, or the end of a VS window interval
      auto tile_mask_of = [&](int c, int e0, int e1, int& wend) -> int {
        wend = hd.local;
        if ((XK & kXkWin) && vsw) {
          wend = qsel ? e1 : e0;
          return (c >= 0 && c + kBlock <= wend && c + kBlock - 1 <= rmin) ? MASK_NONE : MASK_WIN;
        }
        bool full;
        if (causal_eff) {
          full = c < qb;
          if (ashape && full)
            full = ((int64_t)c * kBlock + kBlock - 1 < hd.sink) ||
                   ((int64_t)qb * kBlock + kBlock - 1 - (int64_t)c * kBlock < hd.local);
        } else {
          full = (c + 1) * kBlock <= n;
        }
        return full ? MASK_NONE : ((causal_eff && !ashape) ? MASK_CAUSAL : MASK_GENERAL);
      };
      int c2 = 0, m2 = 0, e02 = 0, e12 = 0;
      bool h0 = next_tile(c_cur, m_cur, e0_cur, e1_cur), h1 = false;
      if (h0) {
        issue_k(c_cur, kt0);
        issue_v(c_cur, vt0);
        if ((XK & kXkPos) && posm) {
          issue_pos(c_cur, ps0);
          bm_cur = hd.blkmax[c_cur];
        }
        h1 = next_tile(c_nxt, m_nxt, e0_nxt, e1_nxt);
        if (h1) issue_k(c_nxt, kt1);
      }
      wait_vmem();
      __syncthreads();
      f32x16 sa[2], sb[2];
      if (h0 && wave_on && ((m_cur >> qsel) & 1)) qk_tile(ws, oo, kt0, sa);
      __syncthreads();  // every wave has read K buffer 0 before tile 2 overwrites it
      auto pstep = [&](f32x16 (&sc)[2], f32x16 (&sn)[2], uint16_t* kc, uint16_t* kn, uint16_t* vc,
                       uint16_t* vn, uint32_t* pc, uint32_t* pn) -> bool {
        const bool h2 = h1 && next_tile(c2, m2, e02, e12);
        if (h2) issue_k(c2, kc);
        if (h1) {
          issue_v(c_nxt, vn);
          if ((XK & kXkPos) && posm) {
            issue_pos(c_nxt, pn);
            bm_nxt = hd.blkmax[c_nxt];
          }
        }
        const bool u0 = wave_on && ((m_cur >> qsel) & 1);
        const bool u1 = h1 && wave_on && ((m_nxt >> qsel) & 1);
        if (u0) {
          int wend;
          int mask = tile_mask_of(c_cur, e0_cur, e1_cur, wend);
          // permuted sequences: the tile is fully visible when its key block's
          // latest position is at most the wave's earliest query position
          if ((XK & kXkPos) && posm) mask = bm_cur <= wminpos ? MASK_NONE : MASK_POS;
          // rpos is the query row itself unless the sequence is permuted
          if (mask != MASK_NONE)
            mask_scores<XK>(sc, mask, kstart(c_cur), (XK & kXkPos) ? pc : nullptr, qsel, rpos, n, causal_eff, ashape,
                            hd.sink, wend);
          if (u1)
            fused_tile_pair(ws, oo, sc, kn, vc, sn, sl2);
          else
            softmax_pv(ws, oo, sc, vc, sl2);
        } else if (u1) {
          qk_tile(ws, oo, kn, sn);
        }
        wait_vmem();
        __syncthreads();
        // tile t + 1 becomes the current one
        h0 = h1;
        c_cur = c_nxt;
        m_cur = m_nxt;
        e0_cur = e0_nxt;
        e1_cur = e1_nxt;
        h1 = h2;
        c_nxt = c2;
        m_nxt = m2;
        e0_nxt = e02;
        e1_nxt = e12;
        bm_cur = bm_nxt;
        return h0;
      };
      while (h0) {
        if (!pstep(sa, sb, kt0, kt1, vt0, vt1, ps0, ps1)) break;
        if (!pstep(sb, sa, kt1, kt0, vt1, vt0, ps1, ps0)) break;
      }
    } else {
    // key-position slots of the two tile buffers (phase B, which uses clist, never runs on BLOCK heads)
    uint32_t* ps0 = sm.clist;
    uint32_t* ps1 = sm.clist + kBlock;
    bool have = next_tile(c_cur, m_cur, e0_cur, e1_cur);
    if (have) issue_tile(c_cur, kt0, vt0, ps0);
    if ((XK & kXkPos) && posm && have) bm_cur = hd.blkmax[c_cur];
    wait_vmem();
    __syncthreads();
    while (have) {
      if (!step(kt0, vt0, ps0, kt1, vt1, ps1)) break;
      have = step(kt1, vt1, ps1, kt0, vt0, ps0);
    }
    }
  }

  // ---------------- phase B: gathered vertical columns (VS and VS window heads)
  if ((hd.kind == KIND_VS || ((XK & kXkWin) && hd.kind == KIND_VSW)) && hd.k_v > 0) {
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
            int m0, m1;
            if ((XK & kXkWin) && hd.kind == KIND_VSW) {
              // outside the block's windows: no offset dl with 64b - dl <= j <= 64b - dl + 63
              m0 = cb <= b0 && !any_offset(hd.dbits, b0 * kBlock - j, n);
              m1 = has_b1 && cb <= b1 && !any_offset(hd.dbits, b1 * kBlock - j, n);
            } else {
              m0 = cb <= b0 && !bit_at(it.bits0, b0 - cb);
              m1 = has_b1 && cb <= b1 && !bit_at(it.bits1, b1 - cb);
            }
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
        // padding slots load row 0 (a valid row) and are never visible
        auto rows_of = [&](int t) {
          return [&, t](int x) -> int {
            const int s = t * kBlock + x;
            return s < kept ? (int)(sm.clist[s] & 0x3fffffffu) : 0;
          };
        };
        auto gstep = [&](int t, uint16_t* ktc, uint16_t* vtc, uint16_t* ktn, uint16_t* vtn) {
          if (t + 1 < ntile) issue_rows(kr, vr, ktn, vtn, rows_of(t + 1));
          if (wave_on) {
            // skip the tile when none of its columns belongs to this wave's query block
            // (padding slots were cleared, so they never count)
            const uint32_t* gc = sm.clist + t * kBlock;
            if (__any((gc[lane] >> (30 + qsel)) & 1u))
              compute_tile<XK>(ws, oo, ktc, vtc, MASK_GATHER, 0, gc, qsel, row, n, 1, 0, 0, 0, sl2);
          }
          wait_vmem();
          __syncthreads();
        };
        issue_rows(kr, vr, kt0, vt0, rows_of(0));
        wait_vmem();
        __syncthreads();
        for (int t = 0; t < ntile; t += 2) {
          gstep(t, kt0, vt0, kt1, vt1);
          if (t + 1 < ntile) gstep(t + 1, kt1, vt1, kt0, vt0);
        }
      }
      if (any_past) break;
    }
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
    if (p.lse && g == 0) {
      p.lse[(size_t)h * n + row] = ltot > 0.f ? (ws.m + __log2f(ltot)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

// The 64 workgroups of one XCD wait for each other between rounds: a counter
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

// XCD-aware work order. Workgroup L runs on XCD L % 8; that XCD's k-th
// workgroup takes item (k / C * 8 + L % 8) * C + k % C, so each XCD works
// through whole chunks of C consecutive items, C = 64 being what one XCD holds
// at once (32 CUs x 2 workgroups): the workgroups resident on an XCD stream
// the same K/V tiles through its L2.
template <int XK>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(const AttnLaunch p) {
  __shared__ Smem sm;
  __shared__ __attribute__((aligned(16))) uint16_t kt0[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t kt1[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t vt0[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t vt1[kTileHalves];
  // when a rounds launch of the same work was queued beside this one, only one of them works
  if (p.rounds_flag != nullptr && *p.rounds_flag != 0) return;
  const int slot = blockIdx.x >> 3;
  const int xcd = (int)(blockIdx.x & (kXcds - 1));
  attn_item<XK>(p, ((slot / kChunk) * kXcds + xcd) * kChunk + slot % kChunk, sm, kt0, kt1, vt0, vt1);
}

// Rounds variant: exactly 8 x 64 workgroups, as many as the device holds at
// once (two per CU), so that they are resident together. In round r workgroup L takes item
// (r * 8 + L % 8) * C + L / 8, and the 64 workgroups of an XCD start every
// round together: long items (thousands of key tiles) then stay near the same
// key position and keep sharing K/V tiles in that XCD's L2. It works only
// when *p.rounds_flag is set (the flag is computed on the device from the
// offset bitmaps); otherwise the ordinary launch queued after it does.
template <int XK>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel_rounds(const AttnLaunch p) {
  __shared__ Smem sm;
  __shared__ __attribute__((aligned(16))) uint16_t kt0[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t kt1[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t vt0[kTileHalves];
  __shared__ __attribute__((aligned(16))) uint16_t vt1[kTileHalves];
  if (*p.rounds_flag == 0) return;
  const int slot = blockIdx.x >> 3;
  const int xcd = (int)(blockIdx.x & (kXcds - 1));
  for (int r = 0; r < p.rounds; ++r) {
    attn_item<XK>(p, (r * kXcds + xcd) * kChunk + slot, sm, kt0, kt1, vt0, vt1);
    xcd_barrier(p.xcd_sync + xcd, kChunk * (r + 1));
  }
}

__global__ void zero_counters_kernel(int32_t* c, int n, int32_t* flag_on) {
  if ((int)threadIdx.x < n) c[threadIdx.x] = 0;
  if (flag_on != nullptr && threadIdx.x == 0) *flag_on = 1;
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
  const int32_t* wcount[kMaxLaunchHeads];  // rounds flag: tile counts of VS window heads
  int32_t n, nb, nw;
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

template <int XK>
static const void* rounds_kernel() { return (const void*)attn_kernel_rounds<XK>; }
static const void* rounds_kernel_of(int xk) {
  switch (xk) {
    case 1: return rounds_kernel<1>();
    case 2: return rounds_kernel<2>();
    case 3: return rounds_kernel<3>();
    default: return rounds_kernel<0>();
  }
}

// Whether this device holds all 8 x 64 workgroups of a rounds launch at once
// (at least two per CU on at least 256 CUs). The launch is an ordinary one: its
// per-XCD waits are bounded, so it ends even if some workgroups were not
// resident together (only the L2 sharing would suffer). Asked once per device
// and instantiation.
static bool rounds_supported(int xk) {
  static int cache[4][64] = {};  // 0 unknown, 1 yes, 2 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  int& c = cache[xk & 3][dev];
  if (c == 0) {
    int cus = 0, per_cu = 0;
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, rounds_kernel_of(xk), kThreads, 0);
    c = (e == hipSuccess && (long long)cus * per_cu >= kXcds * kChunk) ? 1 : 2;
  }
  return c == 1;
}

hipError_t launch_attn(const AttnLaunch& a, hipStream_t stream) {
  const int npairs = (a.nb + 1) / 2;
  if (npairs <= 0 || a.nh <= 0 || a.hgroup <= 0 || a.nh % a.hgroup != 0 || kChunk % a.hgroup != 0)
    return hipErrorInvalidValue;
  const int ppc = kChunk / a.hgroup;
  const long long chunks = (long long)((npairs + ppc - 1) / ppc) * (a.nh / a.hgroup);
  // the grid covers whole rounds of kXcds chunks so that the item map is a bijection
  const long long grid = (chunks + kXcds - 1) / kXcds * kXcds * kChunk;
  int xk = 0;
  for (int i = 0; i < a.nh; ++i) {
    if (a.heads[i].pos != nullptr) xk |= kXkPos;
    if (a.heads[i].kind == KIND_VSW) xk |= kXkWin;
  }
  AttnLaunch c = a;
  c.xcd_sync = nullptr;
  c.rounds_flag = nullptr;
  if (a.xcd_sync != nullptr && a.rounds_flag != nullptr && rounds_supported(xk)) {
    // the rounds launch, then the ordinary one; the device-side flag lets exactly one of them work
    AttnLaunch b = a;
    b.rounds = (int)((chunks + kXcds - 1) / kXcds);
    hipLaunchKernelGGL(zero_counters_kernel, dim3(1), dim3(64), 0, stream, b.xcd_sync, kXcds, b.rounds_flag_set);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 gr(kXcds * kChunk), tr(kThreads);
    switch (xk) {
      case 1: hipLaunchKernelGGL(attn_kernel_rounds<1>, gr, tr, 0, stream, b); break;
      case 2: hipLaunchKernelGGL(attn_kernel_rounds<2>, gr, tr, 0, stream, b); break;
      case 3: hipLaunchKernelGGL(attn_kernel_rounds<3>, gr, tr, 0, stream, b); break;
      default: hipLaunchKernelGGL(attn_kernel_rounds<0>, gr, tr, 0, stream, b); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    c.rounds_flag = a.rounds_flag;
  }
  const dim3 g((unsigned)grid), t(kThreads);
  switch (xk) {
    case 1: hipLaunchKernelGGL(attn_kernel<1>, g, t, 0, stream, c); break;
    case 2: hipLaunchKernelGGL(attn_kernel<2>, g, t, 0, stream, c); break;
    case 3: hipLaunchKernelGGL(attn_kernel<3>, g, t, 0, stream, c); break;
    default: hipLaunchKernelGGL(attn_kernel<0>, g, t, 0, stream, c); break;
  }
  return hipGetLastError();
}

// Rounds pay off when the work items are long: flag = 1 when the listed VS
// heads' offset sets O u (O + 1), and the listed VS window heads' tile covers,
// hold on average at least `min_tiles` tiles (the tile count of the longest
// query-block pairs). One workgroup of 1024 threads walks every head's bitmap
// words as one flat index space.
__global__ __launch_bounds__(1024) void rounds_flag_kernel(const OffBitsLaunch a, int count, int min_tiles,
                                                           int32_t* flag) {
  __shared__ unsigned long long tot;
  if (threadIdx.x == 0) tot = 0;
  __syncthreads();
  const int nwords = (a.nb >> 5) + 1;
  const int total = count * nwords;
  unsigned long long mine = 0;
#pragma unroll 4
  for (int x = threadIdx.x; x < total; x += 1024) {
    const int h = x / nwords;
    const int i = x - h * nwords;
    const uint32_t* w = a.bits[h];
    const uint32_t prev = i > 0 ? w[i - 1] : 0u;
    mine += (unsigned long long)__popc(w[i] | (w[i] << 1) | (prev >> 31));
  }
  if ((int)threadIdx.x < a.nw) mine += (unsigned long long)*a.wcount[threadIdx.x];
  atomicAdd(&tot, mine);
  __syncthreads();
  const int heads = count + a.nw;
  if (threadIdx.x == 0) *flag = (heads > 0 && tot >= (unsigned long long)min_tiles * heads) ? 1 : 0;
}

hipError_t launch_rounds_flag(uint32_t* const* bits, int count, const int32_t* const* wcount, int nw, int n,
                              int min_tiles, int32_t* flag, hipStream_t stream) {
  OffBitsLaunch a{};
  const int c = count < kMaxLaunchHeads ? count : kMaxLaunchHeads;
  for (int i = 0; i < c; ++i) a.bits[i] = bits[i];
  a.nw = nw < kMaxLaunchHeads ? nw : kMaxLaunchHeads;
  for (int i = 0; i < a.nw; ++i) a.wcount[i] = wcount[i];
  a.n = n;
  a.nb = (n + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(rounds_flag_kernel, dim3(1), dim3(1024), 0, stream, a, c, min_tiles, flag);
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
