// Per-wave tile arithmetic of the sparse FlashAttention kernels (gfx950,
// internal header): one wave64 holds 32 query rows and works on 64-key tiles
// staged in LDS. S^T = K Q^T and O^T += V^T P^T run on 32x32x16 bf16 MFMA, so a
// lane owns one query row in both accumulators and the online-softmax
// recurrence (MInference 1.0 article, "Latency and sparse patterns in
// kernels": FlashAttention over the selected blocks) is lane-local.
#pragma once

#include "common.h"

namespace minf {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Chunk swizzle of a tile row: the 16-byte chunk c of row r sits at chunk
// position c ^ swz(r), swz swapping the two 2-bit halves of r mod 16. It is a
// bijection on 16 consecutive rows (the K operand reads 16 rows at one chunk:
// 16 distinct bank groups), and 4 consecutive rows get 4 distinct values of
// bits 2-3 (the V transpose reads touch 4 rows x 4 aligned chunks: 16
// distinct bank groups).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Per-lane LDS byte offsets of the MFMA operands inside a tile.
struct OperandOffsets {
  int k;       // K row r32, chunk (g ^ swz): chunk 2ks + g of the row is at k ^ (ks << 5)
  int v[4][2]; // V transpose reads: d block mt, key half h (+ 4096 per 16-key step)
};

__device__ __forceinline__ OperandOffsets operand_offsets() {
  OperandOffsets o;
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int r32 = lane & 31;
  // (2ks + g) ^ swz = (g ^ swz) ^ 2ks, and the chunk field (bits 4-7) does not overlap the row bits
  o.k = r32 * 256 + ((g ^ swz(r32)) << 4);
  // ds_read_b64_tr_b16 source lane i of 16-lane group G supplies the 4 halves
  // V[kb + i/4][dbase + 4(i%4) ..]; lane i then receives V[kb + e][dbase + i], e = 0..3.
  const int G = lane >> 4;
  const int i = lane & 15;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * h + 4 * g + (i >> 2);             // + 16 kk at read time
      const int chunk = 4 * mt + 2 * (G & 1) + ((i >> 1) & 1);  // d = 32 mt + 16 (G & 1) + 4 (i & 3)
      o.v[mt][h] = row * 256 + ((chunk ^ swz(row)) << 4) + 8 * (i & 1);
    }
  return o;
}

struct WaveState {
  u32x4 qr[8];     // this wave's 32 query rows as MFMA B operands (8 k-steps over d)
  f32x16 o[4];     // O^T accumulators: d = 32*mt + ..., column = query row
  float m, l;      // running max (log2 units) and this lane's partial sum
};

// The 64-wide accumulator rescale runs only on tiles where some row of the
// wave raises its running max (alpha == 1 otherwise, so skipping it is exact).
// Keeping the max exact (no slack) keeps the dominant probability exactly 1.0
// in bf16, which the 2e-2 output bar needs when |O| approaches 8.
constexpr float kRescaleSlack = 0.0f;

// S^T = K Q^T for one tile: two independent accumulation chains (keys 0-31, 32-63), interleaved.
__device__ __forceinline__ void qk_tile(const WaveState& ws, const OperandOffsets& oo, const uint16_t* kt,
                                        f32x16 (&s)[2]) {
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
  s[0] = s0;
  s[1] = s1;
}

// Running-max update for one tile's scores. Sets m to the new max and scales
// l by alpha = 2^(m_old - m_new) (exactly 1 when no row of this lane rose);
// the O accumulators are scaled separately, only when some row of the wave
// rose (`raise`), since alpha == 1 everywhere else.
struct TileStats {
  float alpha, m_use;
  bool raise;
};
__device__ __forceinline__ TileStats tile_stats(WaveState& ws, const f32x16 (&s)[2], float sl2) {
  float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[0][i], s[1][i]));
  const float m_tile = pair_max32(mx) * sl2;
  TileStats t;
  t.raise = __any(m_tile > ws.m + kRescaleSlack);
  const float m_new = fmaxf(ws.m, m_tile);
  t.alpha = fast_exp2(ws.m - (m_new == -INFINITY ? 0.f : m_new));
  {
    // a multiply of its own (not fused with the later += of the tile's sum)
#pragma clang fp contract(off)
    ws.l *= t.alpha;
  }
  ws.m = m_new;
  t.m_use = m_new == -INFINITY ? 0.f : m_new;
  return t;
}

__device__ __forceinline__ void rescale_o(WaveState& ws, float alpha) {
  // keeps the rescale a real branch: its body cannot be speculated into a select
  asm volatile("" : "+v"(alpha));
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) ws.o[mt] *= alpha;
}

// bf16 probabilities of 16 scores (one 32-key half of the tile) as two MFMA
// operands, and their sum (in the order the PV product consumes them: one
// v_dot2_f32_bf16 per packed pair, so the weights sum to exactly one after
// normalisation).
__device__ __forceinline__ void probs_half(const f32x16& s, float m_use, float sl2, u32x4& pa, u32x4& pb,
                                           float& psum) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(s[8 * h + e], sl2, -m_use));
    const u32x4 w = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7])};
    if (h == 0)
      pa = w;
    else
      pb = w;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) psum = sum_bf16x2(pa[w], psum);
#pragma unroll
  for (int w = 0; w < 4; ++w) psum = sum_bf16x2(pb[w], psum);
}

// O^T += V^T P^T for 16 keys (k-step kk): four independent accumulation chains (d = 0-31, ..., 96-127).
__device__ __forceinline__ void pv_step(WaveState& ws, const OperandOffsets& oo, const char* vb, int kk,
                                        const u32x4& p) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)((lds_ptr)(vb + oo.v[mt][0] + 4096 * kk)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)((lds_ptr)(vb + oo.v[mt][1] + 4096 * kk)));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    ws.o[mt] = mfma32(u32x4{l2[0], l2[1], h2[0], h2[1]}, p, ws.o[mt]);
  }
}

// Softmax of an already masked tile followed by its PV product (no overlap).
__device__ __forceinline__ void softmax_pv(WaveState& ws, const OperandOffsets& oo, const f32x16 (&s)[2],
                                           const uint16_t* vt, float sl2) {
  const TileStats st = tile_stats(ws, s, sl2);
  if (st.raise) rescale_o(ws, st.alpha);
  u32x4 pk[4];
  float psum = 0.f;
  probs_half(s[0], st.m_use, sl2, pk[0], pk[1], psum);
  probs_half(s[1], st.m_use, sl2, pk[2], pk[3], psum);
  ws.l += psum;
  const char* vb = (const char*)vt;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) pv_step(ws, oo, vb, kk, pk[kk]);
}

// Software pipeline of a wave over consecutive tiles t, t + 1 (both used by
// the wave). After tile t's row statistics (and the rare rescale of O), the
// scores of tile t + 1 are formed on the matrix cores while the vector ALUs
// form tile t's probabilities, then tile t's PV product runs. The order is
// written out step by step and fenced (sched_barrier), so the compiler keeps
// it: each 32x32x16 product is followed by the LDS read of the operand four
// products ahead and by one pair of probabilities (two exp2, one bf16 pack,
// one dot2 of the row sum), which execute in the product's shadow. The two
// score chains alternate as in qk_tile, the row-sum chain and the PV
// accumulation run in softmax_pv's order: the results are bitwise the same.
constexpr int kReadAhead = 4;
__device__ __forceinline__ void fused_tile_pair(WaveState& ws, const OperandOffsets& oo, const f32x16 (&sc)[2],
                                                const uint16_t* ktn, const uint16_t* vtc, f32x16 (&sn)[2],
                                                float sl2) {
  const TileStats st = tile_stats(ws, sc, sl2);
  if (st.raise) rescale_o(ws, st.alpha);
  const char* kb = (const char*)ktn;
  const char* vb = (const char*)vtc;
  // operand of QK product j = 2 ks + half (keys 32 half .. +31, d 16 ks .. +15)
  auto kread = [&](int j) -> u32x4 { return *(const u32x4*)(kb + (oo.k ^ ((j >> 1) << 5)) + (j & 1) * 32 * 256); };
  // operand of PV product j = 4 kk + mt (keys 16 kk .. +15, d 32 mt .. +31)
  auto vread = [&](int j) -> u32x4 {
    const int kk = j >> 2, mt = j & 3;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)((lds_ptr)(vb + oo.v[mt][0] + 4096 * kk)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)((lds_ptr)(vb + oo.v[mt][1] + 4096 * kk)));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    const u32x2 h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };
  u32x4 kop[16], vop[16], pk[4];
  f32x16 n0 = f32x16{}, n1 = f32x16{};
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < kReadAhead; ++j) kop[j] = kread(j);
  // raised issue priority while the wave feeds the matrix cores: when both
  // waves of a SIMD are ready, the one in this section issues first
  __builtin_amdgcn_s_setprio(1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j & 1)
      n1 = mfma32(kop[j], ws.qr[j >> 1], n1);
    else
      n0 = mfma32(kop[j], ws.qr[j >> 1], n0);
    if (j + kReadAhead < 16)
      kop[j + kReadAhead] = kread(j + kReadAhead);
    else
      vop[j + kReadAhead - 16] = vread(j + kReadAhead - 16);
    // probability pair j: word j & 3 of operand pk[j >> 2], from keys 8 h + 2 w, +1 of score half mt
    const int q = j >> 2, w = j & 3, mt = q >> 1, h = q & 1;
    const float p0 = fast_exp2(fmaf(sc[mt][8 * h + 2 * w], sl2, -st.m_use));
    const float p1 = fast_exp2(fmaf(sc[mt][8 * h + 2 * w + 1], sl2, -st.m_use));
    pk[q][w] = pack_bf16x2(p0, p1);
    psum = sum_bf16x2(pk[q][w], psum);
    asm volatile("" : "+v"(psum));  // keeps the row-sum step in this product's shadow
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    ws.o[j & 3] = mfma32(vop[j], pk[j >> 2], ws.o[j & 3]);
    if (j + kReadAhead < 16) vop[j + kReadAhead] = vread(j + kReadAhead);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_setprio(0);
  ws.l += psum;
  sn[0] = n0;
  sn[1] = n1;
}

}  // namespace
}  // namespace minf
