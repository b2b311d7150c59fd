// Internal host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace minf {

constexpr int kMaxLaunchHeads = 32;  // heads described in one attention launch (kernel arguments)
constexpr int kMaxVsGroups = 32;     // VS head groups in one index launch
constexpr int64_t kMaxTokens = 1 << 20;  // largest n the in-LDS bitmaps cover (16384 blocks)

struct AttnHead {
  int32_t kind, sink, local, k_v, k_b, head;  // head: the query head this entry describes
  const int32_t* v_idx;    // VS: ascending columns
  const uint32_t* obits;   // VS: bitmap of block offsets covered by the slashes
  const int32_t* blk_idx;  // BLOCK
  const int32_t* blk_cnt;  // BLOCK
  const int32_t* pos;      // BLOCK on a permuted sequence: original position of every row (else null)
  const int32_t* blkmax;   // with pos: latest original position in every key block
  const int2* wtiles;      // VS windows: tile cover of the windows relative to a block's first row
  const int32_t* wcount;   // VS windows: number of tiles (device)
  const uint32_t* dbits;   // VS windows: bitmap of the slash offsets over [0, n)
};

constexpr int kRoundXcds = 8;  // XCDs of an MI355X: one barrier counter each in a rounds launch

struct AttnLaunch {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int32_t n, nb, hq, hkv, grp, nh, causal;
  int32_t hgroup;  // heads per work chunk: divides nh and 64; consecutive heads (they share K/V when
                   // they fall in one GQA group)
  float scale_log2;
  int32_t* xcd_sync;          // per-XCD barrier counters (kRoundXcds ints) for a rounds launch, else null
  const int32_t* rounds_flag;  // device flag: 1 = the rounds launch works, 0 = the ordinary launch does
  int32_t* rounds_flag_set;    // non-null: set to 1 before the launches (a launch known to take rounds)
  int32_t rounds;              // set by launch_attn
  AttnHead heads[kMaxLaunchHeads];
};

hipError_t launch_attn(const AttnLaunch& a, hipStream_t stream);
hipError_t launch_vs_offset_bits(const int32_t* const* s_idx, const int32_t* k_s, uint32_t* const* bits,
                                 int count, int n, hipStream_t stream);
// flag = 1 when the VS heads' offset bitmaps and the VS window heads' tile counts (up to 32 each)
// average at least min_tiles tiles per item
hipError_t launch_rounds_flag(uint32_t* const* bits, int count, const int32_t* const* wcount, int nw, int n,
                              int min_tiles, int32_t* flag, hipStream_t stream);

// Slash-aligned window preparation for up to kMaxLaunchHeads heads.
struct VswLaunch {
  const int32_t* s_idx[kMaxLaunchHeads];
  int32_t k_s[kMaxLaunchHeads];
  uint32_t* dbits[kMaxLaunchHeads];  // [(n + 31) / 32]
  int2* tiles[kMaxLaunchHeads];      // [cap]
  int32_t* count[kMaxLaunchHeads];   // [1]
  int32_t n, cap;
};
int vsw_tile_capacity(int n);
hipError_t launch_vsw_prepare(const VswLaunch& a, int count, int max_k_s, hipStream_t stream);

struct VsGroup {
  int32_t kv;        // KV head of the group
  int32_t cnt;       // query heads in the group (1..4)
  int32_t head[4];   // query head ids
  int32_t slot[4];   // output slots (position in the caller's head list)
};

struct VsLaunch {
  const uint16_t* q;
  const uint16_t* k;
  int32_t n, r, ngroups, nchunks, tiles_per_chunk, ntiles, n_slots;
  float scale_log2;
  float* part_m;   // [n_slots][64][nchunks]
  float* part_l;   // [n_slots][64][nchunks]
  float* row_m;    // [n_slots][64]
  float* row_il;   // [n_slots][64]
  float* vcol;     // [n_slots][n]
  float* slsum;    // [n_slots][n]
  float* dedge;    // [n_slots][nchunks][128]: diagonals e = 0..62 of a chunk's last tile, e = 64..126 of its first
  VsGroup groups[kMaxVsGroups];
};

hipError_t launch_vs_scores(const VsLaunch& a, hipStream_t stream);

// Top-k (ties to the lower index, ascending output) of every row of up to two
// row sets with a common row length n, split over chunks of `chunk` entries.
struct TopkSeg {
  const float* src;  // row i at src + i * src_stride
  int32_t* dst;      // row i at dst + i * dst_stride, k entries
  int64_t src_stride, dst_stride;
  int32_t rows, k;
};
struct TopkLaunch {
  TopkSeg seg[2];
  int32_t n, chunk, nchunks;
  int32_t* hist;   // [rows][2048] scratch histograms
  int32_t* state;  // [rows][4] prefix, prefix mask, rank left
  int32_t* cnt;    // [rows][2][nchunks * 4] keys above / equal to the threshold per chunk quarter
};
int topk_chunk_len(int n);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream);

// Pool heads[i] of x ([h][n][128] bf16) into slot slots[i] of out_rm ([slot][nb][128])
// and/or out_t ([slot][128][nb]); either output may be null. Blocks below
// first_block are left untouched.
hipError_t launch_block_pool(const uint16_t* x, int n, const int32_t* heads, const int32_t* slots, int n_heads,
                             float* out_rm, float* out_t, hipStream_t stream, int first_block = 0,
                             const int32_t* col_map = nullptr);

// Decoding: one query row per head against a cache of n keys.
constexpr int kDecMaxBlocks = 16384;  // n_b limit of the single-workgroup block top-k
struct DecodeLaunch {
  const uint16_t* q;     // [hq][128]
  const uint16_t* k;     // [hkv][n][128]
  const uint16_t* v;
  const float* kbar_t;   // [hkv][128][nb] block means of K
  float* scores;         // [hq][nb]
  int32_t* blk;          // [hq][kb] selected blocks; null: entry e is block e (dense)
  float* part;           // [hq][nsplit][130]: max (log2 units), sum, o[128]
  uint16_t* o;           // [hq][128]
  float* lse;            // [hq] or null
  // segmented top-k (null when a single workgroup per head selects): per head
  // and segment the segment's top-kb keys and block ids, and their count
  uint32_t* seg_key;     // [hq][nseg][kb]
  int32_t* seg_id;       // [hq][nseg][kb]
  int32_t* seg_cnt;      // [hq][nseg]
  int32_t n, nb, hq, hkv, grp, kb, nsplit, bps, nseg;
  float scale_log2;
};
constexpr int kDecSeg = 2048;      // candidate blocks per top-k segment
constexpr int kDecSegMaxK = 256;   // largest k_b served by the segmented top-k
// Segments of the segmented decode top-k for n_b blocks and k_b (0: one workgroup per head).
inline int decode_topk_segments(int nb, int kb) {
  return (nb > kDecSeg && kb <= kDecSegMaxK) ? (nb + kDecSeg - 1) / kDecSeg : 0;
}
int decode_blocks_per_split(int kb, int rows);
hipError_t launch_iota_rows(int32_t* dst, int rows, int cols, hipStream_t stream);
hipError_t launch_decode(const DecodeLaunch& a, bool select, hipStream_t stream);
// Orders of the blocks of a permuted sequence (positions distinct): ranks by
// earliest / latest original position and each query rank's eligible count.
struct PermRankLaunch {
  const int32_t* bmin;  // [nb] earliest original position of every block
  const int32_t* bmax;  // [nb] latest
  uint32_t* bits_min;   // [words] bitmap of the earliest positions over [0, n)
  uint32_t* bits_max;   // [words] bitmap of the latest positions
  int32_t* pre_min;     // [words] set bits of bits_min before each word
  int32_t* pre_max;     // [words]
  int32_t* rank_q;      // [nb] rank of block b by latest position
  int32_t* rank_k;      // [nb] rank of block c by earliest position
  int32_t* tau;         // [nb] block of query rank r
  int32_t* sigma;       // [nb] block of key rank s
  int32_t* lrow;        // [nb] key blocks whose earliest position <= the latest of query rank r
  int32_t n, nb, words;
};
hipError_t launch_perm_ranks(const PermRankLaunch& a, hipStream_t stream);
// Scores and top-k for n_heads pooled query heads (qbar_t slots 0..n_heads-1, each
// [128][nb]), head i reading pooled keys kbar_t slot kvslot[i] ([128][nb]); writes
// blk_idx/blk_cnt slot i. Permuted sequences pass lrow / sigma / tau (with the pooled
// columns in rank order: query blocks by rank_q, key blocks by rank_k), else null.
int block_score_rows(int nb, int n_heads);
hipError_t launch_block_topk(const float* qbar_t, const float* kbar_t, const int32_t* kvslot, int n_heads, int nb,
                             int k_b, int32_t* blk_idx, int32_t* blk_cnt, float* scores, int rows,
                             const int32_t* lrow, const int32_t* sigma, const int32_t* tau, hipStream_t stream);
// Per-block min / max of the original positions of a permuted sequence.
hipError_t launch_block_minmax(const int32_t* pos, int n, int32_t* bmin, int32_t* bmax, hipStream_t stream);
// Gather (scatter = 0) or scatter (1) rows of row_bytes bytes of [heads][n] data by src.
hipError_t launch_permute_rows(const void* x, void* out, int heads, int64_t n, int row_bytes, const int32_t* src,
                               int scatter, hipStream_t stream);

// Work of plans in the sparse kernel's unit, and attention recall (pattern search).
enum : int32_t { KIND_W_DENSE = 0, KIND_W_ASHAPE = 1, KIND_W_VS = 2, KIND_W_BLOCK = 3 };
struct WorkHead {
  int32_t kind, sink, local, k_v;
  const int32_t* v_idx;    // VS: ascending columns
  const uint32_t* obits;   // VS: block-offset bitmaps (full blocks, then a partial last block)
  const int32_t* blk_cnt;  // BLOCK
};
struct WorkLaunch {
  WorkHead heads[kMaxLaunchHeads];
  int32_t n, nb;
  double* out;  // [count] work of each head, in 64x64 blocks
};
hipError_t launch_plan_work(const WorkLaunch& a, int count, hipStream_t stream);
hipError_t launch_recall(const float* lse_mask, const float* lse_dense, int n, int hq, const int32_t* rows,
                         int n_rows, double* out, hipStream_t stream);

}  // namespace minf
