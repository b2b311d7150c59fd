// C ABI of the library: argument validation, workspace carving, launches.
// Every check runs before the first launch; a failed check launches nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/minf.h"
#include "common.h"
#include "launch.h"

using namespace minf;

namespace {

thread_local std::string g_detail;

minf_status fail(minf_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return s;
}

minf_status hip_fail(hipError_t e, const char* where) {
  return fail(MINF_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Carver {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t count) {
    T* p = (T*)(base + off);
    off = align_up(off + count * sizeof(T));
    return p;
  }
};

int64_t nblocks(int64_t n) { return (n + kBlock - 1) / kBlock; }

minf_status check_common(const void* q, const void* k, int64_t n, int hq, int hkv, int d, int64_t max_n) {
  if (!q || !k) return fail(MINF_E_INVALID_ARG, "q and k must be non-null device pointers");
  if (n < 1) return fail(MINF_E_INVALID_ARG, "n must be >= 1 (got %lld)", (long long)n);
  if (hq < 1 || hkv < 1) return fail(MINF_E_INVALID_ARG, "hq and hkv must be >= 1");
  if (hq % hkv != 0) return fail(MINF_E_INVALID_ARG, "hq (%d) must be a multiple of hkv (%d)", hq, hkv);
  if (d != kHeadDim) return fail(MINF_E_UNSUPPORTED, "head dim %d is not supported (only 128)", d);
  if (n > max_n) return fail(MINF_E_UNSUPPORTED, "n = %lld exceeds the supported %lld", (long long)n, (long long)max_n);
  return MINF_OK;
}

minf_status check_scale(float scale) {
  if (!(scale > 0.f) || !isfinite(scale)) return fail(MINF_E_INVALID_ARG, "scale must be finite and > 0");
  return MINF_OK;
}

minf_status check_heads(const int32_t* heads, int n_heads, int hq) {
  if (n_heads < 0) return fail(MINF_E_INVALID_ARG, "n_heads must be >= 0");
  if (n_heads > 0 && !heads) return fail(MINF_E_INVALID_ARG, "heads must be a host array of n_heads ids");
  std::vector<char> seen(hq, 0);
  for (int i = 0; i < n_heads; ++i) {
    if (heads[i] < 0 || heads[i] >= hq) return fail(MINF_E_INVALID_ARG, "heads[%d] = %d out of [0, %d)", i, heads[i], hq);
    if (seen[heads[i]]) return fail(MINF_E_INVALID_ARG, "head %d listed twice", heads[i]);
    seen[heads[i]] = 1;
  }
  return MINF_OK;
}

minf_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MINF_OK;
  if (!ws) return fail(MINF_E_WORKSPACE, "workspace is null but %zu bytes are required", need);
  if (((uintptr_t)ws) % 16 != 0) return fail(MINF_E_WORKSPACE, "workspace must be 16-byte aligned");
  if (ws_bytes < need) return fail(MINF_E_WORKSPACE, "workspace has %zu bytes, %zu required", ws_bytes, need);
  return MINF_OK;
}

// ---------------- VS workspace
int vs_max_chunks(int64_t n) { return (int)std::min<int64_t>(nblocks(n), 2048); }

struct VsWs {
  float *part_m, *part_l, *row_m, *row_il, *vcol, *slsum, *dedge;
  int32_t *tk_hist, *tk_state, *tk_cnt;
  int tk_chunk, tk_nchunks;
  size_t bytes;
};

VsWs carve_vs(void* base, int64_t n, int n_heads) {
  Carver c{(char*)base};
  const size_t nh = (size_t)std::max(n_heads, 1);
  const size_t mc = (size_t)vs_max_chunks(n);
  VsWs w;
  w.part_m = c.take<float>(nh * 64 * mc);
  w.part_l = c.take<float>(nh * 64 * mc);
  w.row_m = c.take<float>(nh * 64);
  w.row_il = c.take<float>(nh * 64);
  w.vcol = c.take<float>(nh * (size_t)n);
  w.slsum = c.take<float>(nh * (size_t)n);
  w.dedge = c.take<float>(nh * mc * 128);
  // top-k scratch for the two score rows of every head
  w.tk_chunk = topk_chunk_len((int)std::min<int64_t>(n, 1 << 30));
  w.tk_nchunks = (int)((n + w.tk_chunk - 1) / w.tk_chunk);
  w.tk_hist = c.take<int32_t>(2 * nh * 2048);
  w.tk_state = c.take<int32_t>(2 * nh * 4);
  w.tk_cnt = c.take<int32_t>(2 * nh * 2 * 4 * (size_t)w.tk_nchunks);
  w.bytes = c.off;
  return w;
}

minf_status run_vs_scores(const void* q, const void* k, int64_t n, int hq, int hkv, const int32_t* heads,
                          int n_heads, int last_q, float scale, const VsWs& w, hipStream_t stream) {
  const int grp = hq / hkv;
  // group the listed heads by KV head, at most 4 per group (one wave each)
  std::vector<VsGroup> groups;
  for (int kv = 0; kv < hkv; ++kv) {
    VsGroup cur{};
    cur.kv = kv;
    for (int i = 0; i < n_heads; ++i) {
      if (heads[i] / grp != kv) continue;
      cur.head[cur.cnt] = heads[i];
      cur.slot[cur.cnt] = i;
      if (++cur.cnt == 4) {
        groups.push_back(cur);
        cur = VsGroup{};
        cur.kv = kv;
      }
    }
    if (cur.cnt) groups.push_back(cur);
  }
  const int ntiles = (int)nblocks(n);
  for (size_t g0 = 0; g0 < groups.size(); g0 += kMaxVsGroups) {
    VsLaunch a{};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.n = (int)n;
    a.r = (int)std::min<int64_t>(last_q, n);
    a.ngroups = (int)std::min<size_t>(kMaxVsGroups, groups.size() - g0);
    const int want = std::max(1, (2048 + a.ngroups - 1) / a.ngroups);
    int nch = std::min(std::min(want, ntiles), vs_max_chunks(n));
    a.tiles_per_chunk = (ntiles + nch - 1) / nch;
    a.nchunks = (ntiles + a.tiles_per_chunk - 1) / a.tiles_per_chunk;
    a.ntiles = ntiles;
    a.n_slots = n_heads;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.part_m = w.part_m;
    a.part_l = w.part_l;
    a.row_m = w.row_m;
    a.row_il = w.row_il;
    a.vcol = w.vcol;
    a.slsum = w.slsum;
    a.dedge = w.dedge;
    for (int i = 0; i < a.ngroups; ++i) a.groups[i] = groups[g0 + i];
    hipError_t e = launch_vs_scores(a, stream);
    if (e != hipSuccess) return hip_fail(e, "VS score kernels");
  }
  return MINF_OK;
}

minf_status check_vs_args(const void* q, const void* k, int64_t n, int hq, int hkv, int d, const int32_t* heads,
                          int n_heads, int last_q, float scale, void* ws, size_t ws_bytes) {
  minf_status s;
  if ((s = check_common(q, k, n, hq, hkv, d, kMaxTokens)) != MINF_OK) return s;
  if ((s = check_scale(scale)) != MINF_OK) return s;
  if ((s = check_heads(heads, n_heads, hq)) != MINF_OK) return s;
  if (last_q < 1) return fail(MINF_E_INVALID_ARG, "last_q must be >= 1");
  if (last_q > 64) return fail(MINF_E_UNSUPPORTED, "last_q > 64 is not supported");
  if (n_heads == 0) return MINF_OK;
  return check_ws(ws, ws_bytes, minf_vs_index_workspace_size(n, n_heads));
}

// ---------------- BS workspace
struct BsWs {
  float *qbar_t, *kbar_t, *scores;
  int32_t *blkmin, *blkmax;
  // permuted sequences: the block orders (PermRankLaunch)
  uint32_t *bits_min, *bits_max;
  int32_t *pre_min, *pre_max, *rank_q, *rank_k, *tau, *sigma, *lrow;
  int words;
  int rows;
  size_t bytes;
};

BsWs carve_bs(void* base, int64_t n, int hkv, int n_heads) {
  Carver c{(char*)base};
  const size_t nb = (size_t)nblocks(n);
  BsWs w;
  w.qbar_t = c.take<float>((size_t)std::max(n_heads, 1) * nb * kHeadDim);
  w.kbar_t = c.take<float>((size_t)std::max(std::min(hkv, std::max(n_heads, 1)), 1) * nb * kHeadDim);
  w.rows = block_score_rows((int)nb, std::max(std::min(n_heads, 64), 1));
  w.scores = c.take<float>((size_t)std::max(std::min(n_heads, 64), 1) * w.rows * nb);
  w.blkmin = c.take<int32_t>(nb);
  w.blkmax = c.take<int32_t>(nb);
  w.words = (int)((n + 31) / 32);
  w.bits_min = c.take<uint32_t>((size_t)w.words);
  w.bits_max = c.take<uint32_t>((size_t)w.words);
  w.pre_min = c.take<int32_t>((size_t)w.words);
  w.pre_max = c.take<int32_t>((size_t)w.words);
  w.rank_q = c.take<int32_t>(nb);
  w.rank_k = c.take<int32_t>(nb);
  w.tau = c.take<int32_t>(nb);
  w.sigma = c.take<int32_t>(nb);
  w.lrow = c.take<int32_t>(nb);
  w.bytes = c.off;
  return w;
}

// ---------------- sparse attention workspace
size_t bitmap_words(int64_t n) { return (size_t)(nblocks(n) >> 5) + 1; }

}  // namespace

extern "C" {

const char* minf_status_string(minf_status s) {
  switch (s) {
    case MINF_OK: return "MINF_OK";
    case MINF_E_INVALID_ARG: return "MINF_E_INVALID_ARG";
    case MINF_E_UNSUPPORTED: return "MINF_E_UNSUPPORTED";
    case MINF_E_WORKSPACE: return "MINF_E_WORKSPACE";
    case MINF_E_HIP: return "MINF_E_HIP";
    default: return "MINF_E_UNKNOWN";
  }
}

const char* minf_last_error_detail(void) { return g_detail.c_str(); }

int minf_abi_version(void) { return 3; }

size_t minf_vs_index_workspace_size(int64_t n, int n_heads) {
  if (n < 1 || n_heads < 0) return 0;
  return carve_vs(nullptr, n, n_heads).bytes;
}

minf_status minf_vs_scores(const void* q, const void* k, int64_t n, int hq, int hkv, int d, const int32_t* heads,
                           int n_heads, int last_q, float scale, float* v_out, float* sl_out, void* workspace,
                           size_t ws_bytes, hipStream_t stream) {
  g_detail.clear();
  minf_status s = check_vs_args(q, k, n, hq, hkv, d, heads, n_heads, last_q, scale, workspace, ws_bytes);
  if (s != MINF_OK) return s;
  if (n_heads > 0 && (!v_out || !sl_out)) return fail(MINF_E_INVALID_ARG, "v_out and sl_out must be non-null");
  if (n_heads == 0) return MINF_OK;
  VsWs w = carve_vs(workspace, n, n_heads);
  if ((s = run_vs_scores(q, k, n, hq, hkv, heads, n_heads, last_q, scale, w, stream)) != MINF_OK) return s;
  const size_t bytes = (size_t)n_heads * (size_t)n * sizeof(float);
  hipError_t e = hipMemcpyAsync(v_out, w.vcol, bytes, hipMemcpyDeviceToDevice, stream);
  if (e == hipSuccess) e = hipMemcpyAsync(sl_out, w.slsum, bytes, hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, "copy of VS scores");
  return MINF_OK;
}

minf_status minf_build_vs_index(const void* q, const void* k, int64_t n, int hq, int hkv, int d,
                                const int32_t* heads, int n_heads, int last_q, int k_v, int k_s, float scale,
                                int32_t* v_idx, int32_t* s_idx, void* workspace, size_t ws_bytes,
                                hipStream_t stream) {
  g_detail.clear();
  minf_status s = check_vs_args(q, k, n, hq, hkv, d, heads, n_heads, last_q, scale, workspace, ws_bytes);
  if (s != MINF_OK) return s;
  if (k_v < 0 || k_s < 0) return fail(MINF_E_INVALID_ARG, "k_v and k_s must be >= 0");
  const int kv_eff = (int)std::min<int64_t>(k_v, n);
  const int ks_eff = (int)std::min<int64_t>(k_s, n);
  if (n_heads > 0 && ((kv_eff > 0 && !v_idx) || (ks_eff > 0 && !s_idx)))
    return fail(MINF_E_INVALID_ARG, "v_idx / s_idx must be non-null when their budget is > 0");
  if (n_heads == 0) return MINF_OK;
  VsWs w = carve_vs(workspace, n, n_heads);
  if ((s = run_vs_scores(q, k, n, hq, hkv, heads, n_heads, last_q, scale, w, stream)) != MINF_OK) return s;
  TopkLaunch t{};
  int ns = 0;
  if (kv_eff > 0) t.seg[ns++] = TopkSeg{w.vcol, v_idx, n, kv_eff, n_heads, kv_eff};
  if (ks_eff > 0) t.seg[ns++] = TopkSeg{w.slsum, s_idx, n, ks_eff, n_heads, ks_eff};
  if (ns == 0) return MINF_OK;
  t.n = (int)n;
  t.chunk = w.tk_chunk;
  t.nchunks = w.tk_nchunks;
  t.hist = w.tk_hist;
  t.state = w.tk_state;
  t.cnt = w.tk_cnt;
  hipError_t e = launch_topk(t, stream);
  if (e != hipSuccess) return hip_fail(e, "VS top-k kernels");
  return MINF_OK;
}

size_t minf_block_index_workspace_size(int64_t n, int hq, int hkv, int n_heads) {
  (void)hq;
  if (n < 1 || n_heads < 0 || hkv < 1) return 0;
  return carve_bs(nullptr, n, hkv, n_heads).bytes;
}

static minf_status build_block_index(const void* q, const void* k, int64_t n, int hq, int hkv, int d,
                                     const int32_t* heads, int n_heads, int k_b, const int32_t* pos,
                                     int32_t* blk_idx, int32_t* blk_cnt, void* workspace, size_t ws_bytes,
                                     hipStream_t stream) {
  minf_status s;
  if ((s = check_common(q, k, n, hq, hkv, d, kMaxTokens)) != MINF_OK) return s;
  if ((s = check_heads(heads, n_heads, hq)) != MINF_OK) return s;
  if (k_b < 1) return fail(MINF_E_INVALID_ARG, "k_b must be >= 1");
  if (n_heads == 0) return MINF_OK;
  if (!blk_idx || !blk_cnt) return fail(MINF_E_INVALID_ARG, "blk_idx and blk_cnt must be non-null");
  if ((s = check_ws(workspace, ws_bytes, minf_block_index_workspace_size(n, hq, hkv, n_heads))) != MINF_OK) return s;
  BsWs w = carve_bs(workspace, n, hkv, n_heads);
  const int grp = hq / hkv;
  // distinct KV heads in first-use order, and each query head's KV slot
  std::vector<int32_t> kv_heads, kv_slot(n_heads), q_slots(n_heads);
  for (int i = 0; i < n_heads; ++i) {
    const int kv = heads[i] / grp;
    auto it = std::find(kv_heads.begin(), kv_heads.end(), kv);
    kv_slot[i] = (int32_t)(it - kv_heads.begin());
    if (it == kv_heads.end()) kv_heads.push_back(kv);
    q_slots[i] = i;
  }
  std::vector<int32_t> kv_slots(kv_heads.size());
  for (size_t i = 0; i < kv_heads.size(); ++i) kv_slots[i] = (int32_t)i;
  const int nb = (int)nblocks(n);
  hipError_t e = hipSuccess;
  // permuted sequences: rows (pooled query blocks) in latest-position order and
  // columns (pooled key blocks) in earliest-position order, so that every row's
  // eligible key blocks are its first columns
  if (pos) {
    e = launch_block_minmax(pos, (int)n, w.blkmin, w.blkmax, stream);
    PermRankLaunch pr{w.blkmin, w.blkmax, w.bits_min, w.bits_max, w.pre_min, w.pre_max, w.rank_q,
                      w.rank_k, w.tau, w.sigma, w.lrow, (int32_t)n, nb, w.words};
    if (e == hipSuccess) e = launch_perm_ranks(pr, stream);
  }
  if (e == hipSuccess)
    e = launch_block_pool((const uint16_t*)q, (int)n, heads, q_slots.data(), n_heads, nullptr, w.qbar_t, stream, 0,
                          pos ? w.rank_q : nullptr);
  if (e == hipSuccess)
    e = launch_block_pool((const uint16_t*)k, (int)n, kv_heads.data(), kv_slots.data(), (int)kv_heads.size(),
                          nullptr, w.kbar_t, stream, 0, pos ? w.rank_k : nullptr);
  if (e == hipSuccess)
    e = launch_block_topk(w.qbar_t, w.kbar_t, kv_slot.data(), n_heads, nb, k_b, blk_idx, blk_cnt, w.scores, w.rows,
                          pos ? w.lrow : nullptr, pos ? w.sigma : nullptr, pos ? w.tau : nullptr, stream);
  if (e != hipSuccess) return hip_fail(e, "block index kernels");
  return MINF_OK;
}

minf_status minf_build_block_index(const void* q, const void* k, int64_t n, int hq, int hkv, int d,
                                   const int32_t* heads, int n_heads, int k_b, int32_t* blk_idx, int32_t* blk_cnt,
                                   void* workspace, size_t ws_bytes, hipStream_t stream) {
  g_detail.clear();
  return build_block_index(q, k, n, hq, hkv, d, heads, n_heads, k_b, nullptr, blk_idx, blk_cnt, workspace, ws_bytes,
                           stream);
}

minf_status minf_build_permuted_block_index(const void* q, const void* k, int64_t n, int hq, int hkv, int d,
                                            const int32_t* heads, int n_heads, int k_b, const int32_t* pos,
                                            int32_t* blk_idx, int32_t* blk_cnt, void* workspace, size_t ws_bytes,
                                            hipStream_t stream) {
  g_detail.clear();
  if (!pos) return fail(MINF_E_INVALID_ARG, "pos must be a device array of the rows' original positions");
  return build_block_index(q, k, n, hq, hkv, d, heads, n_heads, k_b, pos, blk_idx, blk_cnt, workspace, ws_bytes,
                           stream);
}

minf_status minf_permute_rows(const void* x, void* out, int heads, int64_t n, int row_bytes, const int32_t* src,
                              int scatter, hipStream_t stream) {
  g_detail.clear();
  if (!x || !out || !src) return fail(MINF_E_INVALID_ARG, "x, out and src must be non-null device pointers");
  if (x == out) return fail(MINF_E_INVALID_ARG, "out must not alias x");
  if (heads < 1 || n < 1) return fail(MINF_E_INVALID_ARG, "heads and n must be >= 1");
  if (row_bytes < 4 || row_bytes % 4 != 0) return fail(MINF_E_INVALID_ARG, "row_bytes must be a positive multiple of 4");
  if (n > kMaxTokens) return fail(MINF_E_UNSUPPORTED, "n = %lld exceeds the supported %lld", (long long)n,
                                  (long long)kMaxTokens);
  if (scatter != 0 && scatter != 1) return fail(MINF_E_INVALID_ARG, "scatter must be 0 or 1");
  if (n * (int64_t)(row_bytes / 4) >= ((int64_t)1 << 31))
    return fail(MINF_E_UNSUPPORTED, "n * row_bytes / 4 = %lld words per head exceeds 2^31 - 1",
                (long long)(n * (int64_t)(row_bytes / 4)));
  hipError_t e = launch_permute_rows(x, out, heads, n, row_bytes, src, scatter, stream);
  if (e != hipSuccess) return hip_fail(e, "row permutation kernel");
  return MINF_OK;
}

minf_status minf_block_pool(const void* x, int64_t n, int h_total, int d, const int32_t* heads, int n_heads,
                            float* out, hipStream_t stream) {
  g_detail.clear();
  minf_status s;
  if ((s = check_common(x, x, n, h_total, 1, d, kMaxTokens)) != MINF_OK) return s;
  if ((s = check_heads(heads, n_heads, h_total)) != MINF_OK) return s;
  if (n_heads == 0) return MINF_OK;
  if (!out) return fail(MINF_E_INVALID_ARG, "out must be non-null");
  std::vector<int32_t> slots(n_heads);
  for (int i = 0; i < n_heads; ++i) slots[i] = i;
  hipError_t e = launch_block_pool((const uint16_t*)x, (int)n, heads, slots.data(), n_heads, out, nullptr, stream);
  if (e != hipSuccess) return hip_fail(e, "pooling kernel");
  return MINF_OK;
}

// Per-head window area of VS window heads: the offset bitmap over [0, n), the
// tile cover, its tile count.
static size_t vsw_head_bytes(int64_t n) {
  return align_up((size_t)((n + 31) / 32) * sizeof(uint32_t)) +
         align_up((size_t)vsw_tile_capacity((int)n) * sizeof(int2)) + kAlign;
}

size_t minf_sparse_attn_workspace_size(int64_t n, int hq) {
  if (n < 1 || hq < 1) return 0;
  // per head: the VS offset bitmaps, then the min / max original position of
  // every key block for Block-Sparse heads on a permuted sequence; per-XCD
  // counters and a flag; then the window areas of VS window heads
  return align_up((size_t)hq * 2 * bitmap_words(n) * sizeof(uint32_t)) +
         align_up((size_t)hq * 2 * nblocks(n) * sizeof(int32_t)) + kAlign + (size_t)hq * vsw_head_bytes(n);
}

// Launches of Vertical-Slash heads only, at long lengths, queue two launches
// of the same work: a rounds one (exactly as many workgroups as the device
// holds at once) in which the 64 workgroups of an XCD run their items in
// rounds that start together, and an ordinary one. A flag
// computed on the device from the offset bitmaps, without a host round trip,
// lets exactly one of them work: rounds when the items are long (thousands of
// key tiles), because workgroups that stay at the same key position keep
// sharing K/V tiles through L2 (at 1M tokens on literal data this cuts the
// attention's HBM reads from ~34 TB to ~3 TB); the ordinary launch when they
// are short, because its hardware dispatch balances the load better.
// MINF_ATTN_ROUNDS=0 in the environment (read on every call), or a stream in
// graph capture, keeps the ordinary launch only; both give bitwise-identical
// results.
constexpr int64_t kRoundsMinTokens = 1 << 17;
constexpr int kRoundsMinTiles = 1024;

static bool rounds_enabled(hipStream_t stream) {
  const char* e = getenv("MINF_ATTN_ROUNDS");
  if (e != nullptr && e[0] == '0') return false;
  // a stream being captured into a graph gets the ordinary launch only (the
  // rounds launch's waits assume it has the device to itself, which a replay
  // beside other graph work need not give)
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs == hipStreamCaptureStatusNone;
}

// Dense causal attention from 2^17 tokens takes the rounds launch too: every
// work item walks all its keys, so the 64 workgroups of an XCD share K/V tiles
// through L2 as long as they stay together (32/8 heads: 128K 132.5 -> 128.5
// ms, 1M 10.07 -> 8.04 s). Its barrier counters and its always-set flag live
// in a static per-GPU array (dense calls take no workspace); calls that
// overlap on one GPU share it, which can only slow their rounds (each wait is
// bounded) and never changes a result.
constexpr int64_t kDenseRoundsMinTokens = 1 << 17;
static __device__ __align__(256) int32_t dense_rounds_state[kRoundXcds + 1];
std::mutex g_dense_rounds_mu;
int32_t* g_dense_rounds_ptr[64] = {};

static int32_t* dense_rounds_state_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_dense_rounds_mu);
  if (!g_dense_rounds_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(dense_rounds_state)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_dense_rounds_ptr[dev] = (int32_t*)ptr;
  }
  return g_dense_rounds_ptr[dev];
}

static minf_status check_attn_common(const void* q, const void* k, const void* v, void* o, int64_t n, int hq,
                                     int hkv, int d, float scale, int64_t max_n) {
  minf_status s;
  if ((s = check_common(q, k, n, hq, hkv, d, max_n)) != MINF_OK) return s;
  if (!v || !o) return fail(MINF_E_INVALID_ARG, "v and o must be non-null device pointers");
  return check_scale(scale);
}

// Heads per attention launch and per work chunk. A launch takes up to 32
// heads; the chunk size hg divides both the launch's head count and 64.
// Dense launches group the heads of one GQA group in a chunk (they read the
// same K/V tiles in the same order). Sparse launches use one head per chunk:
// per-head index sets differ, while the 64 consecutive query-block pairs of
// one head select the same block offsets, so walking keys in ascending order
// they reach each key block at about the same step and share it through L2.
static void head_split(int hq, int grp, int h0, bool group_heads, int& nh, int& hg) {
  const int left = hq - h0;
  if (grp <= kMaxLaunchHeads) {
    const int per = (kMaxLaunchHeads / grp) * grp;
    nh = std::min(per, left);
  } else {
    nh = std::min(kMaxLaunchHeads, left);
  }
  hg = 1;
  if (!group_heads) return;
  for (int c = 64; c >= 1; c >>= 1)
    if (c <= grp && nh % c == 0 && grp % c == 0) {
      hg = c;
      break;
    }
}

static minf_status launch_all_heads(AttnLaunch& a, int hq, hipStream_t stream) {
  for (int h0 = 0; h0 < hq;) {
    int nh, hg;
    head_split(hq, a.grp, h0, true, nh, hg);
    for (int i = 0; i < nh; ++i) a.heads[i].head = h0 + i;
    a.nh = nh;
    a.hgroup = hg;
    hipError_t e = launch_attn(a, stream);
    if (e != hipSuccess) return hip_fail(e, "attention kernel");
    h0 += nh;
  }
  return MINF_OK;
}

minf_status minf_sparse_attn(const void* q, const void* k, const void* v, void* o, float* lse, int64_t n, int hq,
                             int hkv, int d, float scale, const minf_head_plan* plans, void* workspace,
                             size_t ws_bytes, hipStream_t stream) {
  g_detail.clear();
  minf_status s;
  if ((s = check_attn_common(q, k, v, o, n, hq, hkv, d, scale, kMaxTokens)) != MINF_OK) return s;
  if (!plans) return fail(MINF_E_INVALID_ARG, "plans must be a host array of hq entries");
  bool any_vs = false, any_pos = false, any_vsw = false;
  for (int h = 0; h < hq; ++h) {
    const minf_head_plan& p = plans[h];
    if (p.pos && p.kind != MINF_KIND_BLOCK)
      return fail(MINF_E_INVALID_ARG, "head %d: pos is only defined for Block-Sparse plans", h);
    any_pos |= p.pos != nullptr;
    switch (p.kind) {
      case MINF_KIND_DENSE: break;
      case MINF_KIND_ASHAPE:
        if (p.sink < 0 || p.local < 0) return fail(MINF_E_INVALID_ARG, "head %d: sink and local must be >= 0", h);
        break;
      case MINF_KIND_VS:
      case MINF_KIND_VS_WINDOW:
        if (p.k_v < 0 || p.k_s < 0) return fail(MINF_E_INVALID_ARG, "head %d: k_v and k_s must be >= 0", h);
        if ((p.k_v > 0 && !p.v_idx) || (p.k_s > 0 && !p.s_idx))
          return fail(MINF_E_INVALID_ARG, "head %d: v_idx / s_idx null with a positive count", h);
        (p.kind == MINF_KIND_VS ? any_vs : any_vsw) = true;
        break;
      case MINF_KIND_BLOCK:
        if (p.k_b < 1) return fail(MINF_E_INVALID_ARG, "head %d: k_b must be >= 1", h);
        if (!p.blk_idx || !p.blk_cnt) return fail(MINF_E_INVALID_ARG, "head %d: blk_idx / blk_cnt are null", h);
        break;
      default: return fail(MINF_E_INVALID_ARG, "head %d: unknown plan kind %d", h, p.kind);
    }
  }
  if ((any_vs || any_pos || any_vsw) &&
      (s = check_ws(workspace, ws_bytes, minf_sparse_attn_workspace_size(n, hq))) != MINF_OK)
    return s;

  AttnLaunch a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.n = (int)n;
  a.nb = (int)nblocks(n);
  a.hq = hq;
  a.hkv = hkv;
  a.grp = hq / hkv;
  a.causal = 1;
  a.scale_log2 = scale * 1.4426950408889634f;

  const size_t words = 2 * bitmap_words(n);  // full-block bitmap, then the partial-last-block one
  std::vector<const int32_t*> vs_s;
  std::vector<int32_t> vs_k;
  std::vector<uint32_t*> vs_bits;
  for (int h = 0; h < hq; ++h) {
    if (plans[h].kind != MINF_KIND_VS) continue;
    vs_s.push_back(plans[h].s_idx);
    vs_k.push_back(plans[h].k_s);
    vs_bits.push_back((uint32_t*)workspace + (size_t)h * words);
  }
  if (!vs_s.empty()) {
    hipError_t e = launch_vs_offset_bits(vs_s.data(), vs_k.data(), vs_bits.data(), (int)vs_s.size(), (int)n, stream);
    if (e != hipSuccess) return hip_fail(e, "VS offset bitmap kernel");
  }
  const size_t nbk = (size_t)nblocks(n);
  int32_t* pos_ws = (int32_t*)((char*)workspace + align_up((size_t)hq * words * sizeof(uint32_t)));
  int32_t* sync_ws = (int32_t*)((char*)pos_ws + align_up((size_t)hq * 2 * nbk * sizeof(int32_t)));
  char* vsw_ws = (char*)sync_ws + kAlign;
  const int vsw_cap = vsw_tile_capacity((int)n);
  auto vsw_area = [&](int h, uint32_t*& dbits, int2*& tiles, int32_t*& count) {
    char* base = vsw_ws + (size_t)h * vsw_head_bytes(n);
    dbits = (uint32_t*)base;
    tiles = (int2*)(base + align_up((size_t)((n + 31) / 32) * sizeof(uint32_t)));
    count = (int32_t*)((char*)tiles + align_up((size_t)vsw_cap * sizeof(int2)));
  };
  if (any_vsw) {
    // offset bitmaps and window tile covers of the VS window heads
    VswLaunch w{};
    int cnt = 0, max_ks = 0;
    for (int h = 0; h <= hq; ++h) {
      if (cnt == kMaxLaunchHeads || (h == hq && cnt > 0)) {
        w.n = (int)n;
        w.cap = vsw_cap;
        hipError_t e = launch_vsw_prepare(w, cnt, max_ks, stream);
        if (e != hipSuccess) return hip_fail(e, "VS window preparation kernels");
        w = VswLaunch{};
        cnt = max_ks = 0;
      }
      if (h == hq || plans[h].kind != MINF_KIND_VS_WINDOW) continue;
      w.s_idx[cnt] = plans[h].s_idx;
      w.k_s[cnt] = plans[h].k_s;
      max_ks = std::max(max_ks, plans[h].k_s);
      vsw_area(h, w.dbits[cnt], w.tiles[cnt], w.count[cnt]);
      ++cnt;
    }
  }
  for (int h = 0; h < hq && any_pos; ++h) {
    if (!plans[h].pos) continue;
    // heads that share a position array share its block extremes
    int first = h;
    for (int g = 0; g < h; ++g)
      if (plans[g].pos == plans[h].pos) {
        first = g;
        break;
      }
    if (first != h) continue;
    hipError_t e = launch_block_minmax(plans[h].pos, (int)n, pos_ws + (size_t)h * 2 * nbk,
                                       pos_ws + (size_t)h * 2 * nbk + nbk, stream);
    if (e != hipSuccess) return hip_fail(e, "block position kernel");
  }
  // Launch order: the Vertical-Slash heads (and VS windows) first, then the
  // other heads, each in launches of up to kMaxLaunchHeads heads. A launch of
  // VS heads only can take the rounds launch; the short Block-Sparse and
  // A-shape items then do not hold back the rounds of the long VS items.
  std::vector<int> order;
  for (int pass = 0; pass < 2; ++pass)
    for (int h = 0; h < hq; ++h) {
      const bool vs_class = plans[h].kind == MINF_KIND_VS || plans[h].kind == MINF_KIND_VS_WINDOW;
      if (vs_class == (pass == 0)) order.push_back(h);
    }
  for (size_t i0 = 0; i0 < order.size();) {
    const bool vs_class = plans[order[i0]].kind == MINF_KIND_VS || plans[order[i0]].kind == MINF_KIND_VS_WINDOW;
    int nh = 0;
    while (i0 + nh < order.size() && nh < kMaxLaunchHeads) {
      const int h = order[i0 + nh];
      const bool c = plans[h].kind == MINF_KIND_VS || plans[h].kind == MINF_KIND_VS_WINDOW;
      if (c != vs_class) break;
      ++nh;
    }
    for (int i = 0; i < nh; ++i) {
      const int hid = order[i0 + i];
      const minf_head_plan& p = plans[hid];
      AttnHead& d2 = a.heads[i];
      d2 = AttnHead{};
      d2.head = hid;
      d2.kind = p.kind;
      d2.sink = p.sink;
      d2.local = p.local;
      d2.k_v = (p.kind == MINF_KIND_VS || p.kind == MINF_KIND_VS_WINDOW) ? p.k_v : 0;
      if (p.kind == MINF_KIND_VS_WINDOW) {
        uint32_t* db;
        int2* wt;
        int32_t* wc;
        vsw_area(hid, db, wt, wc);
        d2.dbits = db;
        d2.wtiles = wt;
        d2.wcount = wc;
      }
      d2.k_b = p.k_b;
      d2.v_idx = p.v_idx;
      d2.obits = p.kind == MINF_KIND_VS ? (const uint32_t*)workspace + (size_t)hid * words : nullptr;
      d2.blk_idx = p.blk_idx;
      d2.blk_cnt = p.blk_cnt;
      if (p.pos) {
        int first = hid;
        for (int g = 0; g < hid; ++g)
          if (plans[g].pos == p.pos) {
            first = g;
            break;
          }
        d2.pos = p.pos;
        d2.blkmax = pos_ws + (size_t)first * 2 * nbk + nbk;
      }
    }
    std::vector<uint32_t*> launch_bits;
    std::vector<const int32_t*> launch_wcount;
    for (int i = 0; i < nh; ++i) {
      const int hid = order[i0 + i];
      if (plans[hid].kind == MINF_KIND_VS) launch_bits.push_back((uint32_t*)workspace + (size_t)hid * words);
      if (plans[hid].kind == MINF_KIND_VS_WINDOW) launch_wcount.push_back(a.heads[i].wcount);
    }
    a.nh = nh;
    a.hgroup = 1;  // sparse items: one head per work chunk
    a.xcd_sync = nullptr;
    a.rounds_flag = nullptr;
    if (vs_class && n >= kRoundsMinTokens && rounds_enabled(stream)) {
      int32_t* flag = sync_ws + 8;
      hipError_t e = launch_rounds_flag(launch_bits.data(), (int)launch_bits.size(), launch_wcount.data(),
                                        (int)launch_wcount.size(), (int)n, kRoundsMinTiles, flag, stream);
      if (e != hipSuccess) return hip_fail(e, "rounds flag kernel");
      a.xcd_sync = sync_ws;
      a.rounds_flag = flag;
    }
    hipError_t e = launch_attn(a, stream);
    if (e != hipSuccess) return hip_fail(e, "sparse attention kernel");
    i0 += nh;
  }
  return MINF_OK;
}

minf_status minf_plan_work(const minf_head_plan* plans, int64_t n, int hq, double* work, void* workspace,
                           size_t ws_bytes, hipStream_t stream) {
  g_detail.clear();
  if (n < 1) return fail(MINF_E_INVALID_ARG, "n must be >= 1 (got %lld)", (long long)n);
  if (n > kMaxTokens)
    return fail(MINF_E_UNSUPPORTED, "n = %lld exceeds the supported %lld", (long long)n, (long long)kMaxTokens);
  if (hq < 1) return fail(MINF_E_INVALID_ARG, "hq must be >= 1");
  if (!plans) return fail(MINF_E_INVALID_ARG, "plans must be a host array of hq entries");
  if (!work) return fail(MINF_E_INVALID_ARG, "work must be a device array of hq doubles");
  bool any_vs = false;
  for (int h = 0; h < hq; ++h) {
    const minf_head_plan& p = plans[h];
    switch (p.kind) {
      case MINF_KIND_DENSE: break;
      case MINF_KIND_ASHAPE:
        if (p.sink < 0 || p.local < 0) return fail(MINF_E_INVALID_ARG, "head %d: sink and local must be >= 0", h);
        break;
      case MINF_KIND_VS:
        if (p.k_v < 0 || p.k_s < 0) return fail(MINF_E_INVALID_ARG, "head %d: k_v and k_s must be >= 0", h);
        if ((p.k_v > 0 && !p.v_idx) || (p.k_s > 0 && !p.s_idx))
          return fail(MINF_E_INVALID_ARG, "head %d: v_idx / s_idx null with a positive count", h);
        any_vs = true;
        break;
      case MINF_KIND_BLOCK:
        if (!p.blk_cnt) return fail(MINF_E_INVALID_ARG, "head %d: blk_cnt is null", h);
        break;
      case MINF_KIND_VS_WINDOW:
        return fail(MINF_E_UNSUPPORTED, "head %d: the work count covers dense, A-shape, VS and Block-Sparse plans", h);
      default: return fail(MINF_E_INVALID_ARG, "head %d: unknown plan kind %d", h, p.kind);
    }
  }
  minf_status s;
  if (any_vs && (s = check_ws(workspace, ws_bytes, minf_sparse_attn_workspace_size(n, hq))) != MINF_OK) return s;
  // the attention call's block-offset bitmaps, at the same place in the workspace
  const size_t words = 2 * bitmap_words(n);
  std::vector<const int32_t*> vs_s;
  std::vector<int32_t> vs_k;
  std::vector<uint32_t*> vs_bits;
  for (int h = 0; h < hq; ++h) {
    if (plans[h].kind != MINF_KIND_VS) continue;
    vs_s.push_back(plans[h].s_idx);
    vs_k.push_back(plans[h].k_s);
    vs_bits.push_back((uint32_t*)workspace + (size_t)h * words);
  }
  if (!vs_s.empty()) {
    hipError_t e = launch_vs_offset_bits(vs_s.data(), vs_k.data(), vs_bits.data(), (int)vs_s.size(), (int)n, stream);
    if (e != hipSuccess) return hip_fail(e, "VS offset bitmap kernel");
  }
  for (int h0 = 0; h0 < hq; h0 += kMaxLaunchHeads) {
    WorkLaunch a{};
    const int cnt = std::min(kMaxLaunchHeads, hq - h0);
    for (int i = 0; i < cnt; ++i) {
      const minf_head_plan& p = plans[h0 + i];
      WorkHead& w = a.heads[i];
      w.kind = p.kind;
      w.sink = p.sink;
      w.local = p.local;
      w.k_v = p.kind == MINF_KIND_VS ? p.k_v : 0;
      w.v_idx = p.v_idx;
      w.obits = p.kind == MINF_KIND_VS ? (const uint32_t*)workspace + (size_t)(h0 + i) * words : nullptr;
      w.blk_cnt = p.blk_cnt;
    }
    a.n = (int)n;
    a.nb = (int)nblocks(n);
    a.out = work + h0;
    hipError_t e = launch_plan_work(a, cnt, stream);
    if (e != hipSuccess) return hip_fail(e, "plan work kernel");
  }
  return MINF_OK;
}

minf_status minf_attention_recall(const float* lse_mask, const float* lse_dense, int64_t n, int hq,
                                  const int32_t* rows, int n_rows, double* recall, hipStream_t stream) {
  g_detail.clear();
  if (!lse_mask || !lse_dense || !recall) return fail(MINF_E_INVALID_ARG, "lse_mask, lse_dense and recall must be non-null");
  if (n < 1 || n > ((int64_t)1 << 30)) return fail(MINF_E_INVALID_ARG, "n must be in [1, 2^30] (got %lld)", (long long)n);
  if (hq < 1) return fail(MINF_E_INVALID_ARG, "hq must be >= 1");
  if (rows && n_rows < 1) return fail(MINF_E_INVALID_ARG, "n_rows must be >= 1 when rows is given");
  const int nr = rows ? n_rows : (int)n;
  hipError_t e = launch_recall(lse_mask, lse_dense, (int)n, hq, rows, nr, recall, stream);
  if (e != hipSuccess) return hip_fail(e, "recall kernel");
  return MINF_OK;
}

minf_status minf_dense_attn(const void* q, const void* k, const void* v, void* o, float* lse, int64_t n, int hq,
                            int hkv, int d, float scale, int causal, hipStream_t stream) {
  g_detail.clear();
  minf_status s;
  if ((s = check_attn_common(q, k, v, o, n, hq, hkv, d, scale, (int64_t)1 << 24)) != MINF_OK) return s;
  AttnLaunch a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.n = (int)n;
  a.nb = (int)nblocks(n);
  a.hq = hq;
  a.hkv = hkv;
  a.grp = hq / hkv;
  a.causal = causal ? 1 : 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  for (int i = 0; i < kMaxLaunchHeads; ++i) a.heads[i] = AttnHead{};
  if (causal && n >= kDenseRoundsMinTokens && rounds_enabled(stream)) {
    int32_t* st = dense_rounds_state_ptr();
    if (st) {
      a.xcd_sync = st;
      a.rounds_flag = st + kRoundXcds;
      a.rounds_flag_set = st + kRoundXcds;
    }
  }
  return launch_all_heads(a, hq, stream);
}

}  // extern "C"

// ---------------- decoding
namespace {

constexpr int kMaxDecodeGroup = 8;

struct DecWs {
  float* scores;
  int32_t* blk;
  float* part;
  uint32_t* seg_key;
  int32_t* seg_id;
  int32_t* seg_cnt;
  int nseg;
  size_t bytes;
};

// Dense decoding serves up to four heads per workgroup, so it has up to four
// times fewer workgroup rows than sparse decoding.
int decode_split_len(int kb, int hq, bool select) {
  return decode_blocks_per_split(kb, select ? hq : std::max(1, hq / 4));
}

DecWs carve_decode(void* base, int64_t n, int hq, int kb, bool select) {
  Carver c{(char*)base};
  DecWs w{};
  const size_t nb = (size_t)nblocks(n);
  const int bps = decode_split_len(kb, hq, select);
  const int nsplit = (kb + bps - 1) / bps;
  if (select) {
    w.scores = c.take<float>((size_t)hq * nb);
    w.blk = c.take<int32_t>((size_t)hq * kb);
    w.nseg = decode_topk_segments((int)nb, kb);
    if (w.nseg > 1) {
      w.seg_key = c.take<uint32_t>((size_t)hq * w.nseg * kb);
      w.seg_id = c.take<int32_t>((size_t)hq * w.nseg * kb);
      w.seg_cnt = c.take<int32_t>((size_t)hq * w.nseg);
    }
  }
  w.part = c.take<float>((size_t)hq * nsplit * (kHeadDim + 2));
  w.bytes = c.off;
  return w;
}

minf_status check_decode(const void* q, const void* k, const void* v, void* o, int64_t n, int hq, int hkv, int d,
                         float scale) {
  minf_status s;
  if ((s = check_common(q, k, n, hq, hkv, d, (int64_t)kDecMaxBlocks * kBlock)) != MINF_OK) return s;
  if (!v || !o) return fail(MINF_E_INVALID_ARG, "v and o must be non-null device pointers");
  if (hq / hkv > kMaxDecodeGroup)
    return fail(MINF_E_UNSUPPORTED, "decoding supports at most %d query heads per KV head", kMaxDecodeGroup);
  return check_scale(scale);
}

minf_status run_decode(const void* q, const void* k, const void* v, const float* kbar_t, int64_t n, int hq, int hkv,
                       float scale, int kb_eff, bool select, int32_t* blk_idx, void* o, float* lse, const DecWs& w,
                       hipStream_t stream) {
  DecodeLaunch a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.kbar_t = kbar_t;
  a.scores = w.scores;
  a.blk = select ? (blk_idx ? blk_idx : w.blk) : nullptr;
  a.part = w.part;
  a.seg_key = w.seg_key;
  a.seg_id = w.seg_id;
  a.seg_cnt = w.seg_cnt;
  a.nseg = w.nseg;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.n = (int)n;
  a.nb = (int)nblocks(n);
  a.hq = hq;
  a.hkv = hkv;
  a.grp = hq / hkv;
  a.kb = kb_eff;
  a.bps = decode_split_len(kb_eff, hq, select);
  a.nsplit = (kb_eff + a.bps - 1) / a.bps;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = launch_decode(a, select, stream);
  if (e != hipSuccess) return hip_fail(e, "decode kernels");
  return MINF_OK;
}

}  // namespace

extern "C" {

minf_status minf_decode_pool_keys(const void* k, int64_t n, int hkv, int d, int first_block, float* kbar_t,
                                  hipStream_t stream) {
  g_detail.clear();
  minf_status s;
  if ((s = check_common(k, k, n, hkv, hkv, d, (int64_t)kDecMaxBlocks * kBlock)) != MINF_OK) return s;
  if (!kbar_t) return fail(MINF_E_INVALID_ARG, "kbar_t must be non-null");
  if (first_block < 0) return fail(MINF_E_INVALID_ARG, "first_block must be >= 0");
  if (first_block >= nblocks(n)) return MINF_OK;
  std::vector<int32_t> heads(hkv);
  for (int i = 0; i < hkv; ++i) heads[i] = i;
  hipError_t e = launch_block_pool((const uint16_t*)k, (int)n, heads.data(), heads.data(), hkv, nullptr, kbar_t,
                                   stream, first_block);
  if (e != hipSuccess) return hip_fail(e, "key pooling kernel");
  return MINF_OK;
}

size_t minf_decode_workspace_size(int64_t n, int hq, int k_b) {
  if (n < 1 || hq < 1 || k_b < 1) return 0;
  const int64_t nb = nblocks(n);
  const bool select = k_b < nb;
  const int kb_eff = (int)std::min<int64_t>(k_b, nb);
  return carve_decode(nullptr, n, hq, kb_eff, select).bytes;
}

minf_status minf_sparse_decode(const void* q, const void* k, const void* v, const float* kbar_t, int64_t n, int hq,
                               int hkv, int d, float scale, int k_b, int32_t* blk_idx, void* o, float* lse,
                               void* workspace, size_t ws_bytes, hipStream_t stream) {
  g_detail.clear();
  minf_status s;
  if ((s = check_decode(q, k, v, o, n, hq, hkv, d, scale)) != MINF_OK) return s;
  if (k_b < 1) return fail(MINF_E_INVALID_ARG, "k_b must be >= 1");
  const int64_t nb = nblocks(n);
  const bool select = k_b < nb;
  const int kb_eff = (int)std::min<int64_t>(k_b, nb);
  if (select && !kbar_t) return fail(MINF_E_INVALID_ARG, "kbar_t must be non-null when k_b < n_b");
  DecWs w = carve_decode(workspace, n, hq, kb_eff, select);
  if ((s = check_ws(workspace, ws_bytes, w.bytes)) != MINF_OK) return s;
  w = carve_decode(workspace, n, hq, kb_eff, select);
  if ((s = run_decode(q, k, v, kbar_t, n, hq, hkv, scale, kb_eff, select, blk_idx, o, lse, w, stream)) != MINF_OK)
    return s;
  if (!select && blk_idx) {
    // full budget: every block, in order
    hipError_t e = launch_iota_rows(blk_idx, hq, kb_eff, stream);
    if (e != hipSuccess) return hip_fail(e, "full block list");
  }
  return MINF_OK;
}

minf_status minf_dense_decode(const void* q, const void* k, const void* v, int64_t n, int hq, int hkv, int d,
                              float scale, void* o, float* lse, void* workspace, size_t ws_bytes,
                              hipStream_t stream) {
  g_detail.clear();
  minf_status s;
  if ((s = check_decode(q, k, v, o, n, hq, hkv, d, scale)) != MINF_OK) return s;
  const int kb_eff = (int)nblocks(n);
  DecWs w = carve_decode(workspace, n, hq, kb_eff, false);
  if ((s = check_ws(workspace, ws_bytes, w.bytes)) != MINF_OK) return s;
  w = carve_decode(workspace, n, hq, kb_eff, false);
  return run_decode(q, k, v, nullptr, n, hq, hkv, scale, kb_eff, false, nullptr, o, lse, w, stream);
}

}  // extern "C"


// ---------------- decoding without allocation
// Callers that cannot allocate device memory (code under graph capture, tight
// serving loops) use minf_sparse_decode_noalloc: its scratch is this
// file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
namespace {

constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

minf_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MINF_E_UNSUPPORTED, "device %d is beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch symbol address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MINF_OK;
}

}  // namespace

extern "C" {

size_t minf_decode_noalloc_max_bytes(void) { return kDecodeScratchBytes; }

minf_status minf_sparse_decode_noalloc(const void* q, const void* k, const void* v, const float* kbar_t, int64_t n,
                                       int hq, int hkv, int d, float scale, int k_b, int32_t* blk_idx, void* o,
                                       float* lse, hipStream_t stream) {
  g_detail.clear();
  minf_status s;
  if ((s = check_decode(q, k, v, o, n, hq, hkv, d, scale)) != MINF_OK) return s;
  if (k_b < 1) return fail(MINF_E_INVALID_ARG, "k_b must be >= 1");
  const int64_t nb = nblocks(n);
  const bool select = k_b < nb;
  const int kb_eff = (int)std::min<int64_t>(k_b, nb);
  if (select && !kbar_t) return fail(MINF_E_INVALID_ARG, "kbar_t must be non-null when k_b < n_b");
  const size_t need = carve_decode(nullptr, n, hq, kb_eff, select).bytes;
  if (need > kDecodeScratchBytes)
    return fail(MINF_E_UNSUPPORTED, "this decode step needs %zu bytes of scratch; the static scratch holds %zu", need,
                kDecodeScratchBytes);
  void* base = nullptr;
  if ((s = scratch_for_current_device(&base)) != MINF_OK) return s;
  // every scratch word a kernel reads was written earlier in the same call: nothing to clear
  const DecWs w = carve_decode(base, n, hq, kb_eff, select);
  if ((s = run_decode(q, k, v, kbar_t, n, hq, hkv, scale, kb_eff, select, blk_idx, o, lse, w, stream)) != MINF_OK)
    return s;
  if (!select && blk_idx) {
    hipError_t e = launch_iota_rows(blk_idx, hq, kb_eff, stream);
    if (e != hipSuccess) return hip_fail(e, "full block list");
  }
  return MINF_OK;
}

}  // extern "C"
