/*
 * minf.h - C ABI of the MI355X (gfx950) dynamic sparse attention library.
 *
 * The library implements the online half of MInference-style sparse prefill
 * for causal attention: per-head index construction (Vertical-Slash,
 * Block-Sparse; A-shape needs none) and a sparse FlashAttention that computes
 * only the selected 64x64 key blocks and gathered key columns, plus a dense
 * causal FlashAttention used as the baseline.
 *
 * Sources (web pages): "MInference 1.0 article: million-token inference on a
 * single A100", sections "Method" and "Latency and sparse patterns in
 * kernels" (Fig. 3, Fig. 4); "KV-cache-centric efficient long-context
 * methods" talk transcript, section "KV-cache-centric methods" (MInference
 * and the three-step dynamic-sparse framework); the MInference abstract on
 * the authors' page (pattern fixed offline, sparse index built online from
 * the pattern, sparse kernels use the pattern and index).
 *
 * Conventions for every call:
 *  - Tensors are device pointers. bf16 tensors are passed as raw 16-bit
 *    storage. Q and O are [hq][n][d], K and V are [hkv][n][d], row-major and
 *    contiguous. d must be 128 (otherwise MINF_E_UNSUPPORTED).
 *  - GQA: query head h reads KV head h / (hq / hkv); hq % hkv == 0.
 *  - The caller owns every buffer (inputs, outputs, workspace). The library
 *    allocates nothing and keeps no pointer after a call returns.
 *  - Work is enqueued on `stream` and the call returns after enqueue; results
 *    are valid once the stream has reached that point. There is no hidden
 *    device synchronisation.
 *  - Arguments are validated before any launch; a failed validation returns
 *    a status and launches nothing. A HIP launch error returns MINF_E_HIP;
 *    minf_last_error_detail() then holds the HIP error text (thread-local).
 *  - Budgets larger than what exists are clamped ("full budget").
 *  - Identical inputs give bitwise-identical outputs and indices (no float
 *    atomics; every reduction has a fixed order).
 *  - Softmax scale: the pages never state it; callers normally pass
 *    1/sqrt(d). A scale <= 0 or non-finite is rejected.
 */
#ifndef MINF_H
#define MINF_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int minf_status;
#define MINF_OK 0
#define MINF_E_INVALID_ARG 1 /* null pointer, bad size, bad head list, ... */
#define MINF_E_UNSUPPORTED 2 /* valid request the library does not implement (d != 128, last_q > 64) */
#define MINF_E_WORKSPACE 3   /* workspace pointer null or smaller than required */
#define MINF_E_HIP 4         /* a HIP runtime call or launch failed */

/* Human-readable name of a status code. Never returns NULL. */
const char* minf_status_string(minf_status s);

/* Detail text of the last failure on the calling thread ("" if none). */
const char* minf_last_error_detail(void);

/* Library ABI version (incremented when a signature, a struct or the set of plan kinds changes). */
int minf_abi_version(void);

/* ------------------------------------------------------------------------
 * Vertical-Slash index ("Method": the attention between the last queries and
 * all keys estimates the best vertical and slash indices).
 *
 * For each listed query head h (KV head g = h / (hq/hkv)), with
 * r = min(last_q, n) and rows I = [n - r, n):
 *   P[i][j] = softmax over j <= i of scale * q_i . k_j        (i in I)
 *   v[j]    = sum_i P[i][j]                 (column sums)
 *   sl[dl]  = sum_i P[i][i - dl]            (diagonal sums, dl = i - j >= 0)
 *   v_idx   = top-min(k_v, n) of v,  s_idx = top-min(k_s, n) of sl,
 *   ties to the lower index, each list sorted ascending.
 *
 * heads    host array of n_heads distinct query head ids in [0, hq).
 * last_q   1..64 (MINF_E_UNSUPPORTED above 64).
 * v_idx    device int32 [n_heads][min(k_v, n)]  ascending column ids.
 * s_idx    device int32 [n_heads][min(k_s, n)]  ascending diagonal offsets.
 * workspace / ws_bytes  device scratch of at least
 *          minf_vs_index_workspace_size(n, n_heads) bytes, 256-byte aligned.
 * k_v, k_s >= 0 (0 gives an empty list).
 * ---------------------------------------------------------------------- */
size_t minf_vs_index_workspace_size(int64_t n, int n_heads);
minf_status minf_build_vs_index(const void* q, const void* k, int64_t n, int hq, int hkv, int d,
                                const int32_t* heads, int n_heads, int last_q, int k_v, int k_s,
                                float scale, int32_t* v_idx, int32_t* s_idx, void* workspace,
                                size_t ws_bytes, hipStream_t stream);

/* Debug export of the VS estimate before top-k: v_out and sl_out are device
 * float [n_heads][n] (column sums and diagonal sums as defined above). Same
 * arguments, workspace size and errors as minf_build_vs_index. */
minf_status minf_vs_scores(const void* q, const void* k, int64_t n, int hq, int hkv, int d,
                           const int32_t* heads, int n_heads, int last_q, float scale,
                           float* v_out, float* sl_out, void* workspace, size_t ws_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------------
 * Block-Sparse index ("Method": mean pooling of Q and K over 64-token blocks,
 * and its commutativity with the matrix product, estimate the block index).
 *
 * For each listed query head h, with n_b = ceil(n / 64):
 *   Qbar[b] = mean of q_i over block b, Kbar[c] likewise (a partial last
 *   block averages its own rows); score(b, c) = Qbar[b] . Kbar[c], c <= b;
 *   row b keeps the top-min(k_b, b+1) blocks c, ties to the lower c.
 *
 * blk_idx  device int32 [n_heads][n_b][k_b], ascending, padded with -1.
 * blk_cnt  device int32 [n_heads][n_b] = min(k_b, b + 1).
 * workspace / ws_bytes  at least minf_block_index_workspace_size(n, hq, hkv, n_heads).
 * k_b >= 1.
 * ---------------------------------------------------------------------- */
size_t minf_block_index_workspace_size(int64_t n, int hq, int hkv, int n_heads);
minf_status minf_build_block_index(const void* q, const void* k, int64_t n, int hq, int hkv, int d,
                                   const int32_t* heads, int n_heads, int k_b, int32_t* blk_idx,
                                   int32_t* blk_cnt, void* workspace, size_t ws_bytes,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * Grid pattern with permutation (talk transcript, MMInference part: video
 * frames and patches give grid-like attention, and permuting rows and
 * columns together maps the grid onto blocks; MMInference abstract on the
 * authors' page: the Grid pattern and the permutation-based method).
 *
 * The caller permutes Q, K and V (minf_permute_rows, gather) into an order
 * where the grid becomes blocks (for a frame-major video, patch-major order)
 * and keeps pos[t] = the original position of permuted row t. The index is
 * the Block-Sparse estimate on the permuted sequence: pooled means over its
 * 64-row blocks; key block c is eligible for query block b when
 * min(pos over c) <= max(pos over b); score(b, c) = Qbar[b] . Kbar[c] over
 * eligible c; row b keeps the top-min(k_b, #eligible), ties to the lower c,
 * ascending, padded with -1; blk_cnt[b] = that count. Attention then runs
 * with BLOCK plans carrying pos, and the output rows are scattered back.
 * Same arguments, workspace size and errors as minf_build_block_index, plus
 * pos (device int32 [n], a permutation of 0..n-1; non-null).
 * ---------------------------------------------------------------------- */
minf_status minf_build_permuted_block_index(const void* q, const void* k, int64_t n, int hq, int hkv, int d,
                                            const int32_t* heads, int n_heads, int k_b, const int32_t* pos,
                                            int32_t* blk_idx, int32_t* blk_cnt, void* workspace, size_t ws_bytes,
                                            hipStream_t stream);

/* Row permutation of [heads][n] rows of row_bytes bytes (a multiple of 4):
 * scatter == 0 gathers out[h][t] = x[h][src[t]]; scatter == 1 scatters
 * out[h][src[t]] = x[h][t]. src: device int32 [n], a permutation of 0..n-1
 * (not checked). out must not alias x. MINF_E_UNSUPPORTED when one head holds
 * 2^31 or more 4-byte words (n * row_bytes / 4). */
minf_status minf_permute_rows(const void* x, void* out, int heads, int64_t n, int row_bytes, const int32_t* src,
                              int scatter, hipStream_t stream);

/* Debug export of the pooling step: out is device float [n_heads][n_b][d],
 * the 64-row block means of x ([h_total][n][d] bf16) for the listed heads. */
minf_status minf_block_pool(const void* x, int64_t n, int h_total, int d, const int32_t* heads,
                            int n_heads, float* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse FlashAttention ("Latency and sparse patterns in kernels", Fig. 4:
 * verticals as 1x64 pieces, slashes as 64x64 blocks; talk transcript:
 * blockwise sparse computation on top of FlashAttention).
 *
 * One plan per query head. With b = floor(i / 64), the set of keys row i
 * attends to is:
 *   MINF_KIND_DENSE  : j <= i.
 *   MINF_KIND_ASHAPE : j <= i and (j < sink or i - j < local).
 *   MINF_KIND_VS     : j <= i and (block(j) in Bs(b) or j in v_idx), where
 *                      Bs(b) = { floor((i' - dl) / 64) : i' in block b,
 *                      dl in s_idx, i' - dl >= 0 } (slash lines covered by
 *                      whole 64x64 blocks).
 *   MINF_KIND_BLOCK  : j <= i and block(j) in blk_idx[b][0 .. blk_cnt[b]).
 *   MINF_KIND_VS_WINDOW : j <= i and (j in W(b) or j in v_idx), where W(b) is
 *                      the union over dl in s_idx with 64b + 63 - dl >= 0 of the
 *                      keys [64b - dl, 64b - dl + 64): each slash line as the
 *                      contiguous 64 keys it meets from the block's rows,
 *                      rather than the grid blocks it crosses (a reading of
 *                      the index shifting in the talk transcript's MMInference
 *                      part). Same v_idx / s_idx / k_v / k_s fields as
 *                      MINF_KIND_VS.
 * O_i = softmax over that set of scale * q_i . k_j, applied to V (fp32
 * online softmax and accumulation, bf16 MFMA products, bf16 output). An
 * empty set gives O_i = 0 and LSE_i = -inf.
 *
 * o    device bf16 [hq][n][d].   lse  device float [hq][n] or NULL
 *      (natural-log sum of exponentials of the scaled scores over the set).
 * plans host array [hq]; index pointers inside it are device pointers that
 *      must stay valid until the stream reaches the call. v_idx entries must
 *      be ascending and unique; s_idx entries are offsets in [0, n); blk_idx
 *      rows ascending with -1 padding. Out-of-range entries are ignored.
 * workspace / ws_bytes  at least minf_sparse_attn_workspace_size(n, hq).
 * ---------------------------------------------------------------------- */
#define MINF_KIND_DENSE 0
#define MINF_KIND_ASHAPE 1
#define MINF_KIND_VS 2
#define MINF_KIND_BLOCK 3
#define MINF_KIND_VS_WINDOW 4

typedef struct minf_head_plan {
  int32_t kind;           /* MINF_KIND_* */
  int32_t sink;           /* A-shape: sink tokens (>= 0) */
  int32_t local;          /* A-shape: local window tokens (>= 0) */
  int32_t k_v;            /* VS: entries in v_idx (>= 0) */
  int32_t k_s;            /* VS: entries in s_idx (>= 0) */
  int32_t k_b;            /* BLOCK: row stride of blk_idx (>= 1) */
  const int32_t* v_idx;   /* VS: device, ascending column ids */
  const int32_t* s_idx;   /* VS: device, diagonal offsets */
  const int32_t* blk_idx; /* BLOCK: device [n_b][k_b] */
  const int32_t* blk_cnt; /* BLOCK: device [n_b] */
  const int32_t* pos;     /* BLOCK on a permuted sequence: device [n] original position of
                             every row (see minf_build_permuted_block_index), else NULL */
} minf_head_plan;

size_t minf_sparse_attn_workspace_size(int64_t n, int hq);
minf_status minf_sparse_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t n, int hq, int hkv, int d, float scale,
                             const minf_head_plan* plans, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/* Launch order: with Vertical-Slash heads and n >= 2^17, the heads' offset
 * sets decide on the device whether the workgroups of each XCD take their
 * work items in rounds that start together (long items share K/V tiles in
 * L2) or as one ordinary launch; results are bitwise identical either way.
 * The environment variable MINF_ATTN_ROUNDS=0 (read on every call) keeps the
 * ordinary launch only, as does a stream that is being captured into a graph. The rounds launch
 * has exactly as many workgroups as the device holds at once (two per CU); its
 * waits are bounded, so it ends even if some were not resident together. */

/* A BLOCK plan with pos != NULL describes a permuted sequence (q, k, v, o
 * and lse are all in the permuted row order): key block c may appear in any
 * row of blk_idx, and row i attends to key j when block(j) is listed for
 * block(i) and pos[j] <= pos[i] (causal in the original order). Only BLOCK
 * plans may carry pos (else MINF_E_INVALID_ARG); the workspace is then
 * required as for VS plans. */

/* Dense FlashAttention baseline (the comparison kernel of Fig. 3).
 * causal != 0: row i attends to j <= i; causal == 0: to every j < n.
 * Same layouts as minf_sparse_attn; needs no workspace. */
minf_status minf_dense_attn(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t n, int hq, int hkv, int d, float scale, int causal,
                            hipStream_t stream);

/* ------------------------------------------------------------------------
 * Offline pattern search support (MInference 1.0 article, "Method": each
 * head's pattern is chosen offline by a kernel-aware search that compares
 * candidates at their cost in the sparse kernel; talk transcript, MInference
 * part: attention recall, the share of attention an index keeps).
 * ---------------------------------------------------------------------- */

/* Work of each head's plan in the sparse kernel's unit, summed over query
 * blocks b = 0 .. n_b - 1: the 64-key blocks minf_sparse_attn computes for b
 * plus every gathered vertical column as 1/64 of a block.
 *   DENSE : c <= b.
 *   ASHAPE: sink blocks c < ceil(sink / 64), c <= b, and window blocks from
 *           the block of key 64 b - local + 1 up to b (none when local == 0).
 *   VS    : Bs(b) (as in minf_sparse_attn), plus 1/64 for every column j of
 *           v_idx (ascending, unique, in [0, n)) with j <= b's last row and
 *           block(j) not in Bs(b).
 *   BLOCK : blk_cnt[b].
 * plans  host array [hq] as for minf_sparse_attn (index pointers on the device;
 *        pos is ignored). MINF_KIND_VS_WINDOW plans: MINF_E_UNSUPPORTED.
 * work   device double [hq]; exact (integer block and column counts).
 * workspace / ws_bytes  at least minf_sparse_attn_workspace_size(n, hq) when a
 *        VS plan is present (else may be NULL). n <= 2^20. */
minf_status minf_plan_work(const minf_head_plan* plans, int64_t n, int hq, double* work, void* workspace,
                           size_t ws_bytes, hipStream_t stream);

/* Attention recall of each head's mask from the log-sum-exp rows of sparse
 * and dense attention over the same inputs:
 *   recall[h] = (1 / R) * sum over the R listed rows i of exp(lse_mask[h][i] -
 *   lse_dense[h][i]), a row with lse_mask = -inf (empty mask) counting 0.
 * exp(LSE_mask - LSE_dense) is the share of row i's causal softmax mass that
 * lies inside the mask. fp64 accumulation in a fixed order.
 * lse_mask, lse_dense  device float [hq][n]. rows  device int32 [n_rows] of
 * row ids (entries outside [0, n) count 0), or NULL for every row (R = n).
 * recall  device double [hq]. */
minf_status minf_attention_recall(const float* lse_mask, const float* lse_dense, int64_t n, int hq,
                                  const int32_t* rows, int n_rows, double* recall, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse decoding with top-k block loads ("KV-cache-centric efficient
 * long-context methods" talk transcript: in decoding, loading the KV cache is
 * the bottleneck and can be done sparsely; decode attention splits into a
 * top-k selection and attention over the selected keys. The block estimate is
 * the pooled-key score of the MInference 1.0 article, "Method").
 *
 * One new query row per head (q: [hq][d] bf16) attends to a cache of n keys
 * (K, V: [hkv][n][d] bf16, the new token's own key already appended at n - 1;
 * the query is the last position, so every cached key is visible). With
 * n_b = ceil(n / 64):
 *   score_h(c) = q_h . Kbar_g[c], Kbar_g[c] = mean of K_g over block c (a
 *   partial last block averages its own rows);
 *   blocks_h = top-min(k_b, n_b) of score_h, ties to the lower c, ascending;
 *   O_h = softmax over the keys of blocks_h of scale * q_h . k_j, applied to V
 *   (fp32 softmax and accumulation, bf16 output); LSE_h its natural log-sum-exp.
 * k_b >= n_b selects every block (dense decoding; kbar_t may then be NULL).
 * n is at most 16384 * 64 and hq / hkv at most 8 (else MINF_E_UNSUPPORTED).
 * ---------------------------------------------------------------------- */

/* Block means of K for the decode estimate: kbar_t is device float
 * [hkv][d][n_b] (dimension-major). Blocks c >= first_block are (re)computed,
 * the others are left as they are, so after appending tokens only the last
 * block needs first_block = n_b - 1. */
minf_status minf_decode_pool_keys(const void* k, int64_t n, int hkv, int d, int first_block, float* kbar_t,
                                  hipStream_t stream);

/* Workspace for minf_sparse_decode with this budget (k_b >= n_b: dense). */
size_t minf_decode_workspace_size(int64_t n, int hq, int k_b);

/* blk_idx  device int32 [hq][min(k_b, n_b)] (ascending block ids) or NULL.
 * o        device bf16 [hq][d].  lse  device float [hq] or NULL.
 * k_b >= 1. workspace: at least minf_decode_workspace_size(n, hq, k_b). */
minf_status minf_sparse_decode(const void* q, const void* k, const void* v, const float* kbar_t, int64_t n, int hq,
                               int hkv, int d, float scale, int k_b, int32_t* blk_idx, void* o, float* lse,
                               void* workspace, size_t ws_bytes, hipStream_t stream);

/* Dense decoding baseline: every key of the cache. Workspace: at least
 * minf_decode_workspace_size(n, hq, n_b). */
minf_status minf_dense_decode(const void* q, const void* k, const void* v, int64_t n, int hq, int hkv, int d,
                              float scale, void* o, float* lse, void* workspace, size_t ws_bytes,
                              hipStream_t stream);

/* ------------------------------------------------------------------------
 * Sparse decoding without allocation, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results and errors as minf_sparse_decode, without the
 * workspace: the scratch lives in a static device array of the library,
 * minf_decode_noalloc_max_bytes() bytes on each GPU, held until the process
 * ends. A step whose scratch (minf_decode_workspace_size(n, hq, k_b)) exceeds
 * it returns MINF_E_UNSUPPORTED. The call itself allocates nothing (no
 * hipMalloc, no library allocation). Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (two streams, two threads) race and
 * must be ordered by the caller. The scratch keeps the last call's contents;
 * no call relies on them (each kernel writes every scratch word it later
 * reads).
 * ---------------------------------------------------------------------- */
size_t minf_decode_noalloc_max_bytes(void);
minf_status minf_sparse_decode_noalloc(const void* q, const void* k, const void* v, const float* kbar_t, int64_t n,
                                       int hq, int hkv, int d, float scale, int k_b, int32_t* blk_idx, void* o,
                                       float* lse, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MINF_H */
