"""CPU oracle for MInference-style dynamic sparse attention (test infrastructure).

This module is the checker, not the product: only the test suite, the smoke
check and the benchmark's CPU-baseline leg import it, and it shares no code
with the HIP path. Everything here is NumPy in float64 on values the caller
passes in (bf16 inputs are upcast exactly before they arrive). There is no
tiling, fusion or reordering beyond what the definitions state; a row set is
evaluated one query row (or one 64-row query block) at a time.

Sources (web pages, cited by title and section):
  [A] "MInference 1.0 article: million-token inference on a single A100"
      (news write-up of arXiv 2407.02490), sections "Method" and
      "Latency and sparse patterns in kernels" (Fig. 3, Fig. 4).
  [T] "KV-cache-centric efficient long-context methods" (AICon 2025 talk
      transcript), section "KV-cache-centric methods", MInference part
      (second observation: A-shape, vertical and slash lines, block-local
      patterns) and the unified three-step framework.
  [S] "MInference" abstract on the authors' page (offline pattern, online
      index, sparse kernels).
  [P] the MMInference abstract on the authors' page (the Grid pattern of
      video input and the permutation-based method).
  [D] the same talk transcript, fourth stage of the KV-cache lifecycle
      (decoding is bound by loading the KV cache; load it sparsely) and its
      closing part on dynamic sparsity in decoding (attention decomposes into
      a top-k selection and attention over the selected keys).

Readings where the pages are silent (each one is listed in the design notes):
  * softmax scale sigma = 1/sqrt(d), used in both the VS estimate and attention;
  * the "last Q" of the VS estimate is the last `last_q` (64) query rows, with
    the causal mask applied and each row normalised on its own;
  * diagonal sums are plain sums (no division by the diagonal's length);
  * top-k ties go to the lower index; k larger than what exists is clamped;
  * slash lines are computed at 64x64 block granularity (a superset of the
    exact diagonal entries); verticals are single key columns, dropped when
    their 64-block is already computed;
  * Block-Sparse pools over whole 64-row blocks (a partial last block averages
    its own rows); the block score is the dot product of the pooled vectors,
    with c <= b, and every c <= b is kept when b+1 <= k_b;
  * A-shape is a token-level predicate: j < sink or i - j < local (window
    includes the diagonal), with j <= i;
  * a query row whose mask is empty outputs 0 with LSE = -inf;
  * GQA: query head h reads KV head h // (hq // hkv);
  * sparse decoding [D]: one new query row per head attends to the whole
    cache of n keys (it is the last position); its keys are selected at
    64-token block granularity by the same pooled-key estimate as
    Block-Sparse, score(c) = q . mean(K_c), top-k_b blocks per query head,
    ties to the lower block, with no forced blocks;
  * pattern search (offline): a candidate's work is the kernel's unit (key
    blocks with a mask entry, gathered columns at 1/64 block each) on the
    calibration input; its quality is the attention recall (the causal
    softmax mass inside its mask, averaged over query rows); each head takes
    the highest-recall candidate within a work budget;
  * grid pattern [T], [P]: a video of F frames x P patches in frame-major
    order is permuted to patch-major order (the same permutation for rows
    and columns), and the Block-Sparse estimate runs on the permuted
    sequence; a key block is eligible when one of its keys precedes one of
    the block's queries in the original order, and attention stays causal in
    the original order;
  * VS with slash-aligned windows (the index-shifting alternative): for
    query block b each selected slash delta keeps the 64 keys starting at
    64b - delta, so row 64b + r meets its slash key at window position r;
    Mask(i) = j <= i and (j in one of b's windows or j in V). It contains
    every exact slash entry and, for full query blocks, lies inside the
    64x64-block reading.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 64  # token granularity of blocks, [A] "Latency and sparse patterns in kernels", Fig. 4


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _nblocks(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


# ---------------------------------------------------------------------------
# top-k with the lower-index tie rule ([A] "Method": top-k selection of the
# estimated verticals, slashes and blocks)
# ---------------------------------------------------------------------------
def topk_lowidx(x, k: int) -> np.ndarray:
    """Indices of the k largest entries of x, ties to the lower index, ascending.

    k is clamped to len(x) (a budget above what exists means "everything").
    """
    x = _f64(x)
    k = max(0, min(int(k), x.shape[0]))
    # primary key: value descending; secondary key: index ascending
    order = np.lexsort((np.arange(x.shape[0]), -x))
    return np.sort(order[:k]).astype(np.int64)


# ---------------------------------------------------------------------------
# attention over an explicit per-row mask (definition of softmax attention)
# ---------------------------------------------------------------------------
def attend_rows(q_rows, k, v, mask, scale: float):
    """O and LSE for the given query rows of one head.

    q_rows: [R, d]; k, v: [N, d]; mask: [R, N] boolean (True = the key is in
    the row's mask). O_i = sum_j softmax_j(s_ij) v_j over the mask, with
    s_ij = scale * q_i . k_j; LSE_i = log sum_j exp(s_ij). A row with an empty
    mask gets O_i = 0 and LSE_i = -inf.
    """
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    mask = np.asarray(mask, dtype=bool)
    s = scale * (q_rows @ k.T)
    s = np.where(mask, s, -np.inf)
    empty = ~mask.any(axis=1)
    m = np.where(empty, 0.0, s.max(axis=1))
    e = np.exp(s - m[:, None])  # exp(-inf) = 0 off the mask
    z = e.sum(axis=1)
    zs = np.where(empty, 1.0, z)
    out = (e @ v) / zs[:, None]
    out[empty] = 0.0
    lse = np.where(empty, -np.inf, m + np.log(zs))
    return out, lse


def _kv_head(h: int, hq: int, hkv: int) -> int:
    """GQA reading: consecutive groups of hq // hkv query heads share a KV head."""
    return h // (hq // hkv)


def _row_blocks(n: int, rows):
    """Group the requested rows by 64-row query block: {b: [rows in b]}."""
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    groups: dict[int, list[int]] = {}
    for i in rows.tolist():
        groups.setdefault(i // BLOCK, []).append(i)
    return rows, groups


def dense_attn(q, k, v, hq: int, hkv: int, scale: float, causal: bool = True, rows=None):
    """Dense attention, the baseline every pattern is compared to.

    q: [hq, N, d], k/v: [hkv, N, d]. Returns O [hq, R, d] and LSE [hq, R] for
    the rows `rows` (all rows by default), in the order given.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[1]
    rows, _ = _row_blocks(n, rows)
    out = np.zeros((hq, rows.shape[0], q.shape[2]))
    lse = np.zeros((hq, rows.shape[0]))
    j = np.arange(n)
    mask = (j[None, :] <= rows[:, None]) if causal else np.ones((rows.shape[0], n), bool)
    for h in range(hq):
        g = _kv_head(h, hq, hkv)
        out[h], lse[h] = attend_rows(q[h, rows], k[g], v[g], mask, scale)
    return out, lse


# ---------------------------------------------------------------------------
# Vertical-Slash online estimate ([A] "Method": the attention between the last
# queries and all keys estimates the best vertical and slash indices; [T]
# second observation: vertical lines and slash lines)
# ---------------------------------------------------------------------------
def vs_last_query_probs(q, k, last_q: int, scale: float):
    """Causally masked softmax rows of the last r = min(last_q, N) queries.

    q, k: [N, d] for one query head and its KV head. Returns (P [r, N], rows).
    """
    q, k = _f64(q), _f64(k)
    n = q.shape[0]
    r = min(int(last_q), n)
    rows = np.arange(n - r, n)
    s = scale * (q[rows] @ k.T)
    allowed = np.arange(n)[None, :] <= rows[:, None]
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p = p / p.sum(axis=1, keepdims=True)
    return p, rows


def vs_column_diag_sums(p, rows, n: int):
    """Column sums v[j] = sum_i P_ij and diagonal sums sl[delta] = sum_i P_{i,i-delta}."""
    vcol = p.sum(axis=0)
    sl = np.zeros(n)
    for t, i in enumerate(rows.tolist()):
        # entries P[i, i], P[i, i-1], ..., P[i, 0] sit on delta = 0, 1, ..., i
        sl[: i + 1] += p[t, i::-1]
    return vcol, sl


def vs_index(q, k, last_q: int, k_v: int, k_s: int, scale: float):
    """One head's VS index: (V ascending column ids, D ascending offsets, v, sl)."""
    n = _f64(q).shape[0]
    p, rows = vs_last_query_probs(q, k, last_q, scale)
    vcol, sl = vs_column_diag_sums(p, rows, n)
    return topk_lowidx(vcol, k_v), topk_lowidx(sl, k_s), vcol, sl


def build_vs_index(q, k, hq: int, hkv: int, heads, last_q: int, k_v: int, k_s: int, scale: float):
    """Mirror of the library's VS index call for the listed query heads.

    Returns v_idx [n_heads, min(k_v, N)] and s_idx [n_heads, min(k_s, N)],
    both ascending per head, plus the per-head score arrays (v, sl).
    """
    q, k = _f64(q), _f64(k)
    vi, si, vs, ss = [], [], [], []
    for h in heads:
        g = _kv_head(h, hq, hkv)
        a, b, vc, sl = vs_index(q[h], k[g], last_q, k_v, k_s, scale)
        vi.append(a)
        si.append(b)
        vs.append(vc)
        ss.append(sl)
    return np.array(vi, dtype=np.int64), np.array(si, dtype=np.int64), np.array(vs), np.array(ss)


# ---------------------------------------------------------------------------
# VS index -> kernel mask ([A] "Latency and sparse patterns in kernels",
# Fig. 4: verticals as 1x64 pieces, slashes as 64x64 blocks)
# ---------------------------------------------------------------------------
def vs_block_set(n: int, s_idx, b: int) -> np.ndarray:
    """Bs(b): the key blocks crossed, inside query block b, by the selected diagonals.

    Bs(b) = { floor((i - delta) / 64) : i in block b, delta in D, i - delta >= 0 }.
    """
    s_idx = np.asarray(s_idx, dtype=np.int64)
    rows = np.arange(BLOCK * b, min(BLOCK * b + BLOCK, n))
    j = rows[:, None] - s_idx[None, :]
    j = j[j >= 0]
    return np.unique(j // BLOCK)


def vs_column_set(n: int, s_idx, v_idx, b: int) -> np.ndarray:
    """Cv(b): selected columns up to the block's last row whose block is not in Bs(b)."""
    bs = set(vs_block_set(n, s_idx, b).tolist())
    last = min(BLOCK * b + BLOCK - 1, n - 1)
    return np.array(sorted({int(j) for j in np.asarray(v_idx).tolist()
                            if j <= last and (int(j) // BLOCK) not in bs}), dtype=np.int64)


def vs_mask_block(n: int, s_idx, v_idx, b: int, rows) -> np.ndarray:
    """Mask rows for query rows `rows` of block b: j <= i and (block(j) in Bs(b) or j in Cv(b))."""
    j = np.arange(n)
    in_blk = np.isin(j // BLOCK, vs_block_set(n, s_idx, b))
    in_col = np.isin(j, vs_column_set(n, s_idx, v_idx, b))
    rows = np.asarray(rows, dtype=np.int64)
    return (j[None, :] <= rows[:, None]) & (in_blk | in_col)[None, :]


# ---------------------------------------------------------------------------
# VS index with slash-aligned windows ([T] MMInference part: index shifting,
# i.e. reading keys at a row-dependent offset, lines slashes up into dense
# pieces; the reading here keeps, for query block b and each selected slash
# delta, the 64 consecutive keys that start at 64b - delta: row 64b + r finds
# its slash key at window position r, so one 64x64 product per slash covers
# the slash inside the block)
# ---------------------------------------------------------------------------
def vs_window_set(n: int, s_idx, b: int) -> np.ndarray:
    """Keys of query block b's slash windows: union over delta in D with
    64b + 63 - delta >= 0 of [64b - delta, 64b - delta + 64), clipped to [0, n)."""
    keys = set()
    for dl in np.asarray(s_idx, dtype=np.int64).tolist():
        lo = BLOCK * b - dl
        if lo + BLOCK - 1 < 0:
            continue
        keys.update(range(max(0, lo), min(n, lo + BLOCK)))
    return np.array(sorted(keys), dtype=np.int64)


def vsw_mask_block(n: int, s_idx, v_idx, b: int, rows) -> np.ndarray:
    """Mask rows of block b for the window reading: j <= i and (j in a slash
    window of b or j in V)."""
    j = np.arange(n)
    sel = np.isin(j, vs_window_set(n, s_idx, b)) | np.isin(j, np.asarray(v_idx, dtype=np.int64))
    rows = np.asarray(rows, dtype=np.int64)
    return (j[None, :] <= rows[:, None]) & sel[None, :]


def vertical_tiles(n: int, s_idx, v_idx, b: int, windows: bool) -> list:
    """The skip-column read of query block b's vertical lines ([T] MMInference
    part: reading with skipped columns turns the lines into dense pieces): the
    selected columns up to the block's last row that the block's slash tiles
    do not already hold (its windows when `windows`, else the blocks of Bs(b)),
    in ascending order, cut into tiles of 64 columns ([A] Fig. 4: verticals in
    1x64 pieces). Against the block's rows each tile is dense except where a
    column lies past a row (j > i), a staircase inside the diagonal block."""
    last = min(BLOCK * b + BLOCK - 1, n - 1)
    if windows:
        held = set(vs_window_set(n, s_idx, b).tolist())
        cols = sorted({int(j) for j in np.asarray(v_idx).tolist() if 0 <= j <= last and int(j) not in held})
    else:
        cols = vs_column_set(n, s_idx, v_idx, b).tolist()
    return [np.array(cols[i:i + BLOCK], dtype=np.int64) for i in range(0, len(cols), BLOCK)]


# ---------------------------------------------------------------------------
# Block-Sparse online estimate ([A] "Method": mean pooling of Q and K, and the
# commutativity of mean pooling with the matrix product, give the block index)
# ---------------------------------------------------------------------------
def pool_blocks(x) -> np.ndarray:
    """Mean of the rows of each 64-row block of x [N, d] -> [n_b, d]."""
    x = _f64(x)
    n = x.shape[0]
    return np.stack([x[BLOCK * b: BLOCK * b + BLOCK].mean(axis=0) for b in range(_nblocks(n))])


def block_scores(q, k) -> np.ndarray:
    """score(b, c) = mean(Q_b) . mean(K_c) for c <= b; -inf above the block diagonal."""
    qb, kb = pool_blocks(q), pool_blocks(k)
    s = qb @ kb.T
    nb = s.shape[0]
    return np.where(np.arange(nb)[None, :] <= np.arange(nb)[:, None], s, -np.inf)


def block_index(q, k, k_b: int):
    """Per query block b: the top-k_b key blocks c <= b (ascending), and the score matrix."""
    s = block_scores(q, k)
    nb = s.shape[0]
    sel = [topk_lowidx(s[b, : b + 1], k_b) for b in range(nb)]
    return sel, s


def build_block_index(q, k, hq: int, hkv: int, heads, k_b: int):
    """Mirror of the library's block index call.

    Returns blk_idx [n_heads, n_b, k_b] (ascending, padded with -1),
    blk_cnt [n_heads, n_b] = min(k_b, b+1), and the per-head score matrices.
    """
    q, k = _f64(q), _f64(k)
    n = q.shape[1]
    nb = _nblocks(n)
    idx = -np.ones((len(heads), nb, k_b), dtype=np.int64)
    cnt = np.zeros((len(heads), nb), dtype=np.int64)
    scores = []
    for t, h in enumerate(heads):
        g = _kv_head(h, hq, hkv)
        sel, s = block_index(q[h], k[g], k_b)
        for b, cs in enumerate(sel):
            idx[t, b, : len(cs)] = cs
            cnt[t, b] = len(cs)
        scores.append(s)
    return idx, cnt, scores


def bs_mask_block(n: int, blocks, b: int, rows) -> np.ndarray:
    """Mask rows for block b of a Block-Sparse head: j <= i and block(j) selected for b."""
    j = np.arange(n)
    sel = np.isin(j // BLOCK, np.asarray(blocks, dtype=np.int64))
    rows = np.asarray(rows, dtype=np.int64)
    return (j[None, :] <= rows[:, None]) & sel[None, :]


# ---------------------------------------------------------------------------
# A-shape ([T] second observation: attention gathers at the start of the input
# and in a local window around the current position)
# ---------------------------------------------------------------------------
def ashape_mask_row(i: int, n: int, sink: int, local: int) -> np.ndarray:
    j = np.arange(n)
    return (j <= i) & ((j < sink) | (i - j < local))


def ashape_mask_block(n: int, sink: int, local: int, rows) -> np.ndarray:
    return np.stack([ashape_mask_row(int(i), n, sink, local) for i in np.asarray(rows).tolist()])


# ---------------------------------------------------------------------------
# sparse attention over a per-head plan ([A] "Method" and [S]: with the
# pattern and sparse indices, compute attention only where the index says)
# ---------------------------------------------------------------------------
def plan_mask_block(plan: dict, n: int, b: int, rows) -> np.ndarray:
    """Boolean mask [len(rows), N] of one head's plan for rows inside query block b.

    plan kinds: "dense" (causal), "ashape" (sink, local), "vs" (v_idx, s_idx),
    "vs_window" (v_idx, s_idx; slash-aligned windows), "block" (blk_idx
    [n_b, k_b] padded with -1 and blk_cnt [n_b]).
    """
    kind = plan["kind"]
    rows = np.asarray(rows, dtype=np.int64)
    if kind == "dense":
        return np.arange(n)[None, :] <= rows[:, None]
    if kind == "ashape":
        return ashape_mask_block(n, int(plan["sink"]), int(plan["local"]), rows)
    if kind == "vs":
        return vs_mask_block(n, plan["s_idx"], plan["v_idx"], b, rows)
    if kind == "vs_window":
        return vsw_mask_block(n, plan["s_idx"], plan["v_idx"], b, rows)
    if kind == "block":
        c = int(plan["blk_cnt"][b])
        return bs_mask_block(n, np.asarray(plan["blk_idx"][b])[:c], b, rows)
    raise ValueError(f"unknown plan kind {kind!r}")


def sparse_attn(q, k, v, hq: int, hkv: int, scale: float, plans, rows=None):
    """O_i = softmax over Mask(i) of s_ij, applied to V, for every head's plan.

    q: [hq, N, d], k/v: [hkv, N, d]; plans: list of hq dicts. Returns O and
    LSE for `rows` (all rows by default), in the order given.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[1]
    rows, groups = _row_blocks(n, rows)
    pos = {int(i): t for t, i in enumerate(rows.tolist())}
    out = np.zeros((hq, rows.shape[0], q.shape[2]))
    lse = np.zeros((hq, rows.shape[0]))
    for h in range(hq):
        g = _kv_head(h, hq, hkv)
        for b, rs in groups.items():
            m = plan_mask_block(plans[h], n, b, rs)
            o, l = attend_rows(q[h, rs], k[g], v[g], m, scale)
            idx = [pos[i] for i in rs]
            out[h, idx] = o
            lse[h, idx] = l
    return out, lse


# ---------------------------------------------------------------------------
# Sparse decoding with top-k block loads ([D]: the decode step is bound by
# loading the KV cache, so only the keys of the top-k estimated blocks are
# loaded and attended; the estimate is the pooled-key score of [A] "Method")
# ---------------------------------------------------------------------------
def decode_block_index(q_row, k, k_b: int):
    """Top-k_b key blocks of one decode query: ascending block ids, and the scores.

    score(c) = q . mean(K_c) over every 64-token block c of the cache (a partial
    last block averages its own rows); ties go to the lower block.
    """
    s = pool_blocks(k) @ _f64(q_row)
    return topk_lowidx(s, k_b), s


def decode_mask(n: int, blocks) -> np.ndarray:
    """Keys of the selected blocks (the decode query is the last position, so
    every key of the cache is causally visible)."""
    m = np.zeros(n, dtype=bool)
    for c in np.asarray(blocks, dtype=np.int64).tolist():
        m[BLOCK * c: BLOCK * c + BLOCK] = True
    return m


def sparse_decode(q, k, v, hq: int, hkv: int, scale: float, k_b: int):
    """One decode step: q [hq, d] against the cache k/v [hkv, N, d].

    Returns (blk_idx [hq, min(k_b, n_b)], O [hq, d], LSE [hq]). With k_b >= n_b
    every block is selected and this is dense decoding.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = k.shape[1]
    kk = min(int(k_b), _nblocks(n))
    idx = np.zeros((hq, kk), dtype=np.int64)
    out = np.zeros((hq, q.shape[1]))
    lse = np.zeros(hq)
    for h in range(hq):
        g = _kv_head(h, hq, hkv)
        sel, _ = decode_block_index(q[h], k[g], kk)
        idx[h] = sel
        o, l = attend_rows(q[h][None, :], k[g], v[g], decode_mask(n, sel)[None, :], scale)
        out[h], lse[h] = o[0], l[0]
    return idx, out, lse


def dense_decode(q, k, v, hq: int, hkv: int, scale: float):
    """One decode step attending every key of the cache: O [hq, d], LSE [hq]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = k.shape[1]
    out = np.zeros((hq, q.shape[1]))
    lse = np.zeros(hq)
    for h in range(hq):
        g = _kv_head(h, hq, hkv)
        o, l = attend_rows(q[h][None, :], k[g], v[g], np.ones((1, n), bool), scale)
        out[h], lse[h] = o[0], l[0]
    return out, lse


# ---------------------------------------------------------------------------
# Kernel-aware pattern search ([A] "Method": each head's pattern is chosen
# offline by a kernel-aware sparse pattern search; [T]: offline per-head
# pattern search, and attention recall as the share of attention an index
# keeps)
# ---------------------------------------------------------------------------
def plan_blocks(plan: dict, n: int) -> float:
    """Work of a plan in the kernel's unit, summed over query blocks: the key
    blocks whose mask block has an entry, plus each gathered column as 1/64 of
    a block (VS columns outside the computed blocks)."""
    nb = _nblocks(n)
    kind = plan["kind"]
    if kind == "dense":
        return nb * (nb + 1) / 2
    if kind == "block":
        return float(np.sum(plan["blk_cnt"]))
    tot = 0.0
    for b in range(nb):
        rows = np.arange(BLOCK * b, min(BLOCK * b + BLOCK, n))
        if kind == "vs":
            tot += len(vs_block_set(n, plan["s_idx"], b)) + len(vs_column_set(n, plan["s_idx"], plan["v_idx"], b)) / BLOCK
        else:
            m = plan_mask_block(plan, n, b, rows)
            hit = m.any(axis=0)
            tot += len(np.unique(np.nonzero(hit)[0] // BLOCK))
    return tot


def pattern_recall(q, k, plan: dict, scale: float, rows=None) -> float:
    """Mean over query rows of the causal softmax probability mass that falls
    inside the plan's mask (1.0 for the dense plan)."""
    q, k = _f64(q), _f64(k)
    n = q.shape[0]
    rows, groups = _row_blocks(n, rows)
    tot = 0.0
    for b, rs in groups.items():
        s = scale * (q[rs] @ k.T)
        causal = np.arange(n)[None, :] <= np.asarray(rs)[:, None]
        s = np.where(causal, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        m = plan_mask_block(plan, n, b, rs)
        tot += float((p * m).sum())
    return tot / rows.shape[0]


def candidate_plan(q, k, cand: dict, scale: float, last_q: int = 64) -> dict:
    """The plan a candidate pattern gives on this head's data: its index built online."""
    kind = cand["kind"]
    if kind in ("dense", "ashape"):
        return dict(cand)
    if kind == "vs":
        vi, si, _, _ = vs_index(q, k, last_q, int(cand["k_v"]), int(cand["k_s"]), scale)
        return dict(kind="vs", v_idx=vi, s_idx=si)
    if kind == "block":
        k_b = int(cand["k_b"])
        sel, _ = block_index(q, k, k_b)
        idx = -np.ones((len(sel), k_b), dtype=np.int64)
        cnt = np.zeros(len(sel), dtype=np.int64)
        for b, cs in enumerate(sel):
            idx[b, : len(cs)] = cs
            cnt[b] = len(cs)
        return dict(kind="block", blk_idx=idx, blk_cnt=cnt)
    raise ValueError(f"unknown candidate kind {kind!r}")


def search_head_pattern(q, k, candidates, scale: float, budget: float, last_q: int = 64, rows=None):
    """Pick one head's pattern: among the candidates whose work on this input is
    within `budget` blocks, the one with the highest attention recall (ties to
    the lower work, then to the earlier candidate). Returns (index or -1, table
    of (blocks, recall) per candidate)."""
    table = []
    for cand in candidates:
        plan = candidate_plan(q, k, cand, scale, last_q)
        table.append((plan_blocks(plan, _f64(q).shape[0]), pattern_recall(q, k, plan, scale, rows)))
    best = -1
    for c, (cost, rec) in enumerate(table):
        if cost > budget:
            continue
        if best < 0 or rec > table[best][1] or (rec == table[best][1] and cost < table[best][0]):
            best = c
    return best, table


# ---------------------------------------------------------------------------
# Grid pattern with permutation ([T] MMInference part: video frames and
# patches give grid-like attention; permuting rows and columns together
# (attention is invariant under it) turns the grid into blocks that the block
# kernels compute densely; [P] MMInference abstract: the Grid pattern, the
# permutation-based method, the sparse distribution built from the input)
# ---------------------------------------------------------------------------
def grid_permutation(frames: int, patches: int) -> np.ndarray:
    """src[t'] = original index of permuted row t' for the patch-major order of a
    frame-major video layout: original t = f * patches + p, permuted t' = p * frames + f."""
    f = np.arange(frames)
    p = np.arange(patches)
    return (f[None, :] * patches + p[:, None]).reshape(-1).astype(np.int64)


def permuted_block_index(q, k, src, k_b: int):
    """Block index of a permuted head: pooled Q and K over 64-row blocks of the
    permuted sequence (q[src], k[src]); key block c is eligible for query block b
    when some key of c precedes some query of b in the original order
    (min src over c <= max src over b); the top-k_b eligible blocks by the
    pooled score, ties to the lower c, ascending. Returns (list of selections,
    score matrix with -inf where not eligible)."""
    src = np.asarray(src, dtype=np.int64)
    qp, kp = _f64(q)[src], _f64(k)[src]
    n = src.shape[0]
    nb = _nblocks(n)
    lo = np.array([src[BLOCK * c: BLOCK * c + BLOCK].min() for c in range(nb)])
    hi = np.array([src[BLOCK * b: BLOCK * b + BLOCK].max() for b in range(nb)])
    s = pool_blocks(qp) @ pool_blocks(kp).T
    s = np.where(lo[None, :] <= hi[:, None], s, -np.inf)
    sel = []
    for b in range(nb):
        ok = np.nonzero(np.isfinite(s[b]))[0]
        pick = topk_lowidx(s[b, ok], k_b)
        sel.append(np.sort(ok[pick]))
    return sel, s


def permuted_block_attn(q, k, v, src, sel, scale: float, rows=None):
    """Attention of one head whose blocks were chosen in the permuted order,
    evaluated in the original order: key j is in Mask(i) when j <= i and the
    permuted block of j is selected for the permuted block of i. Returns O and
    LSE for the original rows `rows` (all by default)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    src = np.asarray(src, dtype=np.int64)
    n = q.shape[0]
    inv = np.empty(n, dtype=np.int64)
    inv[src] = np.arange(n)
    pblk = inv // BLOCK
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    j = np.arange(n)
    mask = np.zeros((rows.shape[0], n), dtype=bool)
    for t, i in enumerate(rows.tolist()):
        allowed = np.isin(pblk, np.asarray(sel[pblk[i]], dtype=np.int64))
        mask[t] = (j <= i) & allowed
    return attend_rows(q[rows], k, v, mask, scale)


def default_scale(d: int) -> float:
    """sigma = 1/sqrt(d): the pages never state the scale; standard attention's is used."""
    return 1.0 / math.sqrt(d)
