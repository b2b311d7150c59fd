"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the oracle against something the pages or the mathematics
fix: hand-derived closed forms (tests/golden), brute force written as scalar
loops on tiny inputs, a library routine (torch SDPA in float64) for the cases
that reduce to one, identities (full budgets equal dense causal attention;
pooled block scores equal the mean of raw block scores), invariants (each
softmax row sums to 1) and planted-structure recovery.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from workload import planted_qkv

GOLD = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.txt")


def _golden():
    out = {}
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = [float(x) for x in vals]
    return out


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- golden
def test_golden_uniform_causal():
    g = _golden()
    n = int(g["uniform_causal.n"][0])
    q = np.zeros((1, n, 1))
    k = np.zeros((1, n, 1))
    v = np.arange(n, dtype=np.float64).reshape(1, n, 1)
    o, lse = O.dense_attn(q, k, v, 1, 1, 1.0)
    np.testing.assert_allclose(o[0, :, 0], g["uniform_causal.o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], np.log(g["uniform_causal.lse_exp"]), rtol=0, atol=1e-15)


def test_golden_two_keys():
    g = _golden()
    q = np.array([[[0.0], [math.log(3.0)]]])
    k = np.array([[[0.0], [1.0]]])
    v = np.array([[[10.0], [2.0]]])
    o, lse = O.dense_attn(q, k, v, 1, 1, 1.0)
    np.testing.assert_allclose(o[0, :, 0], g["two_keys.o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(g["two_keys.lse_exp"]), rtol=0, atol=1e-14)


def test_golden_vs_uniform():
    g = _golden()
    q = np.zeros((4, 1))
    k = np.zeros((4, 1))
    vi, si, vc, sl = O.vs_index(q, k, last_q=2, k_v=2, k_s=1, scale=1.0)
    np.testing.assert_allclose(vc, np.array(g["vs_uniform.v_num"]) / g["vs_uniform.v_den"][0], atol=1e-15)
    np.testing.assert_allclose(sl, np.array(g["vs_uniform.sl_num"]) / g["vs_uniform.sl_den"][0], atol=1e-15)
    assert vi.tolist() == [int(x) for x in g["vs_uniform.top2_v"]]
    assert si.tolist() == [int(x) for x in g["vs_uniform.top1_s"]]


def test_golden_bs_pool():
    g = _golden()
    q = np.ones((128, 1))
    k = np.arange(128, dtype=np.float64).reshape(128, 1)
    np.testing.assert_allclose(O.pool_blocks(k)[:, 0], g["bs_pool.kbar"], atol=1e-13)
    sel, s = O.block_index(q, k, k_b=1)
    assert sel[1].tolist() == [int(x) for x in g["bs_pool.top1_row1"]]
    assert sel[0].tolist() == [0]


# ---------------------------------------------------------------- top-k
def test_topk_lowidx_against_full_sort():
    rng = np.random.default_rng(3)
    for n in [1, 2, 7, 50]:
        for trial in range(20):
            x = rng.integers(0, 4, size=n).astype(np.float64)  # many exact ties
            pairs = sorted(range(n), key=lambda i: (-x[i], i))
            for k in range(0, n + 2):
                want = sorted(pairs[: min(k, n)])
                assert O.topk_lowidx(x, k).tolist() == want


# ---------------------------------------------------------------- dense
def _dense_loops(q, k, v, scale):
    n, d = q.shape
    out = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i in range(n):
        s = [scale * sum(q[i, t] * k[j, t] for t in range(d)) for j in range(i + 1)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        for j in range(i + 1):
            out[i] += (w[j] / z) * v[j]
        lse[i] = m + math.log(z)
    return out, lse


def test_dense_brute_force_loops():
    n, d = 37, 5
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    want_o, want_l = _dense_loops(q, k, v, 0.7)
    o, l = O.dense_attn(q[None], k[None], v[None], 1, 1, 0.7)
    np.testing.assert_allclose(o[0], want_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l[0], want_l, rtol=0, atol=1e-12)


def test_dense_matches_torch_sdpa_gqa():
    hq, hkv, n, d = 4, 2, 300, 16
    q, k, v = _rand((hq, n, d), 4), _rand((hkv, n, d), 5), _rand((hkv, n, d), 6)
    scale = 1 / math.sqrt(d)
    o, _ = O.dense_attn(q, k, v, hq, hkv, scale)
    kk = torch.from_numpy(np.repeat(k, hq // hkv, axis=0))
    vv = torch.from_numpy(np.repeat(v, hq // hkv, axis=0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kk, vv, is_causal=True, scale=scale).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_dense_noncausal_matches_sdpa():
    n, d = 70, 8
    q, k, v = _rand((1, n, d), 7), _rand((1, n, d), 8), _rand((1, n, d), 9)
    o, _ = O.dense_attn(q, k, v, 1, 1, 0.3, causal=False)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.3).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_row_subset_equals_full():
    n, d = 200, 8
    q, k, v = _rand((2, n, d), 10), _rand((1, n, d), 11), _rand((1, n, d), 12)
    o, l = O.dense_attn(q, k, v, 2, 1, 0.4)
    rows = [199, 0, 64, 65, 130]
    o2, l2 = O.dense_attn(q, k, v, 2, 1, 0.4, rows=rows)
    np.testing.assert_array_equal(o2, o[:, rows])
    np.testing.assert_array_equal(l2, l[:, rows])


# ---------------------------------------------------------------- A-shape
def test_ashape_matches_sdpa_with_explicit_mask():
    n, d, sink, local = 333, 8, 10, 70
    q, k, v = _rand((1, n, d), 13), _rand((1, n, d), 14), _rand((1, n, d), 15)
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    mask = (j <= i) & ((j < sink) | (i - j < local))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=0.35).numpy()
    o, _ = O.sparse_attn(q, k, v, 1, 1, 0.35, [dict(kind="ashape", sink=sink, local=local)])
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- full budgets
@pytest.mark.parametrize("n", [64, 200, 257])
def test_full_budgets_equal_dense(n):
    d, hq, hkv = 8, 2, 1
    q, k, v = _rand((hq, n, d), 16), _rand((hkv, n, d), 17), _rand((hkv, n, d), 18)
    scale = 0.4
    dense_o, dense_l = O.dense_attn(q, k, v, hq, hkv, scale)
    nb = (n + 63) // 64
    vi, si, _, _ = O.build_vs_index(q, k, hq, hkv, [0, 1], 64, n, n, scale)
    bi, bc, _ = O.build_block_index(q, k, hq, hkv, [0, 1], nb)
    plans_list = [
        [dict(kind="vs", v_idx=vi[h], s_idx=si[h]) for h in range(hq)],
        # all offsets alone cover every causal block
        [dict(kind="vs", v_idx=np.array([], np.int64), s_idx=np.arange(n)) for h in range(hq)],
        [dict(kind="block", blk_idx=bi[h], blk_cnt=bc[h]) for h in range(hq)],
        [dict(kind="ashape", sink=0, local=n) for h in range(hq)],
        [dict(kind="ashape", sink=n, local=1) for h in range(hq)],
    ]
    causal = np.tril(np.ones((n, n), bool))
    for plans in plans_list:
        for b in range(nb):
            rows = np.arange(64 * b, min(64 * b + 64, n))
            assert np.array_equal(O.plan_mask_block(plans[0], n, b, rows), causal[rows])
        o, l = O.sparse_attn(q, k, v, hq, hkv, scale, plans)
        np.testing.assert_allclose(o, dense_o, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, dense_l, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- Block-Sparse
def test_pooled_score_equals_mean_of_raw_block_scores():
    n, d = 150, 6  # ragged last block of 22 rows
    q, k = _rand((n, d), 19), _rand((n, d), 20)
    s = O.block_scores(q, k)
    nb = 3
    for b in range(nb):
        for c in range(b + 1):
            rb = range(64 * b, min(64 * b + 64, n))
            rc = range(64 * c, min(64 * c + 64, n))
            tot = 0.0
            for i in rb:
                for j in rc:
                    tot += sum(q[i, t] * k[j, t] for t in range(d))
            want = tot / (len(rb) * len(rc))
            assert abs(s[b, c] - want) <= 1e-12 * max(1.0, abs(want))
        for c in range(b + 1, nb):
            assert s[b, c] == -np.inf


def test_block_index_rows_and_mask():
    n, d, kb = 64 * 9 + 5, 8, 3
    q, k, v = _rand((1, n, d), 21), _rand((1, n, d), 22), _rand((1, n, d), 23)
    idx, cnt, scores = O.build_block_index(q, k, 1, 1, [0], kb)
    for b in range(10):
        c = int(cnt[0, b])
        assert c == min(kb, b + 1)
        sel = idx[0, b, :c]
        assert list(sel) == sorted(sel) and all(0 <= x <= b for x in sel)
        assert (idx[0, b, c:] == -1).all()
        row = scores[0][b, : b + 1]
        worst_kept = min(row[sel])
        others = [row[x] for x in range(b + 1) if x not in set(sel.tolist())]
        assert all(o <= worst_kept for o in others)
    # mask by brute force: (i, j) kept iff j <= i and block(j) selected for block(i)
    plan = dict(kind="block", blk_idx=idx[0], blk_cnt=cnt[0])
    for b in range(10):
        rows = np.arange(64 * b, min(64 * b + 64, n))
        m = O.plan_mask_block(plan, n, b, rows)
        sel = set(idx[0, b, : cnt[0, b]].tolist())
        for t, i in enumerate(rows[::13]):
            for j in range(0, n, 7):
                assert m[t * 13, j] == (j <= i and (j // 64) in sel)


# ---------------------------------------------------------------- Vertical-Slash
def _vs_loops(q, k, last_q, scale):
    n, d = q.shape
    r = min(last_q, n)
    vcol = [0.0] * n
    sl = [0.0] * n
    for i in range(n - r, n):
        s = [scale * sum(q[i, t] * k[j, t] for t in range(d)) for j in range(i + 1)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = sum(w)
        for j in range(i + 1):
            p = w[j] / z
            vcol[j] += p
            sl[i - j] += p
    return vcol, sl


@pytest.mark.parametrize("n,last_q", [(1, 64), (5, 64), (64, 64), (65, 64), (130, 3), (200, 64)])
def test_vs_index_brute_force(n, last_q):
    d = 8
    q, k = _rand((n, d), 24 + n), _rand((n, d), 25 + n, 1.5)
    vcol, sl = _vs_loops(q, k, last_q, 0.5)
    for k_v in sorted({0, 1, 3, n // 2, n, n + 5}):
        for k_s in sorted({0, 2, n // 3, n}):
            vi, si, vc, ss = O.vs_index(q, k, last_q, k_v, k_s, 0.5)
            np.testing.assert_allclose(vc, vcol, rtol=0, atol=1e-12)
            np.testing.assert_allclose(ss, sl, rtol=0, atol=1e-12)
            want_v = sorted(sorted(range(n), key=lambda j: (-vcol[j], j))[: min(k_v, n)])
            want_s = sorted(sorted(range(n), key=lambda j: (-sl[j], j))[: min(k_s, n)])
            assert vi.tolist() == want_v
            assert si.tolist() == want_s
    r = min(last_q, n)
    assert abs(sum(vcol) - r) < 1e-12 and abs(sum(sl) - r) < 1e-12


def test_vs_mask_brute_force():
    n = 64 * 5 + 17
    rng = np.random.default_rng(26)
    for trial in range(6):
        s_idx = np.sort(rng.choice(n, size=rng.integers(0, 6), replace=False))
        v_idx = np.sort(rng.choice(n, size=rng.integers(0, 9), replace=False))
        plan = dict(kind="vs", v_idx=v_idx, s_idx=s_idx)
        for b in range(6):
            rows = np.arange(64 * b, min(64 * b + 64, n))
            m = O.plan_mask_block(plan, n, b, rows)
            # Bs(b) straight from its definition, with loops
            bs = set()
            for i in rows:
                for dlt in s_idx:
                    if i - dlt >= 0:
                        bs.add((i - dlt) // 64)
            for t, i in enumerate(rows):
                for j in range(n):
                    want = j <= i and ((j // 64) in bs or j in set(v_idx.tolist()))
                    assert m[t, j] == want


def test_vs_planted_recovery_c1_shape():
    # 1 head, N = 4096, last_q = 64, top-64 verticals and slashes, planted with the calibrated gain
    for seed in (1000, 1001, 1002):
        q, k, v, info = planted_qkv(4096, 1, 1, seed=seed)
        vi, si, _, _ = O.vs_index(q[0].float().numpy(), k[0].float().numpy(), 64, 64, 64, 1 / math.sqrt(128))
        assert set(info.columns[0]) <= set(vi.tolist())
        assert set(info.offsets) <= set(si.tolist())
        # tight budgets: the 4 planted offsets are exactly the top-4 slashes; the 8 planted
        # columns sit in the top-16 verticals (the other top columns are the last keys,
        # lifted by the delta = 0 and 1 slash plants)
        vi16, si4, _, _ = O.vs_index(q[0].float().numpy(), k[0].float().numpy(), 64, 16, 4, 1 / math.sqrt(128))
        assert set(info.columns[0]) <= set(vi16.tolist())
        assert si4.tolist() == sorted(info.offsets)


def test_vs_literal_gain_does_not_recover_verticals():
    # the recipe's literal gain (1, 3) is too weak to surface the planted columns
    q, k, v, info = planted_qkv(4096, 1, 1, seed=1000, vert_gain=(1.0, 3.0))
    vi, si, _, _ = O.vs_index(q[0].float().numpy(), k[0].float().numpy(), 64, 64, 64, 1 / math.sqrt(128))
    assert len(set(info.columns[0]) & set(vi.tolist())) <= 2
    assert set(info.offsets) <= set(si.tolist())


# ---------------------------------------------------------------- empty rows
def test_empty_rows_give_zero_and_neg_inf():
    n, d = 150, 4
    q, k, v = _rand((1, n, d), 27), _rand((1, n, d), 28), _rand((1, n, d), 29)
    plans = [dict(kind="vs", v_idx=np.array([], np.int64), s_idx=np.array([], np.int64))]
    o, l = O.sparse_attn(q, k, v, 1, 1, 0.5, plans)
    assert (o == 0).all() and np.isneginf(l).all()
    # only offset 64 (block offset 1): block 0 has nothing to attend; later blocks do
    plans = [dict(kind="vs", v_idx=np.array([], np.int64), s_idx=np.array([64]))]
    o, l = O.sparse_attn(q, k, v, 1, 1, 0.5, plans)
    assert (o[0, :64] == 0).all() and np.isneginf(l[0, :64]).all()
    assert np.isfinite(l[0, 64:]).all()


def test_bf16_inputs_upcast_exactly():
    x = torch.randn(16, 8).to(torch.bfloat16)
    np.testing.assert_array_equal(O.minf_oracle._f64(x.float().numpy()), x.double().numpy())


# ---------------------------------------------------------------------------
# sparse decoding (one query row per head against the cache)
# ---------------------------------------------------------------------------
def test_decode_full_budget_equals_last_row_of_causal_sdpa():
    # a decode query is the last position: full budget must equal the last row of
    # causal prefill attention computed by the library routine in fp64
    rng = np.random.default_rng(11)
    n, hq, hkv, d = 200, 4, 2, 16
    q = rng.standard_normal((hq, n, d))
    k = rng.standard_normal((hkv, n, d))
    v = rng.standard_normal((hkv, n, d))
    scale = 1 / math.sqrt(d)
    idx, o, lse = O.sparse_decode(q[:, -1], k, v, hq, hkv, scale, k_b=10)
    assert idx.shape == (hq, 4) and all(list(r) == [0, 1, 2, 3] for r in idx)
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(np.repeat(k, hq // hkv, axis=0))
    vt = torch.from_numpy(np.repeat(v, hq // hkv, axis=0))
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)[:, -1]
    assert np.abs(o - want.numpy()).max() < 1e-12
    od, ld = O.dense_decode(q[:, -1], k, v, hq, hkv, scale)
    assert np.abs(od - o).max() < 1e-12 and np.abs(ld - lse).max() < 1e-12


def test_decode_block_scores_equal_mean_of_raw_scores_and_selection_is_brute_force():
    # commutativity of pooling with the product: q . mean(K_c) = mean_j (q . k_j);
    # selection against a full sort of those raw means; mask by explicit loops
    rng = np.random.default_rng(12)
    n, d = 300, 8
    q = rng.standard_normal(d)
    k = rng.standard_normal((n, d))
    sel, s = O.decode_block_index(q, k, 3)
    raw = [np.mean([q @ k[j] for j in range(64 * c, min(64 * c + 64, n))]) for c in range(5)]
    assert np.allclose(s, raw, rtol=1e-12, atol=1e-12)
    order = sorted(range(5), key=lambda c: (-raw[c], c))[:3]
    assert list(sel) == sorted(order)
    m = O.decode_mask(n, sel)
    for j in range(n):
        assert m[j] == (j // 64 in order)


def test_decode_output_is_softmax_over_selected_keys_brute_force():
    rng = np.random.default_rng(13)
    n, d = 150, 4
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((1, n, d))
    v = rng.standard_normal((1, n, d))
    idx, o, lse = O.sparse_decode(q, k, v, 1, 1, 0.5, k_b=1)
    keys = [j for j in range(n) if j // 64 == idx[0, 0]]
    w = [math.exp(0.5 * sum(q[0, t] * k[0, j, t] for t in range(d))) for j in keys]
    z = sum(w)
    want = [sum(w[a] * v[0, keys[a], t] for a in range(len(keys))) / z for t in range(d)]
    assert np.allclose(o[0], want, rtol=1e-12, atol=1e-12)
    assert abs(lse[0] - math.log(z)) < 1e-12


# ---------------------------------------------------------------------------
# kernel-aware pattern search: work and recall
# ---------------------------------------------------------------------------
def test_pattern_recall_brute_force_and_full_budgets():
    rng = np.random.default_rng(21)
    n, d = 150, 8
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    scale = 0.4
    plan = dict(kind="ashape", sink=5, local=20)
    rows = [0, 7, 63, 64, 100, 149]
    want = 0.0
    for i in rows:
        w = [math.exp(scale * sum(q[i, t] * k[j, t] for t in range(d))) for j in range(i + 1)]
        z = sum(w)
        want += sum(w[j] for j in range(i + 1) if j < 5 or i - j < 20) / z
    assert abs(O.pattern_recall(q, k, plan, scale, rows) - want / len(rows)) < 1e-12
    # every full budget keeps all of the attention
    assert abs(O.pattern_recall(q, k, dict(kind="dense"), scale) - 1.0) < 1e-12
    for cand in (dict(kind="vs", k_v=n, k_s=n), dict(kind="block", k_b=3), dict(kind="ashape", sink=0, local=n)):
        plan = O.candidate_plan(q, k, cand, scale, last_q=64)
        assert abs(O.pattern_recall(q, k, plan, scale) - 1.0) < 1e-12


def test_plan_blocks_counts_blocks_with_mask_entries():
    rng = np.random.default_rng(22)
    n = 700
    nb = (n + 63) // 64
    assert O.plan_blocks(dict(kind="dense"), n) == nb * (nb + 1) / 2
    for sink, local in ((0, 100), (70, 1), (64, 200), (10, 0)):
        want = 0
        for b in range(nb):
            rows = np.arange(64 * b, min(64 * b + 64, n))
            m = np.stack([O.ashape_mask_row(int(i), n, sink, local) for i in rows])
            want += len({j // 64 for j in np.nonzero(m.any(axis=0))[0]})
        assert O.plan_blocks(dict(kind="ashape", sink=sink, local=local), n) == want
    cnt = rng.integers(1, 4, nb)
    assert O.plan_blocks(dict(kind="block", blk_idx=None, blk_cnt=cnt), n) == cnt.sum()


def _vs_work_loops(n, s_idx, v_idx):
    """VS work from scalar loops over rows and offsets: for every query block, the
    key blocks that some row i of the block meets at i - dl (dl selected, i - dl >= 0),
    plus 1/64 for every selected column at or before the block's last row whose key
    block is not among them."""
    tot = 0.0
    for b in range((n + 63) // 64):
        last = min(64 * b + 63, n - 1)
        met = set()
        for i in range(64 * b, last + 1):
            for dl in s_idx:
                if i - int(dl) >= 0:
                    met.add((i - int(dl)) // 64)
        cols = 0
        for j in sorted(set(int(x) for x in v_idx)):
            if j <= last and j // 64 not in met:
                cols += 1
        tot += len(met) + cols / 64
    return tot


@pytest.mark.parametrize("n", [1, 63, 64, 65, 700, 640])
def test_plan_blocks_vs_brute_force(n):
    # the oracle's work count of a VS plan, against scalar loops that never form Bs(b) or Cv(b)
    rng = np.random.default_rng(n)
    cases = [(np.array([0, 130, 400]), np.array([5, 300, 699])), (np.array([]), np.array([0, 3])),
             (np.array([1]), np.array([])), (np.array([63, 64, 65]), np.array([62, 63, 64, 127, 128]))]
    for _ in range(3):
        cases.append((np.sort(rng.choice(n, size=min(n, 7), replace=False)),
                      np.sort(rng.choice(n, size=min(n, 9), replace=False))))
    for s_idx, v_idx in cases:
        s_in = s_idx[s_idx < n]
        v_in = v_idx[v_idx < n]
        got = O.plan_blocks(dict(kind="vs", s_idx=s_in, v_idx=v_in), n)
        assert got == _vs_work_loops(n, s_in, v_in), (n, s_in, v_in)


def test_plan_blocks_vs_closed_forms():
    # hand-derived counts, n = 700 (11 query blocks, the last one of 60 rows):
    #  * D = {0}: every block meets only its own diagonal block -> 11 blocks;
    #  * D = {128}: a multiple of 64 shifts every row by exactly two blocks, so
    #    blocks b >= 2 meet block b - 2 -> 9 blocks;
    #  * D = {1}: rows 64b + 1.. meet block b, row 64b meets block b - 1 (b >= 1)
    #    -> 11 + 10 = 21 blocks;
    #  * D = {0}, V = {5, 699}: column 5 lies in block 0, met by block 0 itself and
    #    gathered by blocks 1..10 (10 columns); column 699 is in the last block,
    #    which computes its own diagonal block -> 11 + 10/64.
    n = 700
    vs = lambda s, v: O.plan_blocks(dict(kind="vs", s_idx=np.array(s), v_idx=np.array(v)), n)  # noqa: E731
    assert vs([0], []) == 11
    assert vs([128], []) == 9
    assert vs([1], []) == 21
    assert vs([0], [5, 699]) == 11 + 10 / 64


def test_search_picks_best_recall_within_budget():
    rng = np.random.default_rng(23)
    n, d = 256, 8
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    cands = [dict(kind="ashape", sink=0, local=64), dict(kind="dense"), dict(kind="ashape", sink=64, local=64)]
    best, table = O.search_head_pattern(q, k, cands, 0.3, budget=1e9)
    assert best == 1 and abs(table[1][1] - 1.0) < 1e-12      # the dense plan keeps everything
    best, table = O.search_head_pattern(q, k, cands, 0.3, budget=table[1][0] - 1)
    assert best == 2                                          # sink + window beats the window alone
    assert table[2][1] > table[0][1] and table[2][0] > table[0][0]
    best, _ = O.search_head_pattern(q, k, cands, 0.3, budget=table[0][0])
    assert best == 0
    assert O.search_head_pattern(q, k, cands, 0.3, budget=0)[0] == -1


def test_pattern_heads_favour_their_patterns():
    from workload import pattern_heads
    n = 2048
    q, k, _ = pattern_heads(n)
    qn, kn = q.float().numpy(), k.float().numpy()
    cands = [dict(kind="ashape", sink=64, local=256), dict(kind="vs", k_v=128, k_s=4), dict(kind="vs", k_v=64, k_s=32),
             dict(kind="block", k_b=4), dict(kind="block", k_b=8)]
    rows = np.arange(0, n, 5)
    picks = [O.search_head_pattern(qn[h], kn[h], cands, 1 / math.sqrt(128), budget=400, rows=rows) for h in range(3)]
    assert cands[picks[0][0]]["kind"] == "vs"                 # vertical head
    assert picks[1][1][picks[1][0]][1] > 0.99                 # local head: almost every candidate keeps it
    assert cands[picks[2][0]]["kind"] == "block"              # block head


# ---------------------------------------------------------------------------
# grid pattern with permutation
# ---------------------------------------------------------------------------
def test_grid_permutation_is_patch_major():
    F, P = 5, 7
    src = O.grid_permutation(F, P)
    assert sorted(src.tolist()) == list(range(F * P))
    for p in range(P):
        for f in range(F):
            assert src[p * F + f] == f * P + p


def test_identity_permutation_reduces_to_block_sparse():
    rng = np.random.default_rng(31)
    n, d = 300, 8
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    sel, s = O.permuted_block_index(q, k, np.arange(n), 2)
    want, ws = O.block_index(q, k, 2)
    assert all(list(a) == list(b) for a, b in zip(sel, want))
    fin = np.isfinite(ws)
    assert np.array_equal(np.isfinite(s), fin) and np.allclose(s[fin], ws[fin], rtol=1e-12, atol=1e-12)


def test_permuted_eligibility_and_mask_brute_force():
    rng = np.random.default_rng(32)
    n, d = 200, 4
    src = rng.permutation(n)
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    sel, s = O.permuted_block_index(q, k, src, 2)
    nb = 4
    for b in range(nb):
        for c in range(nb):
            elig = any(src[j] <= src[i] for i in range(64 * b, min(64 * b + 64, n))
                       for j in range(64 * c, min(64 * c + 64, n)))
            assert elig == bool(np.isfinite(s[b, c]))
        assert len(sel[b]) == min(2, int(np.isfinite(s[b]).sum()))
    inv = np.empty(n, dtype=np.int64)
    inv[src] = np.arange(n)
    o, lse = O.permuted_block_attn(q, k, v, src, sel, 0.5, rows=[0, 57, 199])
    for t, i in enumerate([0, 57, 199]):
        keys = [j for j in range(i + 1) if inv[j] // 64 in set(sel[inv[i] // 64].tolist())]
        if not keys:
            assert np.all(o[t] == 0) and np.isneginf(lse[t])
            continue
        w = [math.exp(0.5 * float(q[i] @ k[j])) for j in keys]
        z = sum(w)
        want = sum(w[a] * v[keys[a]] for a in range(len(keys))) / z
        assert np.allclose(o[t], want, rtol=1e-12, atol=1e-12) and abs(lse[t] - math.log(z)) < 1e-12


def test_permuted_full_budget_is_dense_causal():
    rng = np.random.default_rng(33)
    n, d = 260, 8
    src = rng.permutation(n)
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    sel, _ = O.permuted_block_index(q, k, src, 10)
    o, lse = O.permuted_block_attn(q, k, v, src, sel, 0.3)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None], is_causal=True, scale=0.3)[0]
    assert np.abs(o - want.numpy()).max() < 1e-12


# ---------------------------------------------------------------------------
# VS with slash-aligned windows
# ---------------------------------------------------------------------------
def test_vs_window_contains_exact_slashes_and_lies_inside_block_reading():
    rng = np.random.default_rng(41)
    n = 640
    s_idx = np.sort(rng.choice(n, 9, replace=False))
    v_idx = np.sort(rng.choice(n, 7, replace=False))
    for b in range(n // 64):
        rows = np.arange(64 * b, 64 * b + 64)
        mw = O.vsw_mask_block(n, s_idx, v_idx, b, rows)
        mb = O.vs_mask_block(n, s_idx, v_idx, b, rows)
        assert not (mw & ~mb).any()          # inside the 64x64-block reading (full blocks)
        for t, i in enumerate(rows):
            for dl in s_idx:
                if i - dl >= 0:
                    assert mw[t, i - dl]       # every exact slash entry
            for c in v_idx:
                assert mw[t, c] == (c <= i)    # every vertical column up to the row


def test_vs_window_brute_force_and_full_budget():
    n = 150
    s_idx = np.array([0, 5, 70, 149])
    v_idx = np.array([3, 100])
    for b in range(3):
        want = set()
        for dl in s_idx:
            lo = 64 * b - dl
            if lo + 63 >= 0:
                want |= {j for j in range(lo, lo + 64) if 0 <= j < n}
        assert O.vs_window_set(n, s_idx, b).tolist() == sorted(want)
    # every offset selected: the windows cover every key up to the row
    full = np.arange(n)
    for b in range(3):
        rows = np.arange(64 * b, min(64 * b + 64, n))
        assert np.array_equal(O.vsw_mask_block(n, full, [], b, rows), np.arange(n)[None, :] <= rows[:, None])


def test_vertical_tiles_complete_the_slash_tiles():
    # the skip-column read: selected columns not held by the block's slash tiles, ascending,
    # 64 per tile; with the slash tiles they give exactly the key set of the block's mask
    rng = np.random.default_rng(43)
    n = 64 * 9 + 21
    s_idx = np.sort(rng.choice(n, 6, replace=False))
    v_idx = np.sort(rng.choice(n, 150, replace=False))
    for windows in (False, True):
        for b in range((n + 63) // 64):
            last = min(64 * b + 63, n - 1)
            tiles = O.vertical_tiles(n, s_idx, v_idx, b, windows)
            cols = [int(c) for t in tiles for c in t]
            assert all(1 <= len(t) <= 64 for t in tiles) and all(len(t) == 64 for t in tiles[:-1])
            assert cols == sorted(set(cols))
            if windows:
                held = set(O.vs_window_set(n, s_idx, b).tolist())
                mask = O.vsw_mask_block(n, s_idx, v_idx, b, [last])[0]
            else:
                held = {j for c in O.vs_block_set(n, s_idx, b).tolist() for j in range(64 * c, min(64 * c + 64, n))}
                mask = O.vs_mask_block(n, s_idx, v_idx, b, [last])[0]
            # brute force from the definitions: columns of V up to the last row, not held
            want = sorted({int(j) for j in v_idx if j <= last and int(j) not in held})
            assert cols == want
            # slash tiles and vertical tiles together: the mask's keys at the block's last row
            keys = {j for j in held if j <= last} | set(cols)
            assert keys == set(np.nonzero(mask)[0].tolist())


def test_vertical_tiles_are_dense_triangles():
    # against the block's rows, the visible columns of every row are a prefix of the tile:
    # columns before the block are seen by every row, the block's own columns form a staircase
    n = 64 * 4
    s_idx = np.array([0, 130])
    v_idx = np.array(list(range(0, 256, 3)))
    for b in range(4):
        rows = np.arange(64 * b, 64 * b + 64)
        for t in O.vertical_tiles(n, s_idx, v_idx, b, True):
            vis = t[None, :] <= rows[:, None]
            counts = vis.sum(axis=1)
            for r in range(64):
                assert vis[r, :counts[r]].all() and not vis[r, counts[r]:].any()
            assert np.all(np.diff(counts) >= 0)
            assert vis[:, t < 64 * b].all()

