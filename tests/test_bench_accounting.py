"""The benchmark's work accounting (computed tiles and kept entries) against the
oracle's explicit masks, on small cases with ragged lengths (CPU)."""
import numpy as np
import pytest
import torch

import bench
import oracle as O


def _blocks(n):
    nb = (n + 63) // 64
    return nb, [np.arange(64 * b, min(64 * b + 64, n)) for b in range(nb)]


@pytest.mark.parametrize("n", [37, 64, 700, 704, 1300])
def test_vs_useful_entries_match_oracle_mask(n):
    rng = np.random.default_rng(n)
    nb, rows = _blocks(n)
    for trial in range(4):
        s_idx = np.sort(rng.choice(n, min(n, 6), replace=False))
        v_idx = np.sort(rng.choice(n, min(n, 40), replace=False))
        if trial % 2:
            s_idx = s_idx[s_idx > 0]
        plan = dict(kind="vs", v_idx=torch.tensor(v_idx), s_idx=torch.tensor(s_idx))
        want = sum(int(O.vs_mask_block(n, s_idx, v_idx, b, rows[b]).sum()) for b in range(nb))
        assert bench.useful_entries(plan, n) == want


@pytest.mark.parametrize("n", [100, 704])
def test_vs_computed_blocks_match_oracle_block_sets(n):
    rng = np.random.default_rng(7)
    nb, _ = _blocks(n)
    s_idx = np.sort(rng.choice(n, 9, replace=False))
    v_idx = np.sort(rng.choice(n, 30, replace=False))
    blocks, cols = bench.vs_work(torch.tensor(v_idx), torch.tensor(s_idx), n)
    if n % 64 == 0:  # vs_work counts full query blocks
        assert blocks == sum(len(O.vs_block_set(n, s_idx, b)) for b in range(nb))
        assert cols == sum(len(O.vs_column_set(n, s_idx, v_idx, b)) for b in range(nb))


def test_block_and_ashape_useful_entries_match_oracle_masks():
    n = 1300
    rng = np.random.default_rng(3)
    nb, rows = _blocks(n)
    blk = np.full((nb, 4), -1)
    cnt = np.zeros(nb, int)
    for b in range(nb):
        c = np.sort(rng.choice(b + 1, min(4, b + 1), replace=False))
        blk[b, : len(c)] = c
        cnt[b] = len(c)
    plan = dict(kind="block", blk_idx=torch.tensor(blk), blk_cnt=torch.tensor(cnt))
    want = sum(int(O.bs_mask_block(n, blk[b, : cnt[b]], b, rows[b]).sum()) for b in range(nb))
    assert bench.useful_entries(plan, n) == want
    plan = dict(kind="ashape", sink=70, local=130)
    assert bench.useful_entries(plan, n) == sum(int(O.ashape_mask_row(i, n, 70, 130).sum()) for i in range(n))
    assert bench.useful_entries(dict(kind="dense"), n) == n * (n + 1) // 2
