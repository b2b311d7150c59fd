"""Host-side work accounting of the GPU pattern search against the oracle's
definition (CPU only: no kernel is launched)."""
import numpy as np
import pytest
import torch

import oracle as O
from dynamic_sparse_attention_index_amd import pattern_search as PS


@pytest.mark.parametrize("n", [37, 64, 700, 1300, 4096])
def test_plan_blocks_match_oracle(n):
    rng = np.random.default_rng(n)
    for sink, local in ((0, 100), (70, 1), (64, 200), (10, 0), (128, 4096), (65, 63), (65, 64), (65, 65)):
        plan = dict(kind="ashape", sink=sink, local=local)
        assert PS.plan_blocks(plan, n) == O.plan_blocks(plan, n)
    for _ in range(3):
        s_idx = np.sort(rng.choice(n, min(n, 7), replace=False))
        v_idx = np.sort(rng.choice(n, min(n, 30), replace=False))
        got = PS.plan_blocks(dict(kind="vs", s_idx=torch.tensor(s_idx), v_idx=torch.tensor(v_idx)), n)
        assert abs(got - O.plan_blocks(dict(kind="vs", s_idx=s_idx, v_idx=v_idx), n)) < 1e-9
    nb = (n + 63) // 64
    cnt = rng.integers(1, 4, nb)
    assert PS.plan_blocks(dict(kind="block", blk_cnt=torch.tensor(cnt)), n) == cnt.sum()
    assert PS.plan_blocks(dict(kind="dense"), n) == nb * (nb + 1) / 2
