"""Offline pattern search on the GPU against the oracle (planted heads).

Each candidate's work and recall on the GPU are checked against the oracle
evaluated on the same plan (the index the GPU built, which the index parity
tests already pin): work exactly, recall within 2e-3 (the recall comes from
the kernels' fp32 LSE of bf16 products). The per-head choice must equal the
oracle's wherever the oracle's best recall within the budget beats the
runner-up by more than 0.01.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from parity import to_np
from workload import pattern_heads, planted_qkv

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)
CANDS = [dict(kind="ashape", sink=64, local=256), dict(kind="vs", k_v=128, k_s=4), dict(kind="vs", k_v=64, k_s=32),
         dict(kind="block", k_b=4), dict(kind="block", k_b=8), dict(kind="dense")]


def _np_plan(p):
    out = dict(kind=p["kind"])
    for key in ("sink", "local"):
        if key in p:
            out[key] = p[key]
    for key in ("v_idx", "s_idx", "blk_idx", "blk_cnt"):
        if key in p:
            out[key] = p[key].cpu().numpy().astype(np.int64)
    return out


def _check(q, k, v, budget, rows):
    from dynamic_sparse_attention_index_amd import pattern_search as PS
    res = PS.search_patterns(q, k, v, CANDS, budget, scale=SCALE, rows=rows)
    torch.cuda.synchronize()
    hq, n = q.shape[0], q.shape[1]
    grp = hq // k.shape[0]
    rows_np = np.asarray(rows)
    for h in range(hq):
        qn, kn = to_np(q[h]), to_np(k[h // grp])
        table = []
        for c in range(len(CANDS)):
            plan = _np_plan(res["plans"][c][h])
            wb = O.plan_blocks(plan, n)
            wr = O.pattern_recall(qn, kn, plan, SCALE, rows_np)
            assert abs(float(res["blocks"][h, c]) - wb) < 1e-9, (h, c)
            assert abs(float(res["recall"][h, c]) - wr) <= 2e-3, (h, c, float(res["recall"][h, c]), wr)
            table.append((wb, wr))
        ok = [c for c in range(len(CANDS)) if table[c][0] <= budget]
        if not ok:
            assert res["choice"][h] == -1
            continue
        ranked = sorted(ok, key=lambda c: (-table[c][1], table[c][0], c))
        if len(ranked) == 1 or table[ranked[0]][1] - table[ranked[1]][1] > 0.01:
            assert res["choice"][h] == ranked[0], (h, table)
        print(f"  head {h}: choice {CANDS[res['choice'][h]]}", flush=True)
    return res


def test_pattern_search_planted_heads(gpu_lib):
    n = 2048
    print(f"[case] pattern heads n={n}", flush=True)
    q, k, v = (t.cuda() for t in pattern_heads(n))
    res = _check(q, k, v, budget=400, rows=np.arange(0, n, 5))
    assert CANDS[res["choice"][0]]["kind"] == "vs"
    assert CANDS[res["choice"][2]]["kind"] == "block"


def test_pattern_search_gqa_ragged(gpu_lib):
    n = 3000
    print(f"[case] pattern search GQA n={n}", flush=True)
    q, k, v, _ = planted_qkv(n, 4, 2, seed=77, device="cuda")
    _check(q, k, v, budget=600, rows=np.arange(0, n, 11))


def _np(t):
    return t.cpu().numpy().astype(np.int64)


@pytest.mark.parametrize("n", [37, 64, 700, 1300, 4096 + 17])
def test_plan_work_matches_oracle(gpu_lib, n):
    """minf_plan_work against the oracle's work count (exact: integer block and column counts)."""
    rng = np.random.default_rng(n)
    nb = (n + 63) // 64
    dev = "cuda"
    plans = [dict(kind="dense")]
    for sink, local in ((0, 100), (70, 1), (64, 200), (10, 0), (128, 4096), (65, 63), (65, 64), (65, 65)):
        plans.append(dict(kind="ashape", sink=sink, local=local))
    for ks, kv in ((7, 30), (0, 5), (3, 0), (n, n), (64, 64)):
        si = np.sort(rng.choice(n, min(n, ks), replace=False))
        vi = np.sort(rng.choice(n, min(n, kv), replace=False))
        plans.append(dict(kind="vs", s_idx=torch.tensor(si, dtype=torch.int32, device=dev),
                          v_idx=torch.tensor(vi, dtype=torch.int32, device=dev)))
    cnt = rng.integers(1, 5, nb)
    plans.append(dict(kind="block", blk_idx=torch.zeros((nb, 4), dtype=torch.int32, device=dev),
                      blk_cnt=torch.tensor(cnt, dtype=torch.int32, device=dev)))
    print(f"[case] plan work n={n}, {len(plans)} plans", flush=True)
    got = gpu_lib.minf_plan_work(plans, n).cpu().numpy()
    for h, p in enumerate(plans):
        want = O.plan_blocks(_np_plan(p), n)
        assert got[h] == want, (h, p["kind"], got[h], want)


def test_attention_recall_reduction(gpu_lib):
    """minf_attention_recall against the same reduction of the same LSE values in fp64 on the host."""
    rng = np.random.default_rng(5)
    hq, n = 3, 5000
    ld = rng.normal(5.0, 1.0, (hq, n)).astype(np.float32)
    lm = (ld - rng.exponential(0.5, (hq, n))).astype(np.float32)
    lm[1, ::7] = -np.inf
    lm[2, :] = -np.inf
    rows = rng.integers(0, n, 777).astype(np.int32)
    tm, td = torch.tensor(lm, device="cuda"), torch.tensor(ld, device="cuda")
    for r in (None, rows):
        got = gpu_lib.minf_attention_recall(tm, td, None if r is None else torch.tensor(r, device="cuda")).cpu().numpy()
        idx = np.arange(n) if r is None else r
        e = np.where(np.isneginf(lm[:, idx]), 0.0, np.exp(lm[:, idx].astype(np.float64) - ld[:, idx]))
        want = e.mean(axis=1)
        assert np.allclose(got, want, rtol=1e-12, atol=0), (got, want)
    assert got[2] == 0.0
