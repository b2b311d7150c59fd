"""Offline kernel-aware pattern search on the GPU.

MInference 1.0 article, "Method": each attention head's sparse pattern is
chosen offline by a kernel-aware search before the online index is built;
talk transcript ("KV-cache-centric methods"): offline per-head pattern search,
and attention recall as the share of the attention an index keeps.

For every candidate (A-shape with its sink and window, Vertical-Slash with its
budgets, Block-Sparse with its block budget, or dense) the library builds the
candidate's online index on the calibration input, runs the sparse attention
kernel with it, and reduces the per-row log-sum-exp against the dense
kernel's to one recall per head (minf_attention_recall: the mean of
exp(LSE_mask - LSE_dense), the share of each row's causal softmax mass inside
the mask). The library also counts each plan's work in the kernel's unit
(minf_plan_work: key blocks computed, plus gathered vertical columns at 1/64
of a block, summed over query blocks). Each head takes the highest-recall
candidate whose work is within the budget (ties to the lower work, then to the
earlier candidate); -1 when none fits.

This module only assembles plans, passes arguments to the library and makes
that choice on the host from the numbers the library returns.
"""
from __future__ import annotations

import math

import torch

from . import minf


def _candidate_plans(q, k, cand: dict, scale: float, last_q: int):
    hq = q.shape[0]
    kind = cand["kind"]
    if kind == "dense":
        return [dict(kind="dense") for _ in range(hq)]
    if kind == "ashape":
        return [dict(kind="ashape", sink=int(cand["sink"]), local=int(cand["local"])) for _ in range(hq)]
    heads = list(range(hq))
    if kind == "vs":
        vi, si = minf.minf_build_vs_index(q, k, heads, last_q=last_q, k_v=int(cand["k_v"]), k_s=int(cand["k_s"]),
                                          scale=scale)
        return [dict(kind="vs", v_idx=vi[h], s_idx=si[h]) for h in heads]
    if kind == "block":
        bi, bc = minf.minf_build_block_index(q, k, heads, k_b=int(cand["k_b"]))
        return [dict(kind="block", blk_idx=bi[h], blk_cnt=bc[h]) for h in heads]
    raise ValueError(f"unknown candidate kind {kind!r}")


def choose(blocks, recall, budgets) -> list:
    """Per head, the candidate with the highest recall among those within the head's work
    budget, ties to the lower work and then the earlier candidate; -1 when none fits.
    blocks, recall: [hq][C] host numbers; budgets: one number per head."""
    out = []
    for h in range(len(budgets)):
        best = -1
        for c in range(len(blocks[h])):
            if blocks[h][c] > budgets[h]:
                continue
            if best < 0 or recall[h][c] > recall[h][best] or (recall[h][c] == recall[h][best]
                                                               and blocks[h][c] < blocks[h][best]):
                best = c
        out.append(best)
    return out


def search_patterns(q, k, v, candidates, budget, scale=None, last_q=64, rows=None):
    """Per-head pattern choice on a calibration input (q [hq, n, d], k/v [hkv, n, d] bf16).

    budget: work limit in blocks, one number for every head or a sequence per head.
    rows: query rows whose recall is averaged (all rows by default).
    Returns dict(choice=list[hq], blocks=[hq, C] float64, recall=[hq, C] float64 (host tensors),
    plans=list of per-candidate plan lists).
    """
    hq, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows_t = None if rows is None else torch.as_tensor(rows, device=q.device).to(torch.int32).contiguous()
    budgets = [float(budget)] * hq if not hasattr(budget, "__len__") else [float(x) for x in budget]
    _, lse_dense = minf.minf_dense_attn(q, k, v, scale=scale)
    blocks = torch.zeros((hq, len(candidates)), dtype=torch.float64)
    recall = torch.zeros((hq, len(candidates)), dtype=torch.float64)
    all_plans = []
    for c, cand in enumerate(candidates):
        plans = _candidate_plans(q, k, cand, scale, last_q)
        _, lse = minf.minf_sparse_attn(q, k, v, plans, scale=scale)
        recall[:, c] = minf.minf_attention_recall(lse, lse_dense, rows_t).cpu()
        blocks[:, c] = minf.minf_plan_work(plans, n).cpu()
        all_plans.append(plans)
    choice = choose(blocks.tolist(), recall.tolist(), budgets)
    return dict(choice=choice, blocks=blocks, recall=recall, plans=all_plans)
