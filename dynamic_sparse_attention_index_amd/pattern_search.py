"""Offline kernel-aware pattern search on the GPU.

MInference 1.0 article, "Method": each attention head's sparse pattern is
chosen offline by a kernel-aware search before the online index is built;
talk transcript ("KV-cache-centric methods"): offline per-head pattern search,
and attention recall as the share of the attention an index keeps.

For every candidate (A-shape with its sink and window, Vertical-Slash with its
budgets, Block-Sparse with its block budget, or dense) the library builds the
candidate's online index on the calibration input and runs the sparse
attention kernel with it; the kernel returns each row's log-sum-exp over the
mask, and with the dense kernel's LSE of the same row the recall of row i is
exp(LSE_mask(i) - LSE_dense(i)), the share of the row's causal softmax mass
inside the mask. A candidate's work is counted in the kernel's unit: key
blocks whose mask block has an entry, plus each gathered vertical column as
1/64 of a block, summed over query blocks. Each head takes the highest-recall
candidate whose work is within the budget (ties to the lower work, then to the
earlier candidate); -1 when none fits.

Every attention and index computation runs in the library's kernels; this
module only assembles plans and reduces per-row LSE pairs to one number per
head and candidate.
"""
from __future__ import annotations

import math

import torch

from . import minf

BLOCK = 64


def _offsets(dl, nb, rows_last, device):
    """Block offsets O of a VS plan for a query block with `rows_last` rows."""
    o = torch.zeros(nb + 1, dtype=torch.bool, device=device)
    o[(dl // BLOCK)[dl % BLOCK < rows_last]] = True
    o[(dl // BLOCK + 1)[dl % BLOCK > 0].clamp(max=nb)] = True
    return o[:nb]


def plan_blocks(plan: dict, n: int) -> float:
    """Work of one head's plan in computed 64x64 blocks (gathered columns count 1/64)."""
    nb = (n + BLOCK - 1) // BLOCK
    kind = plan["kind"]
    if kind == "dense":
        return nb * (nb + 1) / 2
    if kind == "block":
        return float(plan["blk_cnt"].long().sum())
    if kind == "ashape":
        b = torch.arange(nb)
        sb = (int(plan["sink"]) + BLOCK - 1) // BLOCK
        sink_n = torch.clamp(b + 1, max=sb)                       # c in [0, min(b, sb - 1)]
        local = int(plan["local"])
        if local <= 0:
            return float(sink_n.sum())
        reach = (local + 62) // BLOCK                             # c >= b - reach has a window entry
        wlo = torch.clamp(b - reach, min=0)
        win_n = b - wlo + 1
        overlap = torch.clamp(torch.minimum(b + 1, torch.full_like(b, sb)) - wlo, min=0)
        return float((sink_n + win_n - overlap).sum())
    # Vertical-Slash: |Bs(b)| + |Cv(b)| / 64 per query block
    dev = plan["s_idx"].device
    dl = plan["s_idx"].long()
    dl = dl[(dl >= 0) & (dl < n)]
    j = plan["v_idx"].long()
    j = j[(j >= 0) & (j < n)]
    cb = j // BLOCK
    last_rows = n - BLOCK * (nb - 1)

    def part(bq, off):
        nblk = torch.cumsum(off.long(), 0)[bq]
        cols = 0
        for chunk in torch.split(bq, 2048):
            rel = chunk[:, None] - cb[None, :]
            cols += int(((rel >= 0) & ~off[rel.clamp(min=0)]).sum())
        return float(nblk.sum()) + cols / BLOCK

    full = _offsets(dl, nb, BLOCK, dev)
    if last_rows == BLOCK:
        return part(torch.arange(nb, device=dev), full)
    tot = part(torch.arange(nb - 1, device=dev), full) if nb > 1 else 0.0
    return tot + part(torch.tensor([nb - 1], device=dev), _offsets(dl, nb, last_rows, dev))


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


def search_patterns(q, k, v, candidates, budget, scale=None, last_q=64, rows=None):
    """Per-head pattern choice on a calibration input (q [hq, n, d], k/v [hkv, n, d] bf16).

    budget: work limit in blocks, one number for every head or a sequence per head.
    rows: query rows whose recall is averaged (all rows by default).
    Returns dict(choice=list[hq], blocks=[hq, C] float64, recall=[hq, C] float64,
    plans=list of per-candidate plan lists).
    """
    hq, n, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = torch.arange(n, device=q.device) if rows is None else torch.as_tensor(rows, device=q.device).long()
    budgets = [float(budget)] * hq if not hasattr(budget, "__len__") else [float(x) for x in budget]
    _, lse_dense = minf.minf_dense_attn(q, k, v, scale=scale)
    ld = lse_dense[:, rows].double()
    blocks = torch.zeros((hq, len(candidates)), dtype=torch.float64)
    recall = torch.zeros((hq, len(candidates)), dtype=torch.float64)
    all_plans = []
    for c, cand in enumerate(candidates):
        plans = _candidate_plans(q, k, cand, scale, last_q)
        _, lse = minf.minf_sparse_attn(q, k, v, plans, scale=scale)
        ls = lse[:, rows].double()
        r = torch.where(torch.isneginf(ls), torch.zeros_like(ls), torch.exp(ls - ld)).mean(dim=1)
        recall[:, c] = r.cpu()
        for h in range(hq):
            blocks[h, c] = plan_blocks(plans[h], n)
        all_plans.append(plans)
    choice = []
    for h in range(hq):
        best = -1
        for c in range(len(candidates)):
            if blocks[h, c] > budgets[h]:
                continue
            if best < 0 or recall[h, c] > recall[h, best] or (recall[h, c] == recall[h, best]
                                                               and blocks[h, c] < blocks[h, best]):
                best = c
        choice.append(best)
    return dict(choice=choice, blocks=blocks, recall=recall, plans=all_plans)
