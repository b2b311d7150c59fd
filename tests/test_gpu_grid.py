"""Grid pattern with permutation through the C ABI against the CPU oracle.

Inputs: a grid-planted video (frames x patches, frame-major) and random
permutations. Bars: row permutation bitwise equal to indexing; the permuted
block index exact under the margin rule; outputs (scattered back to the
original order) within max-abs 2e-2 of the fp64 oracle on the GPU's selected
blocks, LSE within 2e-3; full budgets equal dense causal attention; the
identity permutation reproduces the plain Block-Sparse index.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from parity import check_lse, check_topk, max_abs, to_np
from workload import grid_qkv, planted_qkv

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)


def _permuted_layer(minf, q, k, v, src, k_b):
    """Permute, index, attend with positions, scatter back: (o, lse) in the original order + the index."""
    hq = q.shape[0]
    pos = torch.as_tensor(src, dtype=torch.int32, device=q.device)
    qp = minf.minf_permute_rows(q, pos)
    kp = minf.minf_permute_rows(k, pos)
    vp = minf.minf_permute_rows(v, pos)
    bi, bc = minf.minf_build_permuted_block_index(qp, kp, list(range(hq)), pos, k_b=k_b)
    plans = [dict(kind="block", blk_idx=bi[h], blk_cnt=bc[h], pos=pos) for h in range(hq)]
    op, lp = minf.minf_sparse_attn(qp, kp, vp, plans, scale=SCALE)
    o = minf.minf_permute_rows(op, pos, scatter=True)
    lse = minf.minf_permute_rows(lp.unsqueeze(-1).contiguous(), pos, scatter=True).squeeze(-1)
    torch.cuda.synchronize()
    return o, lse, bi, bc


def _check(q, k, v, src, o, lse, bi, bc, k_b, heads, rows_per_head, seed):
    hq, hkv = q.shape[0], k.shape[0]
    n = q.shape[1]
    rng = np.random.default_rng(seed)
    exact = amb = 0
    worst = 0.0
    for h in heads:
        g = h // (hq // hkv)
        qn, kn, vn = to_np(q[h]), to_np(k[g]), to_np(v[g])
        sel_o, s = O.permuted_block_index(qn, kn, src, k_b)
        qbar = O.pool_blocks(qn[src])
        kabs = np.abs(O.pool_blocks(kn[src]))
        bi_h, bc_h = bi[h].cpu().numpy(), bc[h].cpu().numpy()
        sel = []
        for b in range(len(sel_o)):
            ok = np.nonzero(np.isfinite(s[b]))[0]
            assert bc_h[b] == min(k_b, len(ok))
            got = bi_h[b, : bc_h[b]]
            assert np.all(bi_h[b, bc_h[b]:] == -1)
            assert set(got.tolist()) <= set(ok.tolist()), "an ineligible block was selected"
            abs_tol = 1e-5 * float(np.abs(qbar[b]) @ kabs.max(axis=0))
            # margin rule over the eligible blocks (positions into ok)
            got_pos = np.searchsorted(ok, got)
            want_pos = np.searchsorted(ok, sel_o[b])
            if check_topk(s[b, ok], got_pos, k_b, abs_tol=abs_tol, want=want_pos):
                exact += 1
            else:
                amb += 1
            sel.append(got)
        rows = np.sort(rng.choice(n, size=rows_per_head, replace=False))
        wo, wl = O.permuted_block_attn(qn, kn, vn, src, sel, SCALE, rows=rows)
        t = torch.as_tensor(rows, device=q.device)
        err = max_abs(to_np(o[h][t]), wo)
        worst = max(worst, err)
        assert err <= 2e-2, (h, err)
        check_lse(lse[h][t].cpu().numpy(), wl)
    print(f"  rows exact {exact}, ambiguous {amb}, worst max-abs {worst:.3e}", flush=True)


def test_permute_rows_roundtrip(gpu_lib):
    n = 1000
    x = torch.randn((3, n, 128), device="cuda").to(torch.bfloat16)
    src = torch.randperm(n, generator=torch.Generator().manual_seed(1)).to(torch.int32).cuda()
    g = gpu_lib.minf_permute_rows(x, src)
    assert torch.equal(g, x[:, src.long()])
    back = gpu_lib.minf_permute_rows(g, src, scatter=True)
    assert torch.equal(back, x)
    y = torch.randn((2, n), device="cuda")
    assert torch.equal(gpu_lib.minf_permute_rows(y.unsqueeze(-1).contiguous(), src).squeeze(-1), y[:, src.long()])


@pytest.mark.parametrize("frames,patches,k_b", [(64, 64, 2), (40, 50, 3), (120, 130, 6)])
def test_grid_layer_matches_oracle(gpu_lib, frames, patches, k_b):
    print(f"[case] grid F={frames} P={patches} k_b={k_b}", flush=True)
    q, k, v = grid_qkv(frames, patches, 4, 2, device="cuda")
    src = O.grid_permutation(frames, patches)
    o, lse, bi, bc = _permuted_layer(gpu_lib, q, k, v, src, k_b)
    _check(q, k, v, src, o, lse, bi, bc, k_b, heads=[0, 3], rows_per_head=48, seed=frames)


def test_grid_layer_several_score_bands(gpu_lib):
    # 1024 frames x 256 patches, 32 heads: 4096 blocks, and the index's score
    # buffer holds 1024 rows at a time (four bands); every row of two heads checked
    frames, patches, k_b = 1024, 256, 64
    print(f"[case] grid F={frames} P={patches} 32 heads k_b={k_b}", flush=True)
    q, k, v = grid_qkv(frames, patches, 32, 8, device="cuda")
    src = O.grid_permutation(frames, patches)
    o, lse, bi, bc = _permuted_layer(gpu_lib, q, k, v, src, k_b)
    _check(q, k, v, src, o, lse, bi, bc, k_b, heads=[0, 21], rows_per_head=16, seed=frames)


def test_random_permutation_and_full_budget(gpu_lib):
    n = 1500
    print(f"[case] random permutation n={n}", flush=True)
    q, k, v, _ = planted_qkv(n, 2, 1, seed=91, device="cuda")
    src = np.random.default_rng(5).permutation(n)
    o, lse, bi, bc = _permuted_layer(gpu_lib, q, k, v, src, 3)
    _check(q, k, v, src, o, lse, bi, bc, 3, heads=[0, 1], rows_per_head=40, seed=2)
    # every eligible block: causal attention in the original order
    of, lf, _, _ = _permuted_layer(gpu_lib, q, k, v, src, 64)
    od, ld = gpu_lib.minf_dense_attn(q, k, v, scale=SCALE)
    torch.cuda.synchronize()
    assert max_abs(to_np(of), to_np(od)) <= 2e-2
    assert float((lf - ld).abs().max()) <= 2e-3


def test_random_permutation_whole_and_partial_column_groups(gpu_lib):
    # 600 blocks (the last one ragged): columns 256..511 form a whole group, which
    # the index stores rotated, and 512..599 a partial one, which it stores in place
    n = 64 * 600 - 5
    print(f"[case] random permutation n={n}", flush=True)
    q, k, v, _ = planted_qkv(n, 4, 2, seed=93, device="cuda")
    src = np.random.default_rng(7).permutation(n)
    o, lse, bi, bc = _permuted_layer(gpu_lib, q, k, v, src, 24)
    _check(q, k, v, src, o, lse, bi, bc, 24, heads=[0, 3], rows_per_head=24, seed=3)


def test_identity_permutation_is_block_sparse(gpu_lib):
    n = 4096
    q, k, v, _ = planted_qkv(n, 4, 2, seed=92, device="cuda")
    pos = torch.arange(n, dtype=torch.int32, device="cuda")
    bi, bc = gpu_lib.minf_build_permuted_block_index(q, k, [0, 1, 2, 3], pos, k_b=8)
    bj, bd = gpu_lib.minf_build_block_index(q, k, [0, 1, 2, 3], k_b=8)
    plans_p = [dict(kind="block", blk_idx=bi[h], blk_cnt=bc[h], pos=pos) for h in range(4)]
    plans_b = [dict(kind="block", blk_idx=bj[h], blk_cnt=bd[h]) for h in range(4)]
    op, lp = gpu_lib.minf_sparse_attn(q, k, v, plans_p, scale=SCALE)
    ob, lb = gpu_lib.minf_sparse_attn(q, k, v, plans_b, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(bi, bj) and torch.equal(bc, bd)
    assert max_abs(to_np(op), to_np(ob)) <= 1e-2
    assert float((lp - lb).abs().max()) <= 1e-3
