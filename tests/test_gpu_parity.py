"""GPU path (through the C ABI) against the CPU oracle, element by element.

Sizes span several 64x64 tiles and a ragged tail; the oracle finishes each in
seconds. Bars: index sets exact under the margin rule (tests/parity.py);
bf16 attention outputs within max-abs 2e-2 of the fp64 oracle; LSE within
2e-3; repeated runs bitwise identical.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from parity import check_lse, check_topk, max_abs, to_np
from workload import injected_vs_index, planted_qkv

pytestmark = pytest.mark.gpu
OUT_TOL = 2e-2
SCALE = 1 / math.sqrt(128)


def _qkv(n, hq, hkv, seed, **kw):
    print(f"[case] n={n} hq={hq} hkv={hkv} seed={seed} {kw}", flush=True)
    return planted_qkv(n, hq, hkv, seed=seed, device="cuda", **kw)


def _np_plans(plans):
    out = []
    for p in plans:
        q = dict(kind=p["kind"])
        for key in ("sink", "local"):
            if key in p:
                q[key] = p[key]
        for key in ("v_idx", "s_idx", "blk_idx", "blk_cnt"):
            if key in p:
                q[key] = p[key].cpu().numpy().astype(np.int64)
        out.append(q)
    return out


def _attn_parity(minf, q, k, v, plans, rows=None, tol=OUT_TOL):
    hq = q.shape[0]
    o, lse = minf.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    torch.cuda.synchronize()
    want_o, want_l = O.sparse_attn(to_np(q), to_np(k), to_np(v), hq, k.shape[0], SCALE, _np_plans(plans), rows=rows)
    got_o = to_np(o) if rows is None else to_np(o)[:, rows]
    got_l = to_np(lse) if rows is None else to_np(lse)[:, rows]
    err = max_abs(got_o, want_o)
    print(f"  max-abs err {err:.3e}", flush=True)
    assert err <= tol
    check_lse(got_l, want_l)
    return o, lse


@pytest.mark.parametrize("n,hq,hkv", [(64, 1, 1), (200, 2, 1), (1000, 4, 2), (4160, 2, 2), (1, 1, 1), (65, 2, 2)])
def test_dense_causal(gpu_lib, n, hq, hkv):
    q, k, v, _ = _qkv(n, hq, hkv, 11)
    o, lse = gpu_lib.minf_dense_attn(q, k, v, scale=SCALE)
    torch.cuda.synchronize()
    wo, wl = O.dense_attn(to_np(q), to_np(k), to_np(v), hq, hkv, SCALE)
    assert max_abs(to_np(o), wo) <= OUT_TOL
    check_lse(to_np(lse), wl)


@pytest.mark.parametrize("n", [1 << 19, (1 << 19) + 37])
def test_dense_rounds_launch_matches_ordinary(gpu_lib, monkeypatch, n):
    # at 2^19+ tokens causal dense attention takes the XCD-round launch (counters in a
    # static per-GPU array); MINF_ATTN_ROUNDS=0 forces the ordinary launch
    hq, hkv = 4, 1
    q, k, v, _ = _qkv(n, hq, hkv, 51)
    monkeypatch.delenv("MINF_ATTN_ROUNDS", raising=False)
    o1, l1 = gpu_lib.minf_dense_attn(q, k, v, scale=SCALE)
    o3, l3 = gpu_lib.minf_dense_attn(q, k, v, scale=SCALE)  # a second call reuses the counters
    monkeypatch.setenv("MINF_ATTN_ROUNDS", "0")
    o2, l2 = gpu_lib.minf_dense_attn(q, k, v, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    rows = np.concatenate([np.arange(0, 64), np.arange(n // 2, n // 2 + 64), np.arange(64 * ((n - 1) // 64) - 64, n)])
    t = torch.as_tensor(rows, device="cuda")
    for h in (0, hq - 1):
        qh = np.zeros((1, n, 128), np.float32)
        qh[0, rows] = to_np(q[h][t])
        wo, wl = O.dense_attn(qh, to_np(k), to_np(v), 1, 1, SCALE, rows=rows)
        err = max_abs(to_np(o1[h][t]), wo[0])
        print(f"  dense rounds launch, head {h}: max-abs err {err:.3e}", flush=True)
        assert err <= OUT_TOL
        check_lse(to_np(l1[h][t]), wl[0])


@pytest.mark.parametrize("n", [200, 1000])
def test_dense_noncausal(gpu_lib, n):
    q, k, v, _ = _qkv(n, 2, 1, 12)
    o, lse = gpu_lib.minf_dense_attn(q, k, v, scale=SCALE, causal=False)
    torch.cuda.synchronize()
    wo, wl = O.dense_attn(to_np(q), to_np(k), to_np(v), 2, 1, SCALE, causal=False)
    assert max_abs(to_np(o), wo) <= OUT_TOL
    check_lse(to_np(lse), wl)


@pytest.mark.parametrize("n,sink,local", [(3000, 64, 1024), (1000, 10, 70), (777, 0, 100), (513, 130, 1), (300, 512, 64)])
def test_ashape(gpu_lib, n, sink, local):
    q, k, v, _ = _qkv(n, 2, 1, 13)
    plans = [dict(kind="ashape", sink=sink, local=local)] * 2
    _attn_parity(gpu_lib, q, k, v, plans)


def test_dense_plan_equals_dense_call(gpu_lib):
    q, k, v, _ = _qkv(1000, 2, 1, 14)
    o1, l1 = gpu_lib.minf_sparse_attn(q, k, v, [dict(kind="dense")] * 2, scale=SCALE)
    o2, l2 = gpu_lib.minf_dense_attn(q, k, v, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("n,k_b", [(2000, 5), (4096, 16), (1000, 100)])
def test_block_index_and_attention(gpu_lib, n, k_b):
    hq, hkv = 4, 2
    q, k, v, _ = _qkv(n, hq, hkv, 15)
    heads = [1, 2, 3]
    bi, bc = gpu_lib.minf_build_block_index(q, k, heads, k_b=k_b)
    torch.cuda.synchronize()
    wi, wc, scores = O.build_block_index(to_np(q), to_np(k), hq, hkv, heads, k_b)
    assert np.array_equal(bc.cpu().numpy(), wc)
    qn, kn = to_np(q), to_np(k)
    exact = amb = 0
    for t, h in enumerate(heads):
        qbar = O.pool_blocks(qn[h])
        kbar = O.pool_blocks(kn[h // 2])
        for b in range(wi.shape[1]):
            c = int(wc[t, b])
            row = scores[t][b, : b + 1]
            abs_tol = 1e-5 * float(np.abs(qbar[b]) @ np.abs(kbar[: b + 1]).max(axis=0))
            got = bi[t, b, :c].cpu().numpy()
            if check_topk(row, got, k_b, abs_tol=abs_tol, want=wi[t, b, :c]):
                exact += 1
            else:
                amb += 1
            assert (bi[t, b, c:].cpu().numpy() == -1).all()
    print(f"  block rows exact {exact}, ambiguous {amb}")
    # attention over the GPU-built index
    plans = [dict(kind="dense")] + [dict(kind="block", blk_idx=bi[t].contiguous(), blk_cnt=bc[t].contiguous())
                                    for t in range(3)]
    _attn_parity(gpu_lib, q, k, v, plans)


@pytest.mark.parametrize("n,k_b", [(64 * 300 + 17, 20), (64 * 129, 128)])
def test_block_index_multi_tile(gpu_lib, n, k_b):
    # several 128 x 128 score tiles with a ragged last block; every row checked
    print(f"[case] block index n={n} k_b={k_b}", flush=True)
    hq, hkv = 4, 2
    q, k, v, _ = _qkv(n, hq, hkv, 18)
    heads = [0, 3]
    bi, bc = gpu_lib.minf_build_block_index(q, k, heads, k_b=k_b)
    torch.cuda.synchronize()
    wi, wc, scores = O.build_block_index(to_np(q), to_np(k), hq, hkv, heads, k_b)
    assert np.array_equal(bc.cpu().numpy(), wc)
    qn, kn = to_np(q), to_np(k)
    exact = amb = 0
    for t, h in enumerate(heads):
        qbar = O.pool_blocks(qn[h])
        kabs = np.abs(O.pool_blocks(kn[h // 2]))
        bi_h = bi[t].cpu().numpy()
        for b in range(wi.shape[1]):
            c = int(wc[t, b])
            abs_tol = 1e-5 * float(np.abs(qbar[b]) @ kabs[: b + 1].max(axis=0))
            if check_topk(scores[t][b, : b + 1], bi_h[b, :c], k_b, abs_tol=abs_tol, want=wi[t, b, :c]):
                exact += 1
            else:
                amb += 1
            assert (bi_h[b, c:] == -1).all()
    print(f"  block rows exact {exact}, ambiguous {amb}")
    assert exact > amb


def test_block_pool(gpu_lib):
    n = 64 * 7 + 9
    q, k, v, _ = _qkv(n, 3, 3, 16)
    got = gpu_lib.minf_block_pool(q, [2, 0]).cpu().numpy()
    qn = to_np(q)
    for t, h in enumerate([2, 0]):
        want = O.pool_blocks(qn[h])
        assert np.max(np.abs(got[t] - want)) <= 1e-5 * max(1.0, np.abs(want).max())


@pytest.mark.parametrize("n,last_q", [(4096, 64), (1000, 64), (130, 64), (64, 64), (4096 + 37, 17), (40, 64)])
def test_vs_scores(gpu_lib, n, last_q):
    hq, hkv = 4, 2
    q, k, v, _ = _qkv(n, hq, hkv, 17)
    heads = [0, 1, 3]
    gv, gs = gpu_lib.minf_vs_scores(q, k, heads, last_q=last_q, scale=SCALE)
    torch.cuda.synchronize()
    _, _, wv, ws = O.build_vs_index(to_np(q), to_np(k), hq, hkv, heads, last_q, 1, 1, SCALE)
    r = min(last_q, n)
    for t in range(3):
        assert np.max(np.abs(gv[t].cpu().numpy() - wv[t])) <= 1e-6 + 1e-4 * wv[t].max()
        assert np.max(np.abs(gs[t].cpu().numpy() - ws[t])) <= 1e-6 + 1e-4 * ws[t].max()
        assert abs(float(gv[t].double().sum()) - r) < 1e-3 and abs(float(gs[t].double().sum()) - r) < 1e-3


@pytest.mark.parametrize("n,k_v,k_s", [(4096, 64, 64), (4096, 8, 4), (2000, 100, 30), (300, 500, 500), (4096, 0, 3)])
def test_vs_index(gpu_lib, n, k_v, k_s):
    q, k, v, info = _qkv(n, 2, 1, 18)
    heads = [0, 1]
    gvi, gsi = gpu_lib.minf_build_vs_index(q, k, heads, last_q=64, k_v=k_v, k_s=k_s, scale=SCALE)
    torch.cuda.synchronize()
    wvi, wsi, wv, ws = O.build_vs_index(to_np(q), to_np(k), 2, 1, heads, 64, k_v, k_s, SCALE)
    for t in range(2):
        ev = check_topk(wv[t], gvi[t].cpu().numpy(), k_v, abs_tol=1e-7, want=wvi[t])
        es = check_topk(ws[t], gsi[t].cpu().numpy(), k_s, abs_tol=1e-7, want=wsi[t])
        if (k_v, k_s) == (8, 4):
            # budgets equal to the planted counts: unambiguous, so the lists are the oracle's exactly
            assert ev and es, (t, ev, es)


@pytest.mark.parametrize("n,k_v", [(40000, 1000), (5000, 300)])
def test_vs_index_exact_ties_across_chunks(gpu_lib, n, k_v):
    """Duplicated key rows give exactly equal column sums on both sides (the same
    arithmetic per column); with k_v cutting through that group, the lower-index
    rule fixes the selection, which must equal the oracle's exactly even though the
    margin rule calls it ambiguous. The duplicated keys are spread over many top-k
    chunks and the waves inside them."""
    print(f"[case] exact ties n={n} k_v={k_v}", flush=True)
    g = torch.Generator().manual_seed(n)
    q = torch.randn((1, n, 128), generator=g)
    k = torch.randn((1, n, 128), generator=g)
    u = torch.randn(128, generator=g)
    u = u / u.norm()
    q[0, -64:] += 4.0 * u
    dup = torch.arange(3, n - 200, 7)            # about n / 7 keys, all the same row
    k[0, dup] = 8.0 * u + 0.1 * torch.randn(128, generator=g)
    q, k = q.to(torch.bfloat16).cuda(), k.to(torch.bfloat16).cuda()
    assert dup.numel() > k_v
    gvi, _ = gpu_lib.minf_build_vs_index(q, k, [0], last_q=64, k_v=k_v, k_s=64, scale=SCALE)
    torch.cuda.synchronize()
    wvi, _, wv, _ = O.vs_index(to_np(q[0]), to_np(k[0]), 64, k_v, 64, SCALE)
    # the duplicated columns carry the largest, exactly equal, sums
    assert np.all(wv[dup.numpy()] == wv[dup[0].item()])
    assert gvi[0].cpu().tolist() == wvi.tolist() == dup[:k_v].tolist()


def test_vs_index_c1_exact_and_planted(gpu_lib):
    # 1 head, N = 4096, last_q = 64, k_v = k_s = 64, calibrated plant (7, 14)
    q, k, v, info = _qkv(4096, 1, 1, 1000)
    gvi, gsi = gpu_lib.minf_build_vs_index(q, k, [0], last_q=64, k_v=64, k_s=64, scale=SCALE)
    torch.cuda.synchronize()
    wvi, wsi, wv, ws = O.build_vs_index(to_np(q), to_np(k), 1, 1, [0], 64, 64, 64, SCALE)
    assert check_topk(wv[0], gvi[0].cpu().numpy(), 64, want=wvi[0])  # unambiguous on this seed
    assert check_topk(ws[0], gsi[0].cpu().numpy(), 64, want=wsi[0])
    assert set(info.columns[0]) <= set(gvi[0].cpu().tolist())
    assert set(info.offsets) <= set(gsi[0].cpu().tolist())


@pytest.mark.parametrize("n,k_v,k_s", [(4096, 64, 64), (3000, 200, 100), (1000, 1000, 0), (777, 5, 777), (2500, 1500, 40),
                                       (2500, 2500, 40), (700, 500, 0)])
def test_vs_attention_gpu_index(gpu_lib, n, k_v, k_s):
    hq, hkv = 2, 1
    q, k, v, _ = _qkv(n, hq, hkv, 19)
    vi, si = gpu_lib.minf_build_vs_index(q, k, [0, 1], last_q=64, k_v=k_v, k_s=k_s, scale=SCALE)
    plans = [dict(kind="vs", v_idx=vi[t].contiguous(), s_idx=si[t].contiguous()) for t in range(2)]
    _attn_parity(gpu_lib, q, k, v, plans)


@pytest.mark.parametrize("n", [4096, 8192 + 100])
def test_vs_attention_injected_local(gpu_lib, n):
    # local slashes [0, k_s) and scattered verticals: the gather path at a high column count
    q, k, v, info = _qkv(n, 2, 2, 20)
    plans = []
    for h in range(2):
        vi, si = injected_vs_index(n, 600, 200 + 300 * h, info.columns[h], info.offsets, seed=21 + h)
        plans.append(dict(kind="vs", v_idx=vi.cuda(), s_idx=si.cuda()))
    _attn_parity(gpu_lib, q, k, v, plans)


def test_vs_empty_rows(gpu_lib):
    n = 300
    q, k, v, _ = _qkv(n, 2, 1, 22)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    plans = [dict(kind="vs", v_idx=e, s_idx=e),
             dict(kind="vs", v_idx=e, s_idx=torch.tensor([64], dtype=torch.int32, device="cuda"))]
    o, lse = _attn_parity(gpu_lib, q, k, v, plans)
    assert (o[0] == 0).all() and torch.isneginf(lse[0]).all()
    assert (o[1, :64] == 0).all() and torch.isneginf(lse[1, :64]).all()


def test_vs_and_block_sparse_bitmaps_word_edges(gpu_lib):
    # offsets and key blocks on the 32-bit word edges of the kernel's bitmaps, with long runs of
    # empty words between them (the cursors skip those runs), at a ragged length
    n = 64 * 3000 + 23
    nb = (n + 63) // 64
    q, k, v, _ = _qkv(n, 3, 1, 41)
    dev = "cuda"
    s0 = torch.tensor([64 * 31, 64 * 1023 + 1], dtype=torch.int32, device=dev)
    s1 = torch.tensor([0, 64 * 31, 64 * 63, 64 * 64 + 5, 64 * 1023, 64 * 2000 + 17, 64 * 2999], dtype=torch.int32,
                      device=dev)
    g = torch.Generator().manual_seed(42)
    vi = torch.randperm(n, generator=g)[:50].sort().values.to(torch.int32).to(dev)
    kb = 6
    rows_b = []
    for b in range(nb):
        cand = sorted({c for c in (31, 32, 1023, 1024, b - 1, b) if 0 <= c <= b})
        rows_b.append(cand + [-1] * (kb - len(cand)))
    bi = torch.tensor(rows_b, dtype=torch.int32, device=dev)
    bc = (bi >= 0).sum(dim=1).to(torch.int32)
    plans = [dict(kind="vs", v_idx=vi, s_idx=s0), dict(kind="vs", v_idx=vi, s_idx=s1),
             dict(kind="block", blk_idx=bi.contiguous(), blk_cnt=bc.contiguous())]
    rows = np.concatenate([np.arange(0, 130), np.arange(64 * 1023 - 40, 64 * 1025 + 40),
                           np.arange(64 * 2047, 64 * 2049), np.arange(n - 150, n)])
    _attn_parity(gpu_lib, q, k, v, plans, rows=rows)


@pytest.mark.parametrize("n", [200, 2048 + 64])
def test_full_budgets_match_dense(gpu_lib, n):
    q, k, v, _ = _qkv(n, 4, 2, 23)
    nb = (n + 63) // 64
    vi, si = gpu_lib.minf_build_vs_index(q, k, [0], last_q=64, k_v=n, k_s=n, scale=SCALE)
    bi, bc = gpu_lib.minf_build_block_index(q, k, [1], k_b=nb)
    plans = [dict(kind="vs", v_idx=vi[0].contiguous(), s_idx=si[0].contiguous()),
             dict(kind="block", blk_idx=bi[0].contiguous(), blk_cnt=bc[0].contiguous()),
             dict(kind="ashape", sink=0, local=n), dict(kind="ashape", sink=n, local=0)]
    o, lse = gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    torch.cuda.synchronize()
    wo, wl = O.dense_attn(to_np(q), to_np(k), to_np(v), 4, 2, SCALE)
    assert max_abs(to_np(o), wo) <= OUT_TOL
    check_lse(to_np(lse), wl)


def test_mixed_heads_gqa_and_determinism(gpu_lib):
    n, hq, hkv = 2048 + 77, 8, 2
    q, k, v, info = _qkv(n, hq, hkv, 24)
    vi, si = gpu_lib.minf_build_vs_index(q, k, [0, 3, 5], last_q=64, k_v=100, k_s=150, scale=SCALE)
    bi, bc = gpu_lib.minf_build_block_index(q, k, [1, 6], k_b=8)
    plans = [None] * hq
    for t, h in enumerate([0, 3, 5]):
        plans[h] = dict(kind="vs", v_idx=vi[t].contiguous(), s_idx=si[t].contiguous())
    for t, h in enumerate([1, 6]):
        plans[h] = dict(kind="block", blk_idx=bi[t].contiguous(), blk_cnt=bc[t].contiguous())
    plans[2] = dict(kind="ashape", sink=64, local=256)
    plans[4] = dict(kind="dense")
    plans[7] = dict(kind="ashape", sink=3, local=1000)
    o1, l1 = _attn_parity(gpu_lib, q, k, v, plans)
    o2, l2 = gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    vi2, si2 = gpu_lib.minf_build_vs_index(q, k, [0, 3, 5], last_q=64, k_v=100, k_s=150, scale=SCALE)
    bi2, bc2 = gpu_lib.minf_build_block_index(q, k, [1, 6], k_b=8)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(vi, vi2) and torch.equal(si, si2) and torch.equal(bi, bi2) and torch.equal(bc, bc2)


@pytest.mark.parametrize("n", [(1 << 17) + 37, 1 << 19, (1 << 19) + 37])
def test_rounds_launch_matches_ordinary(gpu_lib, monkeypatch, n):
    # 2^17 and 2^19 tokens (and ragged lengths), scattered slash offsets: long work items,
    # so the XCD-round launch takes the work; MINF_ATTN_ROUNDS=0 forces the ordinary launch
    hq = 4
    q, k, v, _ = _qkv(n, hq, 1, 25)
    g = torch.Generator().manual_seed(26)
    plans = []
    for h in range(hq):
        si = torch.randperm(n, generator=g)[:3000 + 500 * h].sort().values.to(torch.int32)
        vi = torch.randperm(n, generator=g)[:400].sort().values.to(torch.int32)
        plans.append(dict(kind="vs", v_idx=vi.cuda(), s_idx=si.cuda()))
    monkeypatch.delenv("MINF_ATTN_ROUNDS", raising=False)
    o1, l1 = gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    monkeypatch.setenv("MINF_ATTN_ROUNDS", "0")
    o2, l2 = gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # sampled rows of one head against the oracle: the first block, a middle one and the last
    rows = np.concatenate([np.arange(0, 64), np.arange(n // 2, n // 2 + 64), np.arange(64 * ((n - 1) // 64) - 64, n)])
    h = 2
    qh = np.zeros((1, n, 128), np.float32)
    qh[0, rows] = to_np(q[h][torch.as_tensor(rows, device="cuda")])
    wo, wl = O.sparse_attn(qh, to_np(k), to_np(v), 1, 1, SCALE, _np_plans([plans[h]]), rows=rows)
    t = torch.as_tensor(rows, device="cuda")
    err = max_abs(to_np(o1[h][t]), wo[0])
    print(f"  rounds launch: max-abs err {err:.3e}", flush=True)
    assert err <= OUT_TOL
    check_lse(l1[h][t].cpu().numpy(), wl[0])


def _random_block_plan(n, k_b, seed):
    # every query block b selects min(k_b, b + 1) random key blocks c <= b, ascending, padded with -1
    nb = (n + 63) // 64
    g = torch.Generator(device="cuda").manual_seed(seed)
    r = torch.rand(nb, nb, device="cuda", generator=g).tril() + torch.triu(torch.full((nb, nb), -1.0, device="cuda"), 1)
    top = r.topk(k_b, dim=1).indices.sort(dim=1).values
    cnt = torch.clamp(torch.arange(nb, device="cuda") + 1, max=k_b).to(torch.int32)
    ar = torch.arange(k_b, device="cuda")[None, :]
    bi = torch.where(ar < cnt[:, None], top, torch.full_like(top, -1)).to(torch.int32).contiguous()
    return dict(kind="block", blk_idx=bi, blk_cnt=cnt.contiguous())


def test_mixed_heads_rounds_partition_matches_ordinary(gpu_lib, monkeypatch):
    # VS heads between A-shape and Block-Sparse heads at 2^19 + 37 tokens: the VS heads
    # go to a launch of their own that takes the XCD-round launch, the others to an
    # ordinary launch; MINF_ATTN_ROUNDS=0 keeps every launch ordinary
    n, hq, hkv = (1 << 19) + 37, 8, 2
    q, k, v, _ = _qkv(n, hq, hkv, 41)
    g = torch.Generator().manual_seed(42)
    plans = []
    for h in range(hq):
        kind = ("ashape", "vs", "block", "vs", "vs", "ashape", "block", "vs")[h]
        if kind == "vs":
            si = torch.randperm(n, generator=g)[:4000 + 300 * h].sort().values.to(torch.int32)
            vi = torch.randperm(n, generator=g)[:300].sort().values.to(torch.int32)
            plans.append(dict(kind="vs", v_idx=vi.cuda(), s_idx=si.cuda()))
        elif kind == "block":
            plans.append(_random_block_plan(n, 16, 43 + h))
        else:
            plans.append(dict(kind="ashape", sink=100 + h, local=3000 + 7 * h))
    monkeypatch.delenv("MINF_ATTN_ROUNDS", raising=False)
    o1, l1 = gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    monkeypatch.setenv("MINF_ATTN_ROUNDS", "0")
    o2, l2 = gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # sampled rows of a VS, a Block-Sparse and an A-shape head against the oracle
    rows = np.concatenate([np.arange(0, 64), np.arange(n // 2, n // 2 + 64), np.arange(64 * ((n - 1) // 64) - 64, n)])
    t = torch.as_tensor(rows, device="cuda")
    for h in (1, 2, 5):
        kvh = h // (hq // hkv)
        qh = np.zeros((1, n, 128), np.float32)
        qh[0, rows] = to_np(q[h][t])
        p = plans[h]
        wo, wl = O.sparse_attn(qh, to_np(k[kvh:kvh + 1]), to_np(v[kvh:kvh + 1]), 1, 1, SCALE, _np_plans([p]), rows=rows)
        err = max_abs(to_np(o1[h][t]), wo[0])
        print(f"  head {h} ({p['kind']}): max-abs err {err:.3e}", flush=True)
        assert err <= OUT_TOL
        check_lse(l1[h][t].cpu().numpy(), wl[0])


# ---------------------------------------------------------------- VS with slash-aligned windows
def _window_plans(n, hq, seed, k_s, k_v, local=False, aligned=False):
    g = torch.Generator().manual_seed(seed)
    plans = []
    for h in range(hq):
        if local:
            si = torch.arange(min(k_s + h, n), dtype=torch.int32)
        else:
            si = torch.randperm(n, generator=g)[:min(k_s + 7 * h, n)].sort().values.to(torch.int32)
            if aligned:
                si = torch.unique(si // 64 * 64).to(torch.int32)
        vi = torch.randperm(n, generator=g)[:min(k_v, n)].sort().values.to(torch.int32)
        plans.append(dict(kind="vs_window", v_idx=vi.cuda(), s_idx=si.cuda()))
    return plans


@pytest.mark.parametrize("n", [64, 200, 1000, 4160, 4096 + 77])
def test_vs_window_attention(gpu_lib, n):
    # scattered offsets (windows at every alignment, overlapping and isolated) and verticals
    q, k, v, _ = _qkv(n, 4, 2, 26)
    _attn_parity(gpu_lib, q, k, v, _window_plans(n, 4, 27, k_s=40, k_v=30))


@pytest.mark.parametrize("n", [300, 2048 + 64])
def test_vs_window_local_and_edge_offsets(gpu_lib, n):
    # local offsets [0, k_s): one long interval per block; offsets past n and duplicates are ignored
    q, k, v, _ = _qkv(n, 4, 2, 28)
    plans = _window_plans(n, 4, 29, k_s=150, k_v=50, local=True)
    extra = torch.tensor([n, n + 5, -3, 0, 0, 1], dtype=torch.int32, device="cuda")
    gpu_plans = list(plans)
    gpu_plans[3] = dict(kind="vs_window", v_idx=plans[3]["v_idx"], s_idx=torch.cat([plans[3]["s_idx"], extra]))
    o, lse = gpu_lib.minf_sparse_attn(q, k, v, gpu_plans, scale=SCALE)
    torch.cuda.synchronize()
    # the library ignores offsets outside [0, n): the oracle sees the plan without them
    want_o, want_l = O.sparse_attn(to_np(q), to_np(k), to_np(v), 4, 2, SCALE, _np_plans(plans))
    err = max_abs(to_np(o), want_o)
    print(f"  max-abs err {err:.3e}", flush=True)
    assert err <= OUT_TOL
    check_lse(to_np(lse), want_l)


def test_vs_window_block_aligned_equals_block_reading(gpu_lib):
    # offsets that are multiples of 64 give windows equal to the grid blocks they cross
    n = 4096 + 64
    q, k, v, _ = _qkv(n, 4, 2, 30)
    pw = _window_plans(n, 4, 31, k_s=30, k_v=40, aligned=True)
    pb = [dict(kind="vs", v_idx=p["v_idx"], s_idx=p["s_idx"]) for p in pw]
    ow, lw = gpu_lib.minf_sparse_attn(q, k, v, pw, scale=SCALE)
    ob, lb = gpu_lib.minf_sparse_attn(q, k, v, pb, scale=SCALE)
    torch.cuda.synchronize()
    assert max_abs(to_np(ow), to_np(ob)) <= 1e-2
    empty = torch.isneginf(lb)  # rows with no key in either reading
    assert torch.equal(empty, torch.isneginf(lw))
    assert float((lw[~empty] - lb[~empty]).abs().max()) <= 1e-3


def test_vs_window_full_budget_and_empty(gpu_lib):
    n = 1000
    q, k, v, _ = _qkv(n, 2, 1, 32)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    full = torch.arange(n, dtype=torch.int32, device="cuda")
    plans = [dict(kind="vs_window", v_idx=e, s_idx=full), dict(kind="vs_window", v_idx=e, s_idx=e)]
    o, lse = gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    od, ld = gpu_lib.minf_dense_attn(q, k, v, scale=SCALE)
    torch.cuda.synchronize()
    assert max_abs(to_np(o[0]), to_np(od[0])) <= OUT_TOL
    assert float((lse[0] - ld[0]).abs().max()) <= 2e-3
    assert (o[1] == 0).all() and torch.isneginf(lse[1]).all()


def test_vs_window_large_sampled_rows(gpu_lib):
    # 2^19 tokens, scattered offsets: sampled rows against the oracle; mixed with block-reading heads
    n, hq = 1 << 19, 4
    q, k, v, _ = _qkv(n, hq, 1, 33)
    plans = _window_plans(n, hq, 34, k_s=2000, k_v=300)
    plans[1] = dict(kind="vs", v_idx=plans[1]["v_idx"], s_idx=plans[1]["s_idx"])
    o, lse = gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    torch.cuda.synchronize()
    rows = np.concatenate([np.arange(0, 64), np.arange(n // 2 + 64, n // 2 + 128), np.arange(n - 64, n)])
    t = torch.as_tensor(rows, device="cuda")
    for h in (0, 1):
        qh = np.zeros((1, n, 128), np.float32)
        qh[0, rows] = to_np(q[h][t])
        wo, wl = O.sparse_attn(qh, to_np(k), to_np(v), 1, 1, SCALE, _np_plans([plans[h]]), rows=rows)
        err = max_abs(to_np(o[h][t]), wo[0])
        print(f"  head {h} ({plans[h]['kind']}): max-abs err {err:.3e}", flush=True)
        assert err <= OUT_TOL
        check_lse(lse[h][t].cpu().numpy(), wl[0])
