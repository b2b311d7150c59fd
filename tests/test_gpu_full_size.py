"""GPU parity at the full workload sizes, on sampled outputs the oracle computes row by row.

Each test runs the same library calls, with the same shapes, budgets and
launch configuration as the benchmark step: the index of every head built on
the device from the data, then one sparse attention launch over all heads.
The oracle then checks, for sampled heads, the index sets under the margin
rule and, for sampled query blocks of every head, the attention outputs
(max-abs 2e-2) and LSE (2e-3).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from parity import check_lse, check_topk, max_abs, to_np
from workload import CONFIGS, STRUCTURED_LATENT, config_kinds, planted_qkv

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)


def _run_layer(minf, name, latent=None):
    cfg = CONFIGS[name]
    n, hq, hkv = cfg["n"], cfg["hq"], cfg["hkv"]
    kinds = config_kinds(name)
    print(f"[case] {name}: n={n} hq={hq} hkv={hkv} kinds={kinds} latent={latent}", flush=True)
    q, k, v, info = planted_qkv(n, hq, hkv, seed=1000 + cfg["index"], device="cuda", latent=latent)
    vs_heads = [h for h in range(hq) if kinds[h] == "vs"]
    bs_heads = [h for h in range(hq) if kinds[h] == "block"]
    out = dict(cfg=cfg, kinds=kinds, q=q, k=k, v=v, vs_heads=vs_heads, bs_heads=bs_heads)
    if vs_heads:
        out["vi"], out["si"] = minf.minf_build_vs_index(q, k, vs_heads, last_q=cfg["last_q"], k_v=cfg["k_v"],
                                                        k_s=cfg["k_s"], scale=SCALE)
    if bs_heads:
        out["bi"], out["bc"] = minf.minf_build_block_index(q, k, bs_heads, k_b=cfg["k_b"])
    plans = []
    for h in range(hq):
        if kinds[h] == "vs":
            t = vs_heads.index(h)
            plans.append(dict(kind="vs", v_idx=out["vi"][t], s_idx=out["si"][t]))
        elif kinds[h] == "block":
            t = bs_heads.index(h)
            plans.append(dict(kind="block", blk_idx=out["bi"][t], blk_cnt=out["bc"][t]))
        else:
            plans.append(dict(kind="ashape", sink=cfg["sink"], local=cfg["local"]))
    o, lse = minf.minf_sparse_attn(q, k, v, plans, scale=SCALE)
    torch.cuda.synchronize()
    out.update(plans=plans, o=o, lse=lse)
    return out


def _np_plan(p):
    d = dict(kind=p["kind"])
    for key in ("sink", "local"):
        if key in p:
            d[key] = p[key]
    for key in ("v_idx", "s_idx", "blk_idx", "blk_cnt"):
        if key in p:
            d[key] = p[key].cpu().numpy().astype(np.int64)
    return d


def _check_attention(L, heads, blocks_per_head, seed):
    cfg = L["cfg"]
    n, hq, hkv = cfg["n"], cfg["hq"], cfg["hkv"]
    nb = (n + 63) // 64
    rng = np.random.default_rng(seed)
    kv_cache = {}
    worst = 0.0
    for h in heads:
        g = h // (hq // hkv)
        if g not in kv_cache:
            kv_cache.clear()
            kv_cache[g] = (to_np(L["k"][g]), to_np(L["v"][g]))
        kg, vg = kv_cache[g]
        blocks = sorted({0, nb - 1, *rng.choice(nb, size=blocks_per_head, replace=False).tolist()})
        rows = np.concatenate([np.arange(64 * b, min(64 * b + 64, n)) for b in blocks])
        qh = to_np(L["q"][h][torch.as_tensor(rows, device=L["q"].device)])
        # the oracle sees the full K/V and only the sampled query rows of head h
        qfull = np.zeros((1, n, 128), np.float32)
        qfull[0, rows] = qh
        wo, wl = O.sparse_attn(qfull, kg[None], vg[None], 1, 1, SCALE, [_np_plan(L["plans"][h])], rows=rows)
        got_o = to_np(L["o"][h][torch.as_tensor(rows, device=L["o"].device)])
        got_l = L["lse"][h][torch.as_tensor(rows, device=L["lse"].device)].cpu().numpy()
        err = max_abs(got_o, wo[0])
        worst = max(worst, err)
        assert err <= 2e-2, (h, blocks, err)
        check_lse(got_l, wl[0])
    print(f"  attention: {len(heads)} heads, worst max-abs {worst:.3e}", flush=True)


def _check_vs_index(L, sample_heads):
    cfg = L["cfg"]
    hq, hkv = cfg["hq"], cfg["hkv"]
    exact = 0
    for t in sample_heads:
        h = L["vs_heads"][t]
        g = h // (hq // hkv)
        _, _, wv, ws = O.vs_index(to_np(L["q"][h]), to_np(L["k"][g]), cfg["last_q"], cfg["k_v"], cfg["k_s"], SCALE)
        exact += check_topk(wv, L["vi"][t].cpu().numpy(), cfg["k_v"], abs_tol=1e-7)
        exact += check_topk(ws, L["si"][t].cpu().numpy(), cfg["k_s"], abs_tol=1e-7)
    print(f"  VS index: {len(sample_heads)} heads checked, {exact} of {2 * len(sample_heads)} lists unambiguous",
          flush=True)


def _check_bs_index(L, sample_heads):
    cfg = L["cfg"]
    hq, hkv = cfg["hq"], cfg["hkv"]
    exact = amb = 0
    for t in sample_heads:
        h = L["bs_heads"][t]
        g = h // (hq // hkv)
        qn, kn = to_np(L["q"][h]), to_np(L["k"][g])
        sel, s = O.block_index(qn, kn, cfg["k_b"])
        qbar, kbar = O.pool_blocks(qn), O.pool_blocks(kn)
        kabs = np.abs(kbar)
        bi = L["bi"][t].cpu().numpy()
        bc = L["bc"][t].cpu().numpy()
        for b in range(len(sel)):
            assert bc[b] == min(cfg["k_b"], b + 1)
            abs_tol = 1e-5 * float(np.abs(qbar[b]) @ kabs[: b + 1].max(axis=0))
            if check_topk(s[b, : b + 1], bi[b, : bc[b]], cfg["k_b"], abs_tol=abs_tol, want=sel[b]):
                exact += 1
            else:
                amb += 1
    print(f"  BS index: {len(sample_heads)} heads, rows exact {exact}, ambiguous {amb}", flush=True)


def test_c2_ashape_and_block_sparse_32k(gpu_lib):
    L = _run_layer(gpu_lib, "c2_ashape_bs_32k")
    _check_bs_index(L, [0, 1, 2, 3])
    _check_attention(L, list(range(8)), 4, seed=5)


def test_c3_gqa_mixed_128k(gpu_lib):
    L = _run_layer(gpu_lib, "c3_gqa_128k")
    _check_vs_index(L, [0, 7])
    _check_bs_index(L, [0])
    _check_attention(L, list(range(32)), 1, seed=6)


def test_c4_gqa_mixed_512k(gpu_lib):
    # 8 Block-Sparse heads at 8192 blocks: the pooled-score buffer is filled in several row bands
    L = _run_layer(gpu_lib, "c4_gqa_512k")
    _check_bs_index(L, [5])
    _check_vs_index(L, [11])
    _check_attention(L, list(range(0, 32, 5)), 1, seed=9)


def test_c5_gqa_all_vs_1m(gpu_lib):
    L = _run_layer(gpu_lib, "c5_gqa_1m_vs")
    _check_vs_index(L, [0])
    # every head: its first and last query blocks and one seeded block in between
    _check_attention(L, list(range(32)), 1, seed=7)


@pytest.mark.parametrize("name,heads", [("c3_gqa_128k", list(range(32))),
                                        ("c5_gqa_1m_vs", [0, 5, 10, 15, 16, 21, 26, 31])])
def test_vs_index_exact_at_planted_counts(gpu_lib, name, heads):
    """Budgets equal to the planted counts (k_v = 8 columns per KV group, k_s = 4 offsets),
    on the workload's own data and row length: the planted items stand far above the rest,
    so every list is unambiguous under the margin rule and must equal the oracle's exactly
    (MInference 1.0 article, "Method": the VS index from the last queries' attention)."""
    cfg = CONFIGS[name]
    n, hq, hkv = cfg["n"], cfg["hq"], cfg["hkv"]
    print(f"[case] {name}: exact VS index, k_v=8 k_s=4, heads {heads}", flush=True)
    q, k, _, info = planted_qkv(n, hq, hkv, seed=1000 + cfg["index"], device="cuda")
    vi, si = gpu_lib.minf_build_vs_index(q, k, heads, last_q=64, k_v=8, k_s=4, scale=SCALE)
    torch.cuda.synchronize()
    vi, si = vi.cpu().numpy(), si.cpu().numpy()
    planted_cols = planted_offs = 0
    for t, h in enumerate(heads):
        g = h // (hq // hkv)
        wvi, wsi, wv, ws = O.vs_index(to_np(q[h]), to_np(k[g]), 64, 8, 4, SCALE)
        assert check_topk(wv, vi[t], 8, abs_tol=1e-7, want=wvi), (h, "verticals ambiguous")
        assert check_topk(ws, si[t], 4, abs_tol=1e-7, want=wsi), (h, "slashes ambiguous")
        planted_cols += len(set(info.columns[g]) & set(vi[t].tolist()))
        planted_offs += len(set(info.offsets) & set(si[t].tolist()))
    print(f"  {len(heads)} heads exact; planted columns in the top 8: {planted_cols}/{8 * len(heads)}, "
          f"planted offsets in the top 4: {planted_offs}/{4 * len(heads)}", flush=True)


def test_c3_structured_latent_128k(gpu_lib):
    # locality-latent inputs: local slashes, so most query blocks compute few key blocks
    L = _run_layer(gpu_lib, "c3_gqa_128k", latent=STRUCTURED_LATENT)
    _check_vs_index(L, [3, 11])
    _check_bs_index(L, [2])
    _check_attention(L, list(range(0, 32, 3)), 2, seed=8)
