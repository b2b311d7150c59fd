"""Library calls captured into a HIP graph and replayed.

The library allocates nothing and never synchronises inside a call, so a
decode step or a whole prefill step (index builds + sparse attention) can be
captured on torch's stream and replayed. Each graph is replayed several times
with eager library work and synchronisations between the replays, and every
replay must reproduce the eager result bitwise.
"""
import math

import pytest
import torch

from workload import planted_qkv

pytestmark = pytest.mark.gpu
SCALE = 1 / math.sqrt(128)


def _replays(graph, outputs, want, eager_between):
    for r in range(3):
        # the program's own eager work between replays
        eager_between()
        torch.cuda.synchronize()
        for t in outputs:
            t.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip(outputs, want):
            assert torch.equal(got, ref), f"replay {r} differs from the eager result"


def test_decode_step_graph_replay(gpu_lib):
    # 2059 blocks: the segmented top-k path
    n, hq, hkv, k_b = 2048 * 64 + 700, 8, 2, 40
    print(f"[case] decode graph n={n} hq={hq} hkv={hkv} k_b={k_b}", flush=True)
    q, k, v, _ = planted_qkv(n, hq, hkv, seed=71, device="cuda")
    qd = q[:, -1].contiguous()
    kt = gpu_lib.minf_decode_pool_keys(k)
    nb = (n + 63) // 64
    o = torch.empty_like(qd)
    lse = torch.empty((hq,), dtype=torch.float32, device="cuda")
    blk = torch.empty((hq, k_b), dtype=torch.int32, device="cuda")
    ws = torch.empty(gpu_lib.library().minf_decode_workspace_size(n, hq, k_b), dtype=torch.uint8, device="cuda")

    def step():
        gpu_lib.minf_sparse_decode(qd, k, v, kt, k_b, scale=SCALE, out=o, lse=lse, blk_idx=blk, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = (o.clone(), lse.clone(), blk.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    q2 = q[:, -2].contiguous()
    _replays(g, (o, lse, blk), want,
             lambda: gpu_lib.minf_sparse_decode(q2, k, v, kt, nb, scale=SCALE))


def test_prefill_step_graph_replay(gpu_lib):
    # index builds of the VS and BS heads, then one sparse attention launch over mixed plans
    n, hq, hkv = 4096 + 77, 8, 2
    print(f"[case] prefill graph n={n} hq={hq} hkv={hkv}", flush=True)
    q, k, v, _ = planted_qkv(n, hq, hkv, seed=72, device="cuda")
    lib = gpu_lib.library()
    vs_heads, bs_heads = [0, 3, 5], [1, 6]
    nb = (n + 63) // 64
    vi = torch.empty((3, 100), dtype=torch.int32, device="cuda")
    si = torch.empty((3, 150), dtype=torch.int32, device="cuda")
    bi = torch.empty((2, nb, 8), dtype=torch.int32, device="cuda")
    bc = torch.empty((2, nb), dtype=torch.int32, device="cuda")
    ws_vs = torch.empty(lib.minf_vs_index_workspace_size(n, 3), dtype=torch.uint8, device="cuda")
    ws_bs = torch.empty(lib.minf_block_index_workspace_size(n, hq, hkv, 2), dtype=torch.uint8, device="cuda")
    ws_at = torch.empty(lib.minf_sparse_attn_workspace_size(n, hq), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")
    plans = [None] * hq
    for t, h in enumerate(vs_heads):
        plans[h] = dict(kind="vs", v_idx=vi[t], s_idx=si[t])
    for t, h in enumerate(bs_heads):
        plans[h] = dict(kind="block", blk_idx=bi[t], blk_cnt=bc[t])
    plans[2] = dict(kind="ashape", sink=64, local=256)
    plans[4] = dict(kind="dense")
    plans[7] = dict(kind="ashape", sink=3, local=1000)

    def step():
        gpu_lib.minf_build_vs_index(q, k, vs_heads, last_q=64, k_v=100, k_s=150, scale=SCALE, out=(vi, si),
                                    workspace=ws_vs)
        gpu_lib.minf_build_block_index(q, k, bs_heads, k_b=8, out=(bi, bc), workspace=ws_bs)
        gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE, out=o, lse=lse, workspace=ws_at)

    step()
    torch.cuda.synchronize()
    want = (vi.clone(), si.clone(), bi.clone(), bc.clone(), o.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    q2 = (q.float() * 0.5).to(torch.bfloat16)
    _replays(g, (vi, si, bi, bc, o, lse), want,
             lambda: gpu_lib.minf_sparse_attn(q2, k, v, [dict(kind="dense")] * hq, scale=SCALE))


def test_long_vs_launch_graph_replay(gpu_lib, monkeypatch):
    # 2^19 tokens with VS heads: eagerly the XCD-round launch may run; under capture the
    # library keeps the ordinary launch, so the reference is the eager ordinary launch
    # (MINF_ATTN_ROUNDS=0), which every replay must equal bitwise
    monkeypatch.setenv("MINF_ATTN_ROUNDS", "0")
    n, hq = 1 << 19, 2
    print(f"[case] long VS graph n={n} hq={hq}", flush=True)
    q, k, v, _ = planted_qkv(n, hq, 1, seed=73, device="cuda")
    g_ = torch.Generator().manual_seed(74)
    plans = []
    for _ in range(hq):
        si = torch.randperm(n, generator=g_)[:3000].sort().values.to(torch.int32).cuda()
        vi = torch.randperm(n, generator=g_)[:200].sort().values.to(torch.int32).cuda()
        plans.append(dict(kind="vs", v_idx=vi, s_idx=si))
    lib = gpu_lib.library()
    ws = torch.empty(lib.minf_sparse_attn_workspace_size(n, hq), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device="cuda")

    def step():
        gpu_lib.minf_sparse_attn(q, k, v, plans, scale=SCALE, out=o, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = (o.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    _replays(g, (o, lse), want, lambda: None)
