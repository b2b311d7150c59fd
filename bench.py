"""Benchmark: one sparse-prefill attention layer (index build + sparse attention).

Default workload: the 32-query-head / 8-KV-head GQA layer at N = 1,048,576
tokens, every head Vertical-Slash (1000 verticals, 6096 slashes, last 64
queries), bf16 inputs seeded and planted (see workload/gen.py). A step is the
whole hot path for the layer: the VS index of all 32 heads built from the
data, then sparse attention over it. Inputs are resident in HBM before timing.

Printed (one JSON line): latency per layer, the attention kernel's achieved
MFMA TFLOP/s over the blocks and columns it computes against the bf16 peak,
the in-house dense causal FlashAttention on the same inputs (speedup), two
more tracks of the same layer (an index-injected one with the pages'
local-slash structure, and a structured one on locality-latent data with the
index built from the data), and the CPU oracle timed on a bounded sample of
the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
BLOCK_FLOP = 4 * 64 * 64 * 128   # QK^T and PV of one 64x64 block, d = 128
COL_FLOP = 4 * 64 * 128          # one gathered key column for a 64-row query block
METRIC = "sparse prefill attn latency/layer at 128K–1M tok; MFMA util; speedup vs dense"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c5_gqa_1m_vs")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-injected", action="store_true")
    ap.add_argument("--no-structured", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-grid", action="store_true")
    ap.add_argument("--no-window", action="store_true", help="skip the VS slash-aligned window leg")
    ap.add_argument("--grid-blocks", type=int, default=64, help="block budget of the grid track")
    ap.add_argument("--search", action="store_true", help="also time the offline pattern search on the input")
    ap.add_argument("--decode-blocks", type=int, default=64,
                    help="decode budget in 64-token blocks (64 blocks = 4096 tokens)")
    ap.add_argument("--dense-runs", type=int, default=3, help="timed dense runs (after one untimed warm-up)")
    ap.add_argument("--layers", default="c3_gqa_128k,c4_gqa_512k",
                    help="further mixed-pattern layers measured after the headline ('' for none)")
    ap.add_argument("--layer-steps", type=int, default=3, help="timed steps of each further layer")
    ap.add_argument("--only-index", action="store_true",
                    help="time only the index build of the workload (for counter runs of the index kernels)")
    ap.add_argument("--only-dense", action="store_true",
                    help="time only the dense attention of the workload (for counter runs of the attention kernel)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------- work accounting
def vs_work(v_idx, s_idx, n):
    """(computed 64x64 blocks, gathered columns) of one VS head, summed over query blocks."""
    import torch
    nb = (n + 63) // 64
    dev = v_idx.device
    dl = s_idx.long()
    off = torch.zeros(nb + 1, dtype=torch.bool, device=dev)
    q = dl // 64
    off[q] = True
    rho = dl % 64
    off[(q + 1)[rho > 0].clamp(max=nb)] = True
    off = off[:nb]
    blocks = int(torch.cumsum(off.long(), 0).sum())  # sum over b of |{o in O : o <= b}|
    cb = (v_idx.long() // 64)
    cols = 0
    bs = torch.arange(nb, device=dev)
    for part in torch.split(bs, 2048):
        rel = part[:, None] - cb[None, :]
        ok = rel >= 0
        hit = off[rel.clamp(min=0)]
        cols += int((ok & ~hit).sum())
    return blocks, cols


def vsw_work(v_idx, s_idx, n):
    """(computed 64-key window tiles, gathered columns) of one VS window head, summed over query blocks.

    The tiles restate the library's cover of U = union over offsets dl of [-dl, -dl + 64): each
    maximal interval of U cut into 64-key tiles from its start; query block b computes the tiles
    with 64 b + end > 0. Column j lies in block b's windows iff b = floor((dl + j) / 64) for an
    offset dl, so it is gathered for every other block b >= floor(j / 64).
    """
    import torch
    nb = (n + 63) // 64
    dev = s_idx.device
    d = s_idx.long()
    d = torch.unique(d[(d >= 0) & (d < n)])                   # ascending
    if d.numel() == 0:
        tiles = 0
        dset_blocks = None
    else:
        starts = torch.flip(-d, [0])                           # window starts, ascending
        brk = torch.ones_like(starts, dtype=torch.bool)
        brk[1:] = (starts[1:] - starts[:-1]) > 64
        iv_start = starts[brk]
        last_idx = torch.cat([torch.nonzero(brk).flatten()[1:] - 1,
                              torch.tensor([starts.numel() - 1], device=dev)])
        iv_end = starts[last_idx] + 64
        ntile = (iv_end - iv_start + 63) // 64
        first = torch.repeat_interleave(iv_start, ntile)
        off = torch.arange(int(ntile.sum()), device=dev) - torch.repeat_interleave(torch.cumsum(ntile, 0) - ntile, ntile)
        t_start = first + 64 * off
        t_end = torch.minimum(t_start + 64, torch.repeat_interleave(iv_end, ntile))
        bs = torch.arange(nb, device=dev)
        tiles = int((t_end.numel() - torch.searchsorted(t_end, -64 * bs, right=True)).sum())
    cols = 0
    j = v_idx.long()
    j = j[(j >= 0) & (j < n)]
    for part in torch.split(j, 256):
        base = part // 64
        own = nb - base
        if d.numel():
            m = (d[None, :] + part[:, None]) // 64                # covering blocks, non-decreasing per row
            valid = m < nb
            distinct = valid[:, 0].long() + ((m[:, 1:] != m[:, :-1]) & valid[:, 1:]).sum(dim=1)
            own = own - distinct
        cols += int(own.sum())
    return tiles, cols


def useful_entries(plan, n):
    """Attention entries the head's mask keeps (the exact set, not the computed tiles)."""
    import torch
    nb = (n + 63) // 64
    kind = plan["kind"]
    if kind == "dense":
        return n * (n + 1) // 2
    if kind == "ashape":
        i = torch.arange(n, dtype=torch.int64)
        win = torch.clamp(i + 1, max=plan["local"]) if plan["local"] > 0 else torch.zeros_like(i)
        sink_only = torch.clamp(torch.clamp(i + 1 - win, min=0), max=plan["sink"])
        return int((win + sink_only).sum())
    rows_b = lambda b: torch.clamp(n - 64 * b, max=64)  # noqa: E731  rows of query block b
    if kind == "block":
        bi = plan["blk_idx"].long()
        cnt = plan["blk_cnt"].long()
        bq = torch.arange(bi.shape[0], device=bi.device)
        valid = torch.arange(bi.shape[1], device=bi.device)[None, :] < cnt[:, None]
        rb = rows_b(bq)
        diag = ((bi == bq[:, None]) & valid).sum(1)
        return int((rb * 64 * (cnt - diag) + diag * rb * (rb + 1) // 2).sum())
    # VS: full blocks below the diagonal, the causal part of the diagonal block, and per gathered
    # column the rows of its query block at or below it. Block b uses key blocks b - o for o in O;
    # a partial last block of R rows uses its own offset set (offset q + 1 when dl % 64 > 0, offset
    # q only when dl % 64 < R).
    dev = plan["v_idx"].device
    dl = plan["s_idx"].long()
    dl = dl[(dl >= 0) & (dl < n)]
    j = plan["v_idx"].long()
    j = j[(j >= 0) & (j < n)]

    def offsets(r_rows):
        o = torch.zeros(nb + 1, dtype=torch.bool, device=dev)
        o[(dl // 64)[dl % 64 < r_rows]] = True
        o[(dl // 64 + 1)[dl % 64 > 0].clamp(max=nb)] = True
        return o[:nb]

    def block_entries(bq, off):
        rb = rows_b(bq)
        nblk = torch.cumsum(off.long(), 0)[bq]  # |{o in O : o <= b}|
        has_diag = bool(off[0])
        ent = int((rb * 64 * (nblk - int(has_diag))).sum()) + (int((rb * (rb + 1) // 2).sum()) if has_diag else 0)
        cb = j // 64
        for part in torch.split(bq, 2048):
            rel = part[:, None] - cb[None, :]
            keep = (rel >= 0) & ~off[rel.clamp(min=0)]
            rpart = rows_b(part)[:, None]
            rows = torch.where(rel == 0, 64 * part[:, None] + rpart - j[None, :], rpart.expand_as(rel))
            ent += int((rows * keep).sum())
        return ent

    last_rows = n - 64 * (nb - 1)
    if last_rows == 64:
        return block_entries(torch.arange(nb, device=dev), offsets(64))
    ent = block_entries(torch.arange(nb - 1, device=dev), offsets(64)) if nb > 1 else 0
    return ent + block_entries(torch.tensor([nb - 1], device=dev), offsets(last_rows))


def ashape_blocks(n, sink, local):
    nb = (n + 63) // 64
    sb = min((sink + 63) // 64, nb)
    tot = 0
    for b in range(nb):
        lo = max(0, (64 * b - local + 1) // 64) if local > 0 else b + 1
        tot += len(set(range(min(sb, b + 1))) | set(range(lo, b + 1)))
    return tot


# ---------------------------------------------------------------- HBM traffic from the committed profile
def profiled_traffic(workload):
    """Calibrated HBM bytes per attention launch from profiles/, if measured on this kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"attn_kernel_{workload}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line:
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    csrc = os.path.join(ROOT, "dynamic_sparse_attention_index_amd", "csrc")
    sha = hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in ("attn.hip", "tile.h", "common.h")))
    if kv.get("source_sha256") != sha.hexdigest():
        return None
    return int(float(kv["fetch_bytes_per_launch"])) + int(float(kv["write_bytes_per_launch"]))


# ---------------------------------------------------------------- CPU oracle sample
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(q, k, v, kinds, cfg, plans_gpu, n):
    """Time the fp64 oracle: the index build of every head in full, and the sparse attention
    of a sample of query blocks of one head, extrapolated to the layer."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    scale = 1 / math.sqrt(128)
    grp = cfg["hq"] // cfg["hkv"]
    # index build, every head at full length (the VS estimate reads the last queries and all keys)
    t_index = 0.0
    n_vs = n_bs = 0
    for g in range(cfg["hkv"]):
        kg = None
        for h in range(g * grp, (g + 1) * grp):
            if kinds[h] not in ("vs", "block"):
                continue
            if kg is None:
                kg = k[g].float().cpu().numpy()
            qh = q[h].float().cpu().numpy()
            t1 = time.perf_counter()
            if kinds[h] == "vs":
                O.vs_index(qh, kg, cfg["last_q"], cfg["k_v"], cfg["k_s"], scale)
                n_vs += 1
            else:
                O.block_index(qh, kg, cfg["k_b"])
                n_bs += 1
            t_index += time.perf_counter() - t1
        del kg
    # attention: first, last and 14 seeded query blocks of one head, scaled to every block of every head
    h = kinds.index("vs") if "vs" in kinds else 0
    g = h // grp
    qh = q[h].float().cpu().numpy()
    kg = k[g].float().cpu().numpy()
    vg = v[g].float().cpu().numpy()
    nb = (n + 63) // 64
    rng = np.random.default_rng(0)
    mid = rng.choice(np.arange(1, nb - 1), size=min(14, max(nb - 2, 0)), replace=False).tolist()
    sample_blocks = sorted({0, nb - 1, *mid})
    p = plans_gpu[h]
    plan = {key: (val.cpu().numpy() if hasattr(val, "cpu") else val) for key, val in p.items()}
    t0 = time.perf_counter()
    for b in sample_blocks:
        rows = np.arange(64 * b, min(64 * b + 64, n))
        O.sparse_attn(qh[None], kg[None], vg[None], 1, 1, scale, [plan], rows=rows)
    t_attn = time.perf_counter() - t0
    attn_layer_s = (t_attn / len(sample_blocks)) * nb * len(kinds)
    return {
        "value": (t_index + attn_layer_s) * 1e3,
        "unit": "ms/layer (index timed in full, attention extrapolated)",
        "cores": int(cores),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "index_s": round(t_index, 2),
        "attention_extrapolated_s": round(attn_layer_s, 1),
        "sample": (f"fp64 NumPy oracle on {cores} threads: the index of all {n_vs} VS and {n_bs} BS heads at "
                   f"N={n} timed in full ({t_index:.1f} s), and sparse attention of {len(sample_blocks)} query "
                   f"blocks of head {h} ({t_attn:.1f} s) scaled to {nb} query blocks x {len(kinds)} heads"),
        "sample_seconds": round(t_index + t_attn, 2),
    }


def plans_for(kinds, cfg, vs_heads, bs_heads, vi, si, bi, bc):
    plans = []
    for h, kd in enumerate(kinds):
        if kd == "vs":
            t = vs_heads.index(h)
            plans.append(dict(kind="vs", v_idx=vi[t], s_idx=si[t]))
        elif kd == "block":
            t = bs_heads.index(h)
            plans.append(dict(kind="block", blk_idx=bi[t], blk_cnt=bc[t]))
        else:
            plans.append(dict(kind="ashape", sink=cfg["sink"], local=cfg["local"]))
    return plans


def layer_work(plans, n, cfg):
    """(blocks, columns, density per kind) of a layer's plans."""
    nb = (n + 63) // 64
    a_blocks = None
    blocks = cols = 0
    per_kind = {}
    for p in plans:
        if p["kind"] == "vs":
            b_, c_ = vs_work(p["v_idx"], p["s_idx"], n)
        elif p["kind"] == "block":
            b_, c_ = int(p["blk_cnt"].long().sum()), 0
        else:
            if a_blocks is None:
                a_blocks = ashape_blocks(n, cfg["sink"], cfg["local"])
            b_, c_ = a_blocks, 0
        blocks += b_
        cols += c_
        pk = per_kind.setdefault(p["kind"], [0, 0, 0])
        pk[0] += b_
        pk[1] += c_
        pk[2] += 1
    dens = {kd: round((bk + cl / 64) / (cnt * nb * (nb + 1) / 2), 4) for kd, (bk, cl, cnt) in per_kind.items()}
    return blocks, cols, dens


def layer_leg(name, steps, dense_runs, no_dense):
    """One further layer of the pages' length range: the whole step (index of every VS and BS head
    from the data, one sparse attention launch) timed over `steps` after a warm-up, its work, and
    the dense kernel on the same inputs (one warm-up, then `dense_runs` timed runs)."""
    import torch

    from dynamic_sparse_attention_index_amd import minf
    from workload import CONFIGS, config_kinds, planted_qkv
    cfg = CONFIGS[name]
    n, hq, hkv = cfg["n"], cfg["hq"], cfg["hkv"]
    kinds = config_kinds(name)
    scale = 1 / math.sqrt(128)
    q, k, v, _ = planted_qkv(n, hq, hkv, seed=1000 + cfg["index"], device="cuda")
    dev = q.device
    vs_heads = [h for h in range(hq) if kinds[h] == "vs"]
    bs_heads = [h for h in range(hq) if kinds[h] == "block"]
    lib = minf.library()
    ws_vs = torch.empty(max(1, lib.minf_vs_index_workspace_size(n, len(vs_heads))), dtype=torch.uint8, device=dev)
    ws_bs = torch.empty(max(1, lib.minf_block_index_workspace_size(n, hq, hkv, len(bs_heads))), dtype=torch.uint8,
                        device=dev)
    ws_at = torch.empty(max(1, lib.minf_sparse_attn_workspace_size(n, hq)), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    st = {}

    def step(record=None):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        st["vi"] = st["si"] = st["bi"] = st["bc"] = None
        if vs_heads:
            st["vi"], st["si"] = minf.minf_build_vs_index(q, k, vs_heads, last_q=cfg["last_q"], k_v=cfg["k_v"],
                                                          k_s=cfg["k_s"], scale=scale, workspace=ws_vs)
        if bs_heads:
            st["bi"], st["bc"] = minf.minf_build_block_index(q, k, bs_heads, k_b=cfg["k_b"], workspace=ws_bs)
        e[1].record(stream)
        plans = plans_for(kinds, cfg, vs_heads, bs_heads, st["vi"], st["si"], st["bi"], st["bc"])
        minf.minf_sparse_attn(q, k, v, minf.make_plans(plans, n=n, device=dev), scale=scale, out=o, lse=lse,
                              workspace=ws_at)
        e[2].record(stream)
        if record is not None:
            record.append(e)
        return plans

    step()
    torch.cuda.synchronize()
    recs = []
    for _ in range(max(1, steps)):
        plans = step(recs)
    torch.cuda.synchronize()
    idx_ms = sum(a.elapsed_time(b) for a, b, _ in recs) / len(recs)
    attn_ms = sum(b.elapsed_time(c) for _, b, c in recs) / len(recs)
    step_ms = sum(a.elapsed_time(c) for a, _, c in recs) / len(recs)
    blocks, cols, dens = layer_work(plans, n, cfg)
    flop = blocks * BLOCK_FLOP + cols * COL_FLOP
    nb = (n + 63) // 64
    out = {"tokens": n, "patterns": {kd: kinds.count(kd) for kd in sorted(set(kinds))}, "steps": len(recs),
           "warmup": 1, "step_ms": round(step_ms, 3), "index_ms": round(idx_ms, 3), "attn_ms": round(attn_ms, 3),
           "attn_tflops": round(flop / (attn_ms * 1e-3) / 1e12, 1),
           "mfma_frac": round(flop / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "computed_blocks": blocks, "gathered_columns": cols, "density": dens}
    if not no_dense:
        minf.minf_dense_attn(q, k, v, scale=scale, out=o, lse=lse)
        torch.cuda.synchronize()
        runs = []
        for _ in range(max(1, dense_runs)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            minf.minf_dense_attn(q, k, v, scale=scale, out=o, lse=lse)
            b.record(stream)
            runs.append((a, b))
        torch.cuda.synchronize()
        dense_ms = sum(a.elapsed_time(b) for a, b in runs) / len(runs)
        out["dense"] = {"ms": round(dense_ms, 2), "runs": len(runs), "warmup": 1,
                        "tflops": round(hq * nb * (nb + 1) // 2 * BLOCK_FLOP / (dense_ms * 1e-3) / 1e12, 1),
                        "speedup_step": round(dense_ms / step_ms, 3)}
    del q, k, v, o, lse, ws_vs, ws_bs, ws_at, st
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus above 1 is not supported "
                                   "(the heads of a layer would shard across GPUs with no exchange)"}))
        sys.exit(2)
    import torch

    from dynamic_sparse_attention_index_amd import minf
    from workload import CONFIGS, STRUCTURED_LATENT, config_kinds, injected_vs_index, planted_qkv

    torch.cuda.set_device(0)
    cfg = CONFIGS[args.config]
    n, hq, hkv = cfg["n"], cfg["hq"], cfg["hkv"]
    kinds = config_kinds(args.config)
    scale = 1 / math.sqrt(128)
    seed = 1000 + cfg["index"]
    t0 = time.perf_counter()
    q, k, v, info = planted_qkv(n, hq, hkv, seed=seed, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] inputs {args.config}: n={n} hq={hq} hkv={hkv} kinds={kinds.count('vs')} VS / "
          f"{kinds.count('block')} BS / {kinds.count('ashape')} A ({time.perf_counter() - t0:.1f} s)",
          file=sys.stderr, flush=True)

    if args.calib_copy_mib > 0:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] calibration copy of {args.calib_copy_mib} MiB done", file=sys.stderr, flush=True)

    vs_heads = [h for h in range(hq) if kinds[h] == "vs"]
    bs_heads = [h for h in range(hq) if kinds[h] == "block"]
    dev = q.device
    ws_vs = torch.empty(max(1, minf.library().minf_vs_index_workspace_size(n, len(vs_heads))), dtype=torch.uint8,
                        device=dev)
    ws_bs = torch.empty(max(1, minf.library().minf_block_index_workspace_size(n, hq, hkv, len(bs_heads))),
                        dtype=torch.uint8, device=dev)
    ws_at = torch.empty(max(1, minf.library().minf_sparse_attn_workspace_size(n, hq)), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((hq, n), dtype=torch.float32, device=dev)

    state = {}

    def build_index(qx=None, kx=None, st=None):
        qx = q if qx is None else qx
        kx = k if kx is None else kx
        st = state if st is None else st
        if vs_heads:
            st["vi"], st["si"] = minf.minf_build_vs_index(qx, kx, vs_heads, last_q=cfg["last_q"], k_v=cfg["k_v"],
                                                          k_s=cfg["k_s"], scale=scale, workspace=ws_vs)
        if bs_heads:
            st["bi"], st["bc"] = minf.minf_build_block_index(qx, kx, bs_heads, k_b=cfg["k_b"], workspace=ws_bs)

    def plans_from_state(st=None):
        state_ = state if st is None else st
        plans = []
        for h in range(hq):
            if kinds[h] == "vs":
                t = vs_heads.index(h)
                plans.append(dict(kind="vs", v_idx=state_["vi"][t], s_idx=state_["si"][t]))
            elif kinds[h] == "block":
                t = bs_heads.index(h)
                plans.append(dict(kind="block", blk_idx=state_["bi"][t], blk_cnt=state_["bc"][t]))
            else:
                plans.append(dict(kind="ashape", sink=cfg["sink"], local=cfg["local"]))
        return plans

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    if args.only_dense:
        # the dense causal attention alone on the workload's inputs
        for _ in range(args.warmup):
            minf.minf_dense_attn(q, k, v, scale=scale, out=o, lse=lse)
        torch.cuda.synchronize()
        reps = []
        for _ in range(args.steps):
            a, b = ev(), ev()
            a.record(stream)
            minf.minf_dense_attn(q, k, v, scale=scale, out=o, lse=lse)
            b.record(stream)
            reps.append((a, b))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in reps) / len(reps)
        nb_ = (n + 63) // 64
        tf = hq * nb_ * (nb_ + 1) // 2 * BLOCK_FLOP / (ms * 1e-3) / 1e12
        print(json.dumps({"workload": args.config, "dense_only": True, "steps": args.steps, "warmup": args.warmup,
                          "dense_ms": round(ms, 3), "tflops": round(tf, 1),
                          "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4)}))
        return

    if args.only_index:
        # the index build alone (VS and BS heads from the data), e.g. under a counter profiler
        for _ in range(args.warmup):
            build_index()
        torch.cuda.synchronize()
        reps = []
        for _ in range(args.steps):
            a, b = ev(), ev()
            a.record(stream)
            build_index()
            b.record(stream)
            reps.append((a, b))
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in reps) / len(reps)
        print(json.dumps({"workload": args.config, "index_only": True, "steps": args.steps, "warmup": args.warmup,
                          "index_ms": round(ms, 3), "vs_heads": len(vs_heads), "bs_heads": len(bs_heads)}))
        return

    def step(record=None):
        e0, e1, e2 = ev(), ev(), ev()
        e0.record(stream)
        build_index()
        e1.record(stream)
        plans = minf.make_plans(plans_from_state(), n=n, device=dev)
        minf.minf_sparse_attn(q, k, v, plans, scale=scale, out=o, lse=lse, workspace=ws_at)
        e2.record(stream)
        if record is not None:
            record.append((e0, e1, e2))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    recs = []
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    idx_ms = sum(a.elapsed_time(b) for a, b, _ in recs) / len(recs)
    attn_ms = sum(b.elapsed_time(c) for _, b, c in recs) / len(recs)
    step_ms = sum(a.elapsed_time(c) for a, _, c in recs) / len(recs)
    print(f"[bench] step {step_ms:.2f} ms (index {idx_ms:.3f} ms, attention {attn_ms:.2f} ms; wall {wall_ms:.2f})",
          file=sys.stderr, flush=True)

    # algorithmic work of the attention launch
    nb = (n + 63) // 64
    a_blocks = ashape_blocks(n, cfg["sink"], cfg["local"]) if "ashape" in kinds else 0

    def count_work(plans_x):
        blocks_x = cols_x = 0
        per_kind_x, head_work_x = {}, []
        for h in range(hq):
            p = plans_x[h]
            if p["kind"] == "vs":
                b_, c_ = vs_work(p["v_idx"], p["s_idx"], n)
            elif p["kind"] == "block":
                b_, c_ = int(p["blk_cnt"].long().sum()), 0
            else:
                b_, c_ = a_blocks, 0
            head_work_x.append((b_, c_))
            blocks_x += b_
            cols_x += c_
            pk = per_kind_x.setdefault(p["kind"], [0, 0, 0])
            pk[0] += b_
            pk[1] += c_
            pk[2] += 1
        dens = {kd: round((bk + cl / 64) / (cnt * nb * (nb + 1) / 2), 4) for kd, (bk, cl, cnt) in per_kind_x.items()}
        return blocks_x, cols_x, dens, head_work_x

    plans_t = plans_from_state()
    blocks, cols, density, head_work = count_work(plans_t)
    useful_flop = 512 * sum(useful_entries(p, n) for p in plans_t)  # 4 d flop per kept entry
    dense_blocks = hq * nb * (nb + 1) // 2
    flop = blocks * BLOCK_FLOP + cols * COL_FLOP
    attn_tflops = flop / (attn_ms * 1e-3) / 1e12
    print(f"[bench] computed blocks {blocks} + columns {cols} ({flop / 1e12:.1f} TFLOP); density {density}; "
          f"attention {attn_tflops:.0f} TFLOP/s", file=sys.stderr, flush=True)

    # index-build algorithmic HBM bytes: K once per KV group, last queries, and score/index arrays
    idx_bytes = 0
    if vs_heads:
        kv_used = {h // (hq // hkv) for h in vs_heads}
        idx_bytes += len(kv_used) * n * 128 * 2 + len(vs_heads) * (64 * 128 * 2 + 2 * n * 4 * 2)
    if bs_heads:
        kv_used = {h // (hq // hkv) for h in bs_heads}
        idx_bytes += (len(kv_used) + len(bs_heads)) * n * 128 * 2

    extra = {}
    # index-injected track: the pages' local-slash / scattered-vertical heads
    if not args.no_injected and vs_heads:
        inj = []
        vi_l, si_l = [], []
        for t, h in enumerate(vs_heads):
            g = h // (hq // hkv)
            a, b = injected_vs_index(n, cfg["k_v"], cfg["k_s"], info.columns[g], info.offsets, seed=seed + 100 + h)
            vi_l.append(a.cuda())
            si_l.append(b.cuda())
        inj_plans = []
        for h in range(hq):
            if kinds[h] == "vs":
                t = vs_heads.index(h)
                inj_plans.append(dict(kind="vs", v_idx=vi_l[t], s_idx=si_l[t]))
            else:
                inj_plans.append(plans_t[h])
        cp = minf.make_plans(inj_plans, n=n, device=dev)
        minf.minf_sparse_attn(q, k, v, cp, scale=scale, out=o, lse=lse, workspace=ws_at)
        torch.cuda.synchronize()
        reps = []
        for _ in range(max(2, args.steps)):
            a, b = ev(), ev()
            a.record(stream)
            minf.minf_sparse_attn(q, k, v, cp, scale=scale, out=o, lse=lse, workspace=ws_at)
            b.record(stream)
            reps.append((a, b))
        torch.cuda.synchronize()
        inj_attn_ms = sum(a.elapsed_time(b) for a, b in reps) / len(reps)
        ib = ic = 0
        for h in range(hq):
            if kinds[h] == "vs":
                t = vs_heads.index(h)
                b_, c_ = vs_work(vi_l[t], si_l[t], n)
            else:
                b_, c_ = head_work[h]
            ib += b_
            ic += c_
        inj_flop = ib * BLOCK_FLOP + ic * COL_FLOP
        extra["injected_track"] = {
            "attn_ms": round(inj_attn_ms, 3),
            "step_ms": round(inj_attn_ms + idx_ms, 3),
            "attn_tflops": round(inj_flop / (inj_attn_ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(inj_flop / (inj_attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "computed_blocks": ib, "gathered_columns": ic,
            "density": round((ib + ic / 64) / dense_blocks, 5),
            "note": "slashes [0, k_s) plus planted, verticals seeded-uniform plus planted; index build timed on the data",
        }
        print(f"[bench] injected track: attention {inj_attn_ms:.2f} ms, "
              f"{extra['injected_track']['attn_tflops']} TFLOP/s", file=sys.stderr, flush=True)

    # VS with slash-aligned windows (index shifting) on the same indexes: literal data (T1) and,
    # when run, the index-injected track (T3); compared with the block reading of those indexes
    if not args.no_window and vs_heads:
        def window_leg(plans_x, ref_ms):
            pw = [dict(kind="vs_window", v_idx=p["v_idx"], s_idx=p["s_idx"]) if p["kind"] == "vs" else p
                  for p in plans_x]
            cpw = minf.make_plans(pw, n=n, device=dev)
            minf.minf_sparse_attn(q, k, v, cpw, scale=scale, out=o, lse=lse, workspace=ws_at)
            torch.cuda.synchronize()
            reps_w = []
            for _ in range(max(2, args.steps)):
                a, b = ev(), ev()
                a.record(stream)
                minf.minf_sparse_attn(q, k, v, cpw, scale=scale, out=o, lse=lse, workspace=ws_at)
                b.record(stream)
                reps_w.append((a, b))
            torch.cuda.synchronize()
            ms = sum(a.elapsed_time(b) for a, b in reps_w) / len(reps_w)
            wt = wc = 0
            for h in range(hq):
                if pw[h]["kind"] == "vs_window":
                    t_, c_ = vsw_work(pw[h]["v_idx"], pw[h]["s_idx"], n)
                else:
                    t_, c_ = head_work[h]
                wt += t_
                wc += c_
            wf = wt * BLOCK_FLOP + wc * COL_FLOP
            return {"attn_ms": round(ms, 3), "computed_tiles": wt, "gathered_columns": wc,
                    "attn_tflops": round(wf / (ms * 1e-3) / 1e12, 1), "vs_block_reading_attn_ms": round(ref_ms, 3),
                    "time_vs_block_reading": round(ms / ref_ms, 3)}
        wl = {"literal": window_leg(plans_t, attn_ms)}
        if "injected_track" in extra:
            wl["injected"] = window_leg(inj_plans, extra["injected_track"]["attn_ms"])
        extra["vs_window"] = wl
        print(f"[bench] VS windows: " + ", ".join(
            f"{kk} {vv['attn_ms']:.2f} ms ({vv['computed_tiles']} tiles + {vv['gathered_columns']} columns, "
            f"{vv['attn_tflops']} TFLOP/s; x{vv['time_vs_block_reading']} the block reading)" for kk, vv in wl.items()),
            file=sys.stderr, flush=True)

    # structured track: the same layer on locality-latent data, index built from the data
    if not args.no_structured:
        t1 = time.perf_counter()
        q2, k2, v2, info2 = planted_qkv(n, hq, hkv, seed=seed, device="cuda", latent=STRUCTURED_LATENT)
        torch.cuda.synchronize()
        print(f"[bench] structured inputs: latent a^2={STRUCTURED_LATENT[0]} w={STRUCTURED_LATENT[1]} "
              f"({time.perf_counter() - t1:.1f} s)", file=sys.stderr, flush=True)
        st2 = {}

        def step2(record=None):
            e0, e1, e2 = ev(), ev(), ev()
            e0.record(stream)
            build_index(q2, k2, st2)
            e1.record(stream)
            cp2 = minf.make_plans(plans_from_state(st2), n=n, device=dev)
            minf.minf_sparse_attn(q2, k2, v2, cp2, scale=scale, out=o, lse=lse, workspace=ws_at)
            e2.record(stream)
            if record is not None:
                record.append((e0, e1, e2))

        step2()
        torch.cuda.synchronize()
        recs2 = []
        for _ in range(max(2, args.steps)):
            step2(recs2)
        torch.cuda.synchronize()
        s_idx_ms = sum(a.elapsed_time(b) for a, b, _ in recs2) / len(recs2)
        s_attn_ms = sum(b.elapsed_time(c) for _, b, c in recs2) / len(recs2)
        s_step_ms = sum(a.elapsed_time(c) for a, _, c in recs2) / len(recs2)
        sb, sc, sdens, _ = count_work(plans_from_state(st2))
        s_flop = sb * BLOCK_FLOP + sc * COL_FLOP
        diag = {}
        if vs_heads:
            w_lat = STRUCTURED_LATENT[1]
            loc = float((st2["si"] < w_lat).float().mean())
            rc = ro = 0
            for t, h in enumerate(vs_heads):
                g = h // (hq // hkv)
                cols_g = torch.tensor(info2.columns[g], device=dev, dtype=torch.int32)
                offs = torch.tensor(info2.offsets, device=dev, dtype=torch.int32)
                rc += int(torch.isin(cols_g, st2["vi"][t]).sum())
                ro += int(torch.isin(offs, st2["si"][t]).sum())
            diag = {"local_slash_frac": round(loc, 4),
                    "planted_columns_recovered": f"{rc}/{len(vs_heads) * len(info2.columns[0])}",
                    "planted_offsets_recovered": f"{ro}/{len(vs_heads) * len(info2.offsets)}"}
        extra["structured_track"] = {
            "step_ms": round(s_step_ms, 3), "index_ms": round(s_idx_ms, 3), "attn_ms": round(s_attn_ms, 3),
            "attn_tflops": round(s_flop / (s_attn_ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(s_flop / (s_attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "computed_blocks": sb, "gathered_columns": sc, "density": sdens,
            "latent": {"a2": STRUCTURED_LATENT[0], "w": STRUCTURED_LATENT[1]}, **diag,
        }
        print(f"[bench] structured track: step {s_step_ms:.2f} ms (index {s_idx_ms:.3f}, attention {s_attn_ms:.2f}), "
              f"{extra['structured_track']['attn_tflops']} TFLOP/s, density {sdens}, {diag}",
              file=sys.stderr, flush=True)
        del q2, k2, v2, st2

    dense = None
    if not args.no_dense:
        minf.minf_dense_attn(q, k, v, scale=scale, out=o, lse=lse)  # untimed warm-up
        torch.cuda.synchronize()
        runs = []
        for _ in range(max(1, args.dense_runs)):
            a, b = ev(), ev()
            a.record(stream)
            minf.minf_dense_attn(q, k, v, scale=scale, out=o, lse=lse)
            b.record(stream)
            runs.append((a, b))
        torch.cuda.synchronize()
        dense_ms = sum(a.elapsed_time(b) for a, b in runs) / len(runs)
        dense = {
            "ms": round(dense_ms, 2), "runs": max(1, args.dense_runs), "warmup": 1,
            "tflops": round(dense_blocks * BLOCK_FLOP / (dense_ms * 1e-3) / 1e12, 1),
            "speedup_step": round(dense_ms / step_ms, 3),
            "speedup_attention": round(dense_ms / attn_ms, 3),
        }
        for trk in ("injected_track", "structured_track"):
            if trk in extra:
                extra[trk]["speedup_step_vs_dense"] = round(dense_ms / extra[trk]["step_ms"], 2)
        print(f"[bench] dense {dense_ms:.1f} ms ({dense['tflops']} TFLOP/s), speedup {dense['speedup_step']}x",
              file=sys.stderr, flush=True)

    # grid track: a video-like input (frames x 256 patches) with grid-planted heads, permuted to
    # patch-major order, Block-Sparse index and attention in that order, output scattered back;
    # beside it the same block budget without the permutation, and dense attention on the same data
    if not args.no_grid and n % 256 == 0:
        from workload import grid_qkv
        patches = 256
        frames = n // patches
        k_b = args.grid_blocks
        t1 = time.perf_counter()
        qg, kg, vg = grid_qkv(frames, patches, hq, hkv, device="cuda")
        # patch-major order: permuted row p * frames + f holds original row f * patches + p
        fr = torch.arange(frames, device=dev, dtype=torch.int32)
        pa = torch.arange(patches, device=dev, dtype=torch.int32)
        src = (fr[None, :] * patches + pa[:, None]).reshape(-1).contiguous()
        torch.cuda.synchronize()
        print(f"[bench] grid inputs: {frames} frames x {patches} patches ({time.perf_counter() - t1:.1f} s)",
              file=sys.stderr, flush=True)
        heads_all = list(range(hq))
        og = torch.empty_like(qg)
        lg = torch.empty((hq, n), dtype=torch.float32, device=dev)

        def grid_step(record=None):
            e0, e1, e2, e3 = ev(), ev(), ev(), ev()
            e0.record(stream)
            qp = minf.minf_permute_rows(qg, src)
            kp = minf.minf_permute_rows(kg, src)
            vp = minf.minf_permute_rows(vg, src)
            bi, bc = minf.minf_build_permuted_block_index(qp, kp, heads_all, src, k_b=k_b)
            e1.record(stream)
            plans_g = minf.make_plans([dict(kind="block", blk_idx=bi[h], blk_cnt=bc[h], pos=src) for h in heads_all],
                                       n=n, device=dev)
            op, lp = minf.minf_sparse_attn(qp, kp, vp, plans_g, scale=scale, workspace=ws_at)
            e2.record(stream)
            minf.minf_permute_rows(op, src, scatter=True, out=og)
            minf.minf_permute_rows(lp.unsqueeze(-1).contiguous(), src, scatter=True, out=lg.unsqueeze(-1))
            e3.record(stream)
            if record is not None:
                record.append((e0, e1, e2, e3))
            return bc

        grid_step()
        torch.cuda.synchronize()
        recs_g = []
        for _ in range(max(2, args.steps)):
            bc_g = grid_step(recs_g)
        torch.cuda.synchronize()
        g_step = sum(a.elapsed_time(d_) for a, _, _, d_ in recs_g) / len(recs_g)
        g_attn = sum(b.elapsed_time(c) for _, b, c, _ in recs_g) / len(recs_g)
        g_pre = sum(a.elapsed_time(b) for a, b, _, _ in recs_g) / len(recs_g)
        g_blocks = int(bc_g.long().sum())
        lse_perm = lg.clone()
        # the same budget in the original order
        bj, bd = minf.minf_build_block_index(qg, kg, heads_all, k_b=k_b)
        plans_b = minf.make_plans([dict(kind="block", blk_idx=bj[h], blk_cnt=bd[h]) for h in heads_all], n=n, device=dev)
        a_, b_ = ev(), ev()
        a_.record(stream)
        _, lse_plain = minf.minf_sparse_attn(qg, kg, vg, plans_b, scale=scale, workspace=ws_at)
        b_.record(stream)
        torch.cuda.synchronize()
        plain_ms = a_.elapsed_time(b_)
        rows_s = torch.arange(0, n, 4099, device=dev)
        grid = {
            "frames": frames, "patches": patches, "k_b": k_b,
            "step_ms": round(g_step, 3), "permute_and_index_ms": round(g_pre, 3), "attn_ms": round(g_attn, 3),
            "computed_blocks": g_blocks, "density": round(g_blocks / dense_blocks, 5),
            "attn_tflops": round(g_blocks * BLOCK_FLOP / (g_attn * 1e-3) / 1e12, 1),
            "unpermuted_same_budget_attn_ms": round(plain_ms, 3),
        }
        if not args.no_dense:
            a_, b_ = ev(), ev()
            a_.record(stream)
            _, lse_d = minf.minf_dense_attn(qg, kg, vg, scale=scale)
            b_.record(stream)
            torch.cuda.synchronize()
            grid["dense_ms"] = round(a_.elapsed_time(b_), 2)
            grid["speedup_step_vs_dense"] = round(grid["dense_ms"] / g_step, 2)
            rec = lambda l_: float(torch.exp(l_[:, rows_s].double() - lse_d[:, rows_s].double()).mean())  # noqa: E731
            grid["recall_permuted"] = round(rec(lse_perm), 4)
            grid["recall_unpermuted_same_budget"] = round(rec(lse_plain), 4)
            del lse_d
        extra["grid_track"] = grid
        print(f"[bench] grid track: step {g_step:.2f} ms (permute + index {g_pre:.2f}, attention {g_attn:.2f}), "
              f"density {grid['density']}, recall {grid.get('recall_permuted')} vs unpermuted "
              f"{grid.get('recall_unpermuted_same_budget')}", file=sys.stderr, flush=True)
        del qg, kg, vg, og, lg, lse_perm

    # decoding on the same cache: the last query row of every head is the new token
    if not args.no_decode:
        qd = q[:, -1].contiguous()
        kt = minf.minf_decode_pool_keys(k)
        k_b = args.decode_blocks
        nb_ = (n + 63) // 64
        od = torch.empty_like(qd)
        ld = torch.empty((hq,), dtype=torch.float32, device=dev)
        blk = torch.empty((hq, min(k_b, nb_)), dtype=torch.int32, device=dev)
        ws_s = torch.empty(max(1, minf.library().minf_decode_workspace_size(n, hq, k_b)), dtype=torch.uint8,
                           device=dev)
        ws_d = torch.empty(max(1, minf.library().minf_decode_workspace_size(n, hq, nb_)), dtype=torch.uint8,
                           device=dev)

        def timed(fn, reps=50):
            fn()
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps

        def sparse_step():
            minf.minf_sparse_decode(qd, k, v, kt, k_b, scale=scale, out=od, lse=ld, blk_idx=blk, workspace=ws_s)

        sparse_us = 1e3 * timed(sparse_step)
        # the same step captured once into a HIP graph and replayed (one launch per step)
        sparse_step()
        torch.cuda.synchronize()
        ref = (od.clone(), ld.clone(), blk.clone())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            sparse_step()
        torch.cuda.synchronize()
        graph_us = 1e3 * timed(graph.replay)
        graph_ok = torch.equal(od, ref[0]) and torch.equal(ld, ref[1]) and torch.equal(blk, ref[2])

        def latency_us(fn, reps=50):
            # one step at a time, each waited for: what a token-by-token decoder sees
            fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                fn()
                torch.cuda.synchronize()
            return (time.perf_counter() - t0) / reps * 1e6

        lat_eager_us = latency_us(sparse_step)
        lat_graph_us = latency_us(graph.replay)
        dense_us = 1e3 * timed(lambda: minf.minf_dense_decode(qd, k, v, scale=scale, out=od, lse=ld, workspace=ws_d))
        pool_us = 1e3 * timed(lambda: minf.minf_decode_pool_keys(k, first_block=nb_ - 1, out=kt))
        row = 128 * 2 * 2  # one key row of K and V, bf16
        dense_bytes = hkv * n * row
        sel_rows = int(sum(min(64, n - 64 * c) for c in blk.flatten().tolist()))
        sparse_bytes = sel_rows * row + hkv * nb_ * 128 * 4 + hq * nb_ * 4 * 2
        extra["decode"] = {
            "k_b": k_b, "tokens_loaded_per_head": sel_rows // hq,
            "sparse_us": round(sparse_us, 2), "sparse_graph_us": round(graph_us, 2),
            "step_latency_us": {"eager": round(lat_eager_us, 1), "graph": round(lat_graph_us, 1)},
            "graph_replay_matches_eager": graph_ok, "dense_us": round(dense_us, 2),
            "speedup": round(dense_us / sparse_us, 2),
            "dense_hbm_gbs": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
            "sparse_algorithmic_bytes": sparse_bytes,
            "sparse_hbm_gbs": round(sparse_bytes / (sparse_us * 1e-6) / 1e9, 1),
            "append_pool_us": round(pool_us, 2),
            "note": "one new query row per head against the cache; top-k_b 64-token blocks by the pooled-key score; "
                    "dense loads every K/V row of every KV head",
        }
        print(f"[bench] decode: sparse {sparse_us:.1f} us (k_b={k_b}; {graph_us:.1f} us replayed from a graph; "
              f"one step waited for: {lat_eager_us:.1f} us eager, {lat_graph_us:.1f} us graph), "
              f"dense {dense_us:.1f} us "
              f"({extra['decode']['dense_hbm_gbs']} GB/s), speedup {extra['decode']['speedup']}x",
              file=sys.stderr, flush=True)
        del kt, ws_s, ws_d, graph

    # offline pattern search on this input (optional: it re-runs attention once per candidate)
    if args.search:
        from dynamic_sparse_attention_index_amd import pattern_search as PS
        cands = [dict(kind="ashape", sink=128, local=4096), dict(kind="vs", k_v=1000, k_s=6096),
                 dict(kind="vs", k_v=1000, k_s=1024), dict(kind="block", k_b=256), dict(kind="block", k_b=64)]
        budget = 0.1 * nb * (nb + 1) / 2
        torch.cuda.synchronize()
        t_s = time.perf_counter()
        res = PS.search_patterns(q, k, v, cands, budget, scale=scale, rows=torch.arange(0, n, 97, device=dev))
        torch.cuda.synchronize()
        search_s = time.perf_counter() - t_s
        picks = {}
        for c in res["choice"]:
            key = "none" if c < 0 else f"{cands[c]['kind']}:{','.join(str(cands[c][x]) for x in cands[c] if x != 'kind')}"
            picks[key] = picks.get(key, 0) + 1
        extra["pattern_search"] = {
            "seconds": round(search_s, 2), "candidates": len(cands), "budget_blocks_per_head": budget,
            "choices": picks, "mean_recall_of_choice": round(float(sum(
                res["recall"][h, c] for h, c in enumerate(res["choice"]) if c >= 0) / max(1, sum(
                    1 for c in res["choice"] if c >= 0))), 4),
            "note": "recall over every 97th query row; work budget 10% of the causal blocks",
        }
        print(f"[bench] pattern search: {search_s:.2f} s, choices {picks}", file=sys.stderr, flush=True)

    # further layers of the pages' length range (mixed pattern maps), after the headline
    layers = [x for x in args.layers.split(",") if x and x != args.config] if args.layers else []
    if layers:
        extra["layers"] = {}
        for name in layers:
            t_l = time.perf_counter()
            r = layer_leg(name, args.layer_steps, args.dense_runs, args.no_dense)
            extra["layers"][name] = r
            print(f"[bench] layer {name}: step {r['step_ms']:.2f} ms (index {r['index_ms']:.3f}, attention "
                  f"{r['attn_ms']:.2f}), {r['attn_tflops']} TFLOP/s, density {r['density']}, dense "
                  f"{r.get('dense', {}).get('ms')} ms ({time.perf_counter() - t_l:.1f} s)", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(q, k, v, kinds, cfg, plans_t, n)
        print(f"[bench] cpu oracle sample {cpu['sample_seconds']} s", file=sys.stderr, flush=True)

    out = {
        "metric": METRIC,
        "value": round(step_ms, 3),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": (f"synthetic seeded N(0,1) Q/K/V with planted verticals (8 columns per KV head, gain "
                 f"Q += {info.vert_gain[0]:g} u, K[c] += {info.vert_gain[1]:g} u, calibrated; the literal recipe's "
                 f"(1, 3) is not recoverable) and slashes (offsets {list(info.offsets)}, K_j += "
                 f"{info.slash_gain:g} Q0_(j+d)); index built on device from the data"),
        "config": {"workload": args.config, "tokens": n, "q_heads": hq, "kv_heads": hkv, "head_dim": 128,
                   "patterns": {kd: kinds.count(kd) for kd in sorted(set(kinds))},
                   "budgets": {key: cfg[key] for key in ("last_q", "k_v", "k_s", "k_b", "sink", "local") if key in cfg},
                   "causal": True},
        "index_ms": round(idx_ms, 3),
        "attention_ms": round(attn_ms, 3),
        "index_hbm_gbs": round(idx_bytes / (idx_ms * 1e-3) / 1e9, 1) if idx_ms > 0 else None,
        "index_hbm_frac": round(idx_bytes / (idx_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if idx_ms > 0 else None,
        "density": density,
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": profiled_traffic(args.config),
                     "kernel": "attn_kernel_rounds or attn_kernel (one sparse attention launch)", "flop_per_launch": flop,
                     "flop_rule": "4*64*64*128 per computed 64x64 block + 4*64*128 per gathered column per query block",
                     "useful_flop_per_launch": useful_flop,
                     "useful_tflops": round(useful_flop / (attn_ms * 1e-3) / 1e12, 1)},
        "dense": dense,
        "cpu_baseline": cpu,
    }
    out.update(extra)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
