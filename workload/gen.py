"""Seeded synthetic workloads shaped like the pages' long-context prefill.

The pages measure on long-context suites (InfiniteBench, RULER, PG-19, needle
retrieval) with 8B-class models; none of those datasets or weights are used.
These generators stand in for them with the context lengths (4K to 1M tokens)
and the GQA layer shape (32 query heads, 8 KV heads, d = 128), plus planted
vertical and slash structure:

  * Q0, K, V ~ N(0, 1) drawn from the seed (float32, then rounded to bf16);
  * vertical plant: per KV head a random unit vector u and n_vert columns c;
    every query of the group's heads gets + a_v * u, and K[c] gets + b_v * u;
  * slash plant: K_j += slash_gain * Q0_{j + delta} for each planted offset
    delta (with j + delta < N), where Q0 is the pre-plant draw of the group's
    first query head.

The vertical gain (a_v, b_v) is a calibrated knob: at the literal (1, 3) the
planted columns add only ~0.27 nats to their logits and are not recoverable,
so a calibrated value is used and recorded with each workload.

Structured variant (locality latent, `latent=(a2, w)`): per KV group a latent
X_i = sum of the w white-noise rows ending at i, divided by the square root of
the number of rows summed, so every coordinate stays N(0, 1); then
Q0 = a X + sqrt(1 - a^2) Z_q for each query head of the group and
K = a X + sqrt(1 - a^2) Z_k, with a = sqrt(a2). Keys within w tokens of a
query share part of its latent, which makes attention local (as the pages
describe for real heads) while the marginals stay N(0, 1). The slash plant
uses the pre-latent draw Z_q of the group's first head.
"""
from __future__ import annotations

import dataclasses

import torch

SLASH_OFFSETS = (0, 1, 17, 300)


@dataclasses.dataclass
class PlantInfo:
    columns: list          # per KV head: sorted planted vertical columns
    offsets: tuple         # planted slash offsets
    vert_gain: tuple       # (a_v, b_v)
    slash_gain: float


def vertical_gain_for(n: int) -> tuple:
    """Calibrated vertical plant gain (the literal recipe's gain is (1, 3)).

    (7, 14) adds ~8.7 nats to a planted column's logits. With the oracle's
    VS estimate it recovers all 8 planted columns and all 4 planted offsets
    at N = 4096 (k = 64, 10 seeds), N = 32768 (k = 64, 4 seeds) and
    N = 131072 (k_v = 1000, k_s = 6096, 4 seeds); (10, 20) and above swamp the
    slashes at N = 32768. One value serves every length.
    """
    return (7.0, 14.0)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _latent(n: int, d: int, w: int, gen, device) -> torch.Tensor:
    """Moving sum of the last w rows of an N(0, 1) draw, scaled back to unit variance."""
    x = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
    x = torch.cumsum(x, dim=0)
    if w < n:
        x[w:] = x[w:] - x[:-w].clone()
    cnt = torch.clamp(torch.arange(1, n + 1, device=device, dtype=torch.float32), max=float(w))
    return x / cnt.sqrt()[:, None]


def planted_qkv(n: int, hq: int, hkv: int, d: int = 128, seed: int = 1000, device="cpu",
                vert_gain=None, n_vert: int = 8, slash_offsets=SLASH_OFFSETS,
                slash_gain: float = 0.8, plant: bool = True, latent=None):
    """Q [hq, n, d], K/V [hkv, n, d] as bf16 on `device`, plus the PlantInfo.

    latent: None (plain N(0, 1) draws) or (a2, w) for the locality latent.
    """
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    grp = hq // hkv
    gen = _gen(device, seed)
    if vert_gain is None:
        vert_gain = vertical_gain_for(n)
    a_v, b_v = float(vert_gain[0]), float(vert_gain[1])
    q = torch.empty((hq, n, d), dtype=torch.bfloat16, device=device)
    k = torch.empty((hkv, n, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((hkv, n, d), dtype=torch.bfloat16, device=device)
    cols_all = []
    offs = tuple(int(o) for o in slash_offsets if 0 <= int(o) < n)
    for g in range(hkv):
        u = torch.randn((d,), generator=gen, device=device, dtype=torch.float32)
        u = u / u.norm()
        kg = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
        vg = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
        span = max(1, n - 64)
        nv = min(n_vert, span)
        cols = torch.randperm(span, generator=gen, device=device)[:nv].sort().values
        if latent is not None:
            a = float(latent[0]) ** 0.5
            b = (1.0 - float(latent[0])) ** 0.5
            xg = _latent(n, d, int(latent[1]), gen, device)
            kg.mul_(b).add_(xg, alpha=a)
        for t in range(grp):
            h = g * grp + t
            q0 = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32)
            if plant and t == 0:
                for o in offs:
                    kg[: n - o] += slash_gain * q0[o:]
            if latent is not None:
                q0.mul_(b).add_(xg, alpha=a)
            if plant:
                q0 = q0 + a_v * u
            q[h] = q0.to(torch.bfloat16)
            del q0
        if plant and nv:
            kg[cols] += b_v * u
        k[g] = kg.to(torch.bfloat16)
        v[g] = vg.to(torch.bfloat16)
        cols_all.append(cols.cpu().tolist())
        del kg, vg
        if latent is not None:
            del xg
    return q, k, v, PlantInfo(cols_all, offs, (a_v, b_v), slash_gain)


def pattern_heads(n: int, d: int = 128, seed: int = 2000, device="cpu"):
    """Three synthetic heads (MHA: q, k, v [3, n, d] bf16), each built to favour
    one pattern, for the offline pattern search:

      head 0, vertical: 16 seeded key columns share a direction u with every
        query (Q += 4u, K[c] += 16u, about 5.7 nats);
      head 1, local: the locality latent with a short window (a^2 = 0.9, w = 256);
      head 2, block: every query block b >= 1 shares a random direction u_b
        with one seeded earlier key block c_b (Q_b += 8 u_b, K_{c_b} += 8 u_b).
    """
    gen = _gen(device, seed)
    q = torch.randn((3, n, d), generator=gen, device=device, dtype=torch.float32)
    k = torch.randn((3, n, d), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((3, n, d), generator=gen, device=device, dtype=torch.float32)
    # vertical head
    u = torch.randn((d,), generator=gen, device=device)
    u = u / u.norm()
    cols = torch.randperm(n, generator=gen, device=device)[:16]
    q[0] += 4.0 * u
    k[0, cols] += 16.0 * u
    # local head
    a2, w = 0.9, 256
    x = _latent(n, d, w, gen, device)
    q[1] = (1 - a2) ** 0.5 * q[1] + a2 ** 0.5 * x
    k[1] = (1 - a2) ** 0.5 * k[1] + a2 ** 0.5 * x
    # block head
    nb = (n + 63) // 64
    for b in range(1, nb):
        c = int(torch.randint(0, b, (1,), generator=gen, device=device))
        ub = torch.randn((d,), generator=gen, device=device)
        ub = ub / ub.norm()
        q[2, 64 * b: 64 * b + 64] += 8.0 * ub
        k[2, 64 * c: 64 * c + 64] += 8.0 * ub
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def grid_qkv(frames: int, patches: int, hq: int, hkv: int, d: int = 128, seed: int = 3000, gain: float = 8.0,
             device="cpu"):
    """Video-like inputs in frame-major order (token t = f * patches + p) whose
    heads show the grid pattern: every KV group has a random unit direction
    u_p per patch position p, added to the queries and keys of every frame at
    that position (Q += gain u_p, K += gain u_p, about gain^2 / sqrt(d) nats),
    so a query attends to the same patch in every earlier frame. Q, K, V
    [h, F * P, d] bf16 on `device`."""
    if hq % hkv:
        raise ValueError("hq must be a multiple of hkv")
    n = frames * patches
    gen = _gen(device, seed)
    q = torch.empty((hq, n, d), dtype=torch.bfloat16, device=device)
    k = torch.empty((hkv, n, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((hkv, n, d), dtype=torch.bfloat16, device=device)
    grp = hq // hkv
    for g in range(hkv):
        u = torch.randn((patches, d), generator=gen, device=device)
        u = u / u.norm(dim=1, keepdim=True)
        plant = u.repeat(frames, 1) * gain  # row f * patches + p gets u_p
        k[g] = (torch.randn((n, d), generator=gen, device=device) + plant).to(torch.bfloat16)
        v[g] = torch.randn((n, d), generator=gen, device=device).to(torch.bfloat16)
        for t in range(grp):
            q[g * grp + t] = (torch.randn((n, d), generator=gen, device=device) + plant).to(torch.bfloat16)
        del plant
    return q, k, v


def pattern_map(hq: int, n_vs: int, n_bs: int, n_a: int, seed: int) -> list:
    """Seeded per-head pattern kinds: a permutation of n_vs 'vs', n_bs 'block', n_a 'ashape'."""
    if n_vs + n_bs + n_a != hq:
        raise ValueError("pattern counts must add up to hq")
    kinds = ["vs"] * n_vs + ["block"] * n_bs + ["ashape"] * n_a
    perm = torch.randperm(hq, generator=_gen("cpu", seed)).tolist()
    out = [None] * hq
    for slot, h in enumerate(perm):
        out[h] = kinds[slot]
    return out


def injected_vs_index(n: int, k_v: int, k_s: int, planted_cols, planted_offsets, seed: int):
    """Index-injected VS structure (local slashes, scattered verticals).

    Slashes: the planted offsets plus the smallest offsets, k_s in total.
    Verticals: the planted columns plus seeded uniform columns, k_v in total.
    Both returned as sorted int32 tensors on the CPU.
    """
    k_s = min(k_s, n)
    k_v = min(k_v, n)
    s = sorted(set(int(o) for o in planted_offsets if 0 <= o < n))
    fill = 0
    ss = set(s)
    while len(ss) < k_s:
        ss.add(fill)
        fill += 1
    cols = set(int(c) for c in planted_cols if 0 <= c < n)
    if len(cols) < k_v:
        perm = torch.randperm(n, generator=_gen("cpu", seed)).tolist()
        for c in perm:
            if len(cols) >= k_v:
                break
            cols.add(c)
    sv = torch.tensor(sorted(cols)[:k_v], dtype=torch.int32)
    so = torch.tensor(sorted(ss)[:k_s], dtype=torch.int32)
    return sv, so


# Locality-latent knobs of the structured track, fixed for every length.
STRUCTURED_LATENT = (0.8, 32768)

# Named workloads (seed = 1000 + index; pattern maps use seed + 7).
CONFIGS = {
    "c1_vs_4k": dict(index=0, n=4096, hq=1, hkv=1, map=("vs",), last_q=64, k_v=64, k_s=64),
    "c2_ashape_bs_32k": dict(index=1, n=32768, hq=8, hkv=8,
                             map=("ashape",) * 4 + ("block",) * 4, sink=64, local=1024, k_b=128),
    "c3_gqa_128k": dict(index=2, n=131072, hq=32, hkv=8, counts=(20, 8, 4), last_q=64,
                        k_v=1000, k_s=6096, k_b=256, sink=128, local=4096),
    "c4_gqa_512k": dict(index=3, n=524288, hq=32, hkv=8, counts=(20, 8, 4), last_q=64,
                        k_v=1000, k_s=6096, k_b=256, sink=128, local=4096),
    "c5_gqa_1m_vs": dict(index=4, n=1048576, hq=32, hkv=8, counts=(32, 0, 0), last_q=64,
                         k_v=1000, k_s=6096),
}


def config_kinds(name: str) -> list:
    cfg = CONFIGS[name]
    if "map" in cfg:
        return list(cfg["map"])
    n_vs, n_bs, n_a = cfg["counts"]
    return pattern_map(cfg["hq"], n_vs, n_bs, n_a, 1000 + cfg["index"] + 7)
