"""Checks of the seeded input generators (CPU): determinism, marginals and the
locality latent's structure. These pin the inputs, not the method."""
import math

import numpy as np
import torch

import oracle as O
from workload import STRUCTURED_LATENT, planted_qkv


def test_generator_is_deterministic():
    a = planted_qkv(512, 2, 1, seed=7)
    b = planted_qkv(512, 2, 1, seed=7)
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    assert a[3].columns == b[3].columns


def test_latent_keeps_unit_marginals_and_plain_track_unchanged():
    n, w = 4096, 256
    q, k, v, _ = planted_qkv(n, 1, 1, seed=3, plant=False, latent=(0.8, w))
    for x in (q, k, v):
        xs = x.float()
        assert abs(float(xs.mean())) < 0.03
        assert abs(float(xs.std()) - 1.0) < 0.03
    # the plain draw ignores the latent knobs entirely
    q0, k0, v0, _ = planted_qkv(n, 1, 1, seed=3, plant=False)
    assert torch.equal(v, v0)  # V draws are not mixed with the latent
    assert not torch.equal(k, k0)


def test_latent_makes_scores_local():
    # q_i . k_j has mean a^2 d (1 - |i - j| / w) inside the window and 0 beyond it
    n, w, a2 = 8192, 512, 0.8
    q, k, _, _ = planted_qkv(n, 1, 1, seed=5, plant=False, latent=(a2, w))
    qf, kf = q[0].double(), k[0].double()
    i = torch.arange(2048, n, 97)
    for lag, want in ((0, a2 * 128), (w // 2, a2 * 128 * 0.5), (2 * w, 0.0)):
        got = float((qf[i] * kf[i - lag]).sum(-1).mean())
        assert abs(got - want) < 0.15 * a2 * 128 + 3, (lag, got, want)


def test_structured_vs_index_is_local_and_keeps_planted_slashes():
    n = 32768
    q, k, _, info = planted_qkv(n, 1, 1, seed=1003, latent=STRUCTURED_LATENT)
    vi, si, _, _ = O.vs_index(q[0].float().numpy(), k[0].float().numpy(), 64, 1000, 6096, 1 / math.sqrt(128))
    assert np.all(si < STRUCTURED_LATENT[1])
    assert set(info.offsets) <= set(si.tolist())
