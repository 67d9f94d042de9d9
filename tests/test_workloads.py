"""Seeded generators: determinism, layout and the paged scatter (CPU)."""

import numpy as np
import torch

from workloads import make_random, make_well_separated, to_paged


def test_generator_is_deterministic_and_shaped():
    a = make_random("t", seed=7, hq=4, hkv=2, d=32, lq=[256, 128], lk=[512, 128])
    b = make_random("t", seed=7, hq=4, hkv=2, d=32, lq=[256, 128], lk=[512, 128])
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    assert a.q.shape == (384, 4, 32) and a.k.shape == (640, 2, 32)
    assert a.cu_q == [0, 256, 384] and a.cu_k == [0, 512, 640]
    assert a.q.dtype == torch.bfloat16


def test_planted_keys_are_large():
    w = make_random("t", seed=8, hq=2, hkv=1, d=64, lq=[256], lk=[1024], dtype=torch.float32, planted=8)
    norms = w.k[:, 0, :].norm(dim=-1)
    assert int((norms > 0.9 * 4 * 8).sum()) == 8  # 4*sqrt(64) = 32


def test_paged_scatter_roundtrip():
    w = make_random("t", seed=9, hq=2, hkv=1, d=16, lq=[128, 256], lk=[384, 640], dtype=torch.float32)
    to_paged(w, np.random.default_rng(0), max_blocks=8)
    bt = w.block_table
    assert bt.shape == (2, 8) and (bt[0, 3:] == -1).all() and (bt[1, 5:] == -1).all()
    ids = sorted(bt[bt >= 0].tolist())
    assert ids == list(range(8))
    for b in range(2):
        for n in range((w.cu_k[b + 1] - w.cu_k[b]) // 128):
            t0 = w.cu_k[b] + n * 128
            assert torch.equal(w.k_cache[bt[b, n]], w.k[t0:t0 + 128])


def test_well_separated_shapes():
    w = make_well_separated("ws", seed=101, hq=4, hkv=2, d=32, lq=[256], lk=[512])
    assert w.q.shape == (256, 4, 32) and w.k.shape == (512, 2, 32)
