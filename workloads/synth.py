"""Seeded synthetic workloads (shapes and value distributions only).

The pages measure this path on RULER needle-in-a-haystack prompts run through
trained Qwen3 / Llama models; neither the data nor the weights exist here, so
Gaussian Q/K/V with a few "planted" peaked keys stand in for them (the planted
keys play the needle).  Recipe:

* ``rng = numpy.random.default_rng(seed)``; draw order Q ``[total_q, Hq, d]``,
  then K, then V ``[total_k, Hkv, d]``, all standard normal float64.
* Planting (when ``planted > 0``): per sequence and KV head, ``planted``
  distinct key positions from ``rng.choice(Lk, planted, replace=False)``
  over the whole key range; those keys are set to ``4*sqrt(d)*u_hat`` where
  ``u_hat`` is the unit vector along the mean of that sequence's queries over
  the query heads of the group.
* Paged layout: the physical block ids are ``rng.permutation(num_blocks)``
  (drawn after planting); the table is padded with -1 (the convention of the
  paged-attention page's ``block_table`` example).
* Values are cast to the workload dtype (fp32 or bf16) with ``torch.to``;
  both sides consume the cast values.

The well-separated family (``make_well_separated``) makes every block's
estimated logit an integer rank, so block masses differ by a factor of ``e``
and the threshold cut has a wide margin.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

BLOCK = 128


@dataclasses.dataclass
class Workload:
    name: str
    q: torch.Tensor  # [total_q, Hq, d]
    k: torch.Tensor  # [total_k, Hkv, d] (logical, contiguous)
    v: torch.Tensor
    cu_q: list
    cu_k: list
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: torch.dtype
    stride: int
    block_size: int
    threshold: float
    kv_chunk_tokens: int
    select_mode: str  # "per_kvhead" | "chunk_vote"
    group_agg: str = "any"  # "any" | "majority"
    ring: bool = False
    ring_slots: int = 4
    ring_slot_blocks: int = 32
    # Paged view of the same K/V (filled by to_paged()).
    block_table: Optional[torch.Tensor] = None  # [batch, max_blocks] int32
    k_cache: Optional[torch.Tensor] = None  # [num_phys, 128, Hkv, d]
    v_cache: Optional[torch.Tensor] = None
    description: str = ""

    @property
    def batch(self) -> int:
        return len(self.cu_q) - 1

    def lens(self, b: int):
        return (self.cu_q[b + 1] - self.cu_q[b], self.cu_k[b + 1] - self.cu_k[b])

    @property
    def total_q(self) -> int:
        return self.cu_q[-1]

    @property
    def total_k(self) -> int:
        return self.cu_k[-1]


def _cast(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).contiguous()


def make_random(
    name: str,
    *,
    seed: int,
    hq: int,
    hkv: int,
    d: int,
    lq,
    lk,
    dtype=torch.bfloat16,
    stride: int = 8,
    threshold: float = 0.9,
    select_mode: str = "chunk_vote",
    kv_chunk_tokens: int = 4096,
    group_agg: str = "any",
    planted: int = 8,
    paged: bool = False,
    ring: bool = False,
    description: str = "",
) -> Workload:
    lq = list(lq)
    lk = list(lk)
    assert len(lq) == len(lk)
    cu_q = [0]
    cu_k = [0]
    for a, b in zip(lq, lk):
        cu_q.append(cu_q[-1] + a)
        cu_k.append(cu_k[-1] + b)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((cu_q[-1], hq, d))
    k = rng.standard_normal((cu_k[-1], hkv, d))
    v = rng.standard_normal((cu_k[-1], hkv, d))
    group = hq // hkv
    if planted > 0:
        for b in range(len(lq)):
            if lk[b] == 0:
                continue
            for g in range(hkv):
                pos = rng.choice(lk[b], planted, replace=False)
                qs = q[cu_q[b]:cu_q[b + 1], g * group:(g + 1) * group, :]
                u = qs.reshape(-1, d).mean(axis=0) if qs.size else np.ones(d)
                nrm = np.linalg.norm(u)
                u_hat = u / nrm if nrm > 0 else np.ones(d) / math.sqrt(d)
                k[cu_k[b] + pos, g, :] = 4.0 * math.sqrt(d) * u_hat
    w = Workload(
        name=name,
        q=_cast(q, dtype),
        k=_cast(k, dtype),
        v=_cast(v, dtype),
        cu_q=cu_q,
        cu_k=cu_k,
        num_q_heads=hq,
        num_kv_heads=hkv,
        head_dim=d,
        dtype=dtype,
        stride=stride,
        block_size=BLOCK,
        threshold=threshold,
        kv_chunk_tokens=kv_chunk_tokens,
        select_mode=select_mode,
        group_agg=group_agg,
        ring=ring,
        description=description,
    )
    if paged:
        to_paged(w, rng)
    return w


def to_paged(w: Workload, rng: np.random.Generator, max_blocks: Optional[int] = None) -> Workload:
    """Scatter the logical K/V into a shuffled cache of 128-token pages."""
    nblk = [(w.cu_k[b + 1] - w.cu_k[b] + BLOCK - 1) // BLOCK for b in range(w.batch)]
    total = sum(nblk)
    if max_blocks is None:
        max_blocks = max(nblk) if nblk else 0
    perm = rng.permutation(total)
    table = -np.ones((w.batch, max(max_blocks, 1)), dtype=np.int32)
    hkv, d = w.num_kv_heads, w.head_dim
    kc = torch.zeros((max(total, 1), BLOCK, hkv, d), dtype=w.dtype)
    vc = torch.zeros_like(kc)
    off = 0
    for b in range(w.batch):
        for n in range(nblk[b]):
            phys = int(perm[off + n])
            table[b, n] = phys
            t0 = w.cu_k[b] + n * BLOCK
            t1 = min(t0 + BLOCK, w.cu_k[b + 1])
            kc[phys, : t1 - t0] = w.k[t0:t1]
            vc[phys, : t1 - t0] = w.v[t0:t1]
        off += nblk[b]
    w.block_table = torch.from_numpy(table)
    w.k_cache = kc
    w.v_cache = vc
    return w


def make_well_separated(
    name: str,
    *,
    seed: int,
    hq: int,
    hkv: int,
    d: int,
    lq,
    lk,
    dtype=torch.bfloat16,
    stride: int = 8,
    threshold: float = 0.9,
    select_mode: str = "per_kvhead",
    kv_chunk_tokens: int = 4096,
    noise: float = 0.05,
    paged: bool = False,
    shared_ranks: bool = False,
    rank_step: float = 1.0,
    ring: bool = False,
    perms: Optional[list] = None,
) -> Workload:
    """Q[x,h] = sqrt(d) u_g + noise; K[y,g] = rank_step * pi_g(y // 128) u_g + noise.

    With est_scale = 1/(stride*sqrt(d)) the estimated logit of key block j is
    close to rank_step * pi_g(j), so sorted block masses fall by a factor of
    e^rank_step from one to the next.  ``shared_ranks`` draws one permutation
    per sequence for all KV heads (instead of one per head), so the heads
    agree on the important blocks and a chunk vote keeps them: the voted
    history is then a scattered subset whose size falls as rank_step grows.
    """
    lq = list(lq)
    lk = list(lk)
    cu_q = [0]
    cu_k = [0]
    for a, b in zip(lq, lk):
        cu_q.append(cu_q[-1] + a)
        cu_k.append(cu_k[-1] + b)
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((hkv, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    group = hq // hkv
    q = np.empty((cu_q[-1], hq, d))
    k = np.empty((cu_k[-1], hkv, d))
    for b in range(len(lq)):
        kb = lk[b] // BLOCK
        if shared_ranks:
            seq_perms = [rng.permutation(kb)] * hkv
        else:
            seq_perms = [rng.permutation(kb) for _ in range(hkv)]
        if perms is not None:  # given ranks (the draws above keep the stream aligned)
            seq_perms = [np.asarray(perms[b])] * hkv
        for g in range(hkv):
            for hh in range(group):
                h = g * group + hh
                q[cu_q[b]:cu_q[b + 1], h, :] = math.sqrt(d) * u[g]
            ranks = np.repeat(seq_perms[g], BLOCK)[: lk[b]].astype(np.float64)
            k[cu_k[b]:cu_k[b + 1], g, :] = rank_step * ranks[:, None] * u[g][None, :]
    q += noise * rng.standard_normal(q.shape)
    k += noise * rng.standard_normal(k.shape)
    v = rng.standard_normal((cu_k[-1], hkv, d))
    w = Workload(
        name=name,
        q=_cast(q, dtype),
        k=_cast(k, dtype),
        v=_cast(v, dtype),
        cu_q=cu_q,
        cu_k=cu_k,
        num_q_heads=hq,
        num_kv_heads=hkv,
        head_dim=d,
        dtype=dtype,
        stride=stride,
        block_size=BLOCK,
        threshold=threshold,
        kv_chunk_tokens=kv_chunk_tokens,
        select_mode=select_mode,
        ring=ring,
        description="well-separated block ranks (step %g%s)" % (rank_step, ", shared by the kv heads" if shared_ranks else ""),
    )
    if paged:
        to_paged(w, rng)
    return w


def make_layer_pair(seed: int, mix: float, **kw):
    """Two layers of one sequence whose important blocks partly agree: layer
    A is make_well_separated with shared ranks; layer B draws its own Q/K/V
    (seed + 1) with A's block ranks, except that a fraction ``mix`` of the
    blocks trade their ranks among themselves (0: the same ranks, 1: ranks
    unrelated to A's).  Single sequence; kw as make_well_separated."""
    wa = make_well_separated("layer_a", seed=seed, shared_ranks=True, **kw)
    lk = list(kw["lk"])[0]
    kb = lk // BLOCK
    ra = np.random.default_rng(seed)
    ra.standard_normal((kw["hkv"], kw["d"]))  # the draw of A's directions
    pa = ra.permutation(kb)  # A's shared ranks (first permutation drawn)
    rng = np.random.default_rng(seed + 1000)
    moved = rng.choice(kb, size=int(round(mix * kb)), replace=False)
    pb = pa.copy()
    pb[moved] = pa[rng.permutation(moved)]
    wb = make_well_separated("layer_b", seed=seed + 1, shared_ranks=True, perms=[pb], **kw)
    return wa, wb


def _tiny(seed=1):
    return make_random(
        "tiny_causal_fp32_1k",
        seed=seed, hq=1, hkv=1, d=64, lq=[1024], lk=[1024], dtype=torch.float32,
        stride=8, threshold=0.9, select_mode="per_kvhead", kv_chunk_tokens=0, planted=0,
        description="1 q head / 1 kv head, d=64, Lq=Lk=1024 causal, fp32 N(0,1), s=8, tau=0.9, one chunk",
    )


def _qwen06_4k(seed=2):
    return make_random(
        "qwen3_0p6b_4k",
        seed=seed, hq=16, hkv=8, d=128, lq=[4096], lk=[4096], dtype=torch.bfloat16,
        stride=8, threshold=0.9, select_mode="per_kvhead", kv_chunk_tokens=4096, planted=8,
        description="Qwen3-0.6B-shaped layer, 16q/8kv, d=128, bf16, Lq=Lk=4096 causal, planted peaks",
    )


def _chunk32k(seed=3):
    return make_random(
        "chunked_prefill_32k",
        seed=seed, hq=16, hkv=8, d=128, lq=[4096], lk=[32768], dtype=torch.bfloat16,
        stride=8, threshold=0.9, select_mode="chunk_vote", kv_chunk_tokens=4096, planted=8,
        description="last 4096-token chunk over 28K history (7 history chunks + current), 16q/8kv, d=128, bf16",
    )


def _ring128k(seed=4):
    return make_random(
        "qwen3_4b_128k_ring",
        seed=seed, hq=32, hkv=8, d=128, lq=[4096], lk=[131072], dtype=torch.bfloat16,
        stride=16, threshold=0.95, select_mode="chunk_vote", kv_chunk_tokens=4096, planted=8,
        ring=True,
        description="Qwen3-4B-shaped 128K context, 32q/8kv, d=128, bf16, history in pinned host memory via 4-slot ring",
    )


def _paged3(seed=5):
    return make_random(
        "paged_varlen_3seq",
        seed=seed, hq=16, hkv=8, d=128, lq=[2048, 2048, 2048], lk=[8192, 16384, 32768],
        dtype=torch.bfloat16, stride=8, threshold=0.9, select_mode="chunk_vote",
        kv_chunk_tokens=4096, planted=8, paged=True,
        description="3 sequences, KV 8K/16K/32K, 2048 new queries each, shuffled 128-token pages",
    )


def _chunk32k_sparse_vote(seed=203):
    w = make_well_separated(
        "chunked_prefill_32k_sparse_vote",
        seed=seed, hq=16, hkv=8, d=128, lq=[4096], lk=[32768], stride=8, threshold=0.9,
        select_mode="chunk_vote", kv_chunk_tokens=4096, shared_ranks=True, rank_step=0.04)
    w.description = ("the 32K chunk's shape on well-separated inputs whose block ranks the kv heads share "
                     "(step 0.04): the vote keeps about a quarter of the history")
    return w


def _chunk32k_sparse_kvhead(seed=204):
    w = make_well_separated(
        "chunked_prefill_32k_sparse_kvhead",
        seed=seed, hq=16, hkv=8, d=128, lq=[4096], lk=[32768], stride=8, threshold=0.9,
        select_mode="per_kvhead", kv_chunk_tokens=4096, shared_ranks=True, rank_step=0.1)
    w.description = ("the 32K chunk's shape on well-separated inputs (shared ranks, step 0.1), per-KV-head "
                     "selection: about a tenth of each row's blocks")
    return w


WORKLOADS = {
    "tiny_causal_fp32_1k": _tiny,
    "qwen3_0p6b_4k": _qwen06_4k,
    "chunked_prefill_32k": _chunk32k,
    "qwen3_4b_128k_ring": _ring128k,
    "paged_varlen_3seq": _paged3,
    # sparse regimes at the 32K shape (measurement stages, not configs)
    "chunked_prefill_32k_sparse_vote": _chunk32k_sparse_vote,
    "chunked_prefill_32k_sparse_kvhead": _chunk32k_sparse_kvhead,
}


def make_workload(name: str, seed: Optional[int] = None) -> Workload:
    fn = WORKLOADS[name]
    return fn() if seed is None else fn(seed)
