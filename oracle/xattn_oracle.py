"""float64 reference for XAttention block-sparse prefill (estimate, select, attend).

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg; the product path never calls it and it
never imports the HIP library.

Everything is plain NumPy in float64 on values widened from the exact fp32 /
bf16 tensors the GPU receives.  Loops are per head and per 128-row query
block, so memory stays bounded; matrix products (``@``), ``argsort`` and
``cumsum`` are the only library steps.

Pages cited (by title and section):

* [BSA] "XAttention BSA Policy 设计文档" (nano-vllm design doc of
  ``XAttentionBSAPolicy``): 核心算法 §1 select_blocks Steps 1-4, §2
  compute_chunked_prefill, 参数配置, 限制, Density 统计 API.
* [SYNC] "XAttention Offload Stream Synchronization Fix": 技术细节 /
  三阶段 KV Chunking 流程 (partial stats, merge, normalise + block sum).
* [PAGED] "Atenção paginada" (transformers paged-attention page): Caminho
  Varlen / Exemplo (cu_seq_lens) and Caminho de decodificação / Exemplo
  (block_table, -1 = unallocated).

Readings where the pages are silent or ambiguous (each is listed with its
reason in the design notes of the repository):

R1  "stride reshape" scores pair query ``r*s + s-1-t`` with key ``c*s + t``
    (query rows reversed, key rows forward): the anti-diagonal of each s x s
    tile of Q K^T.
R2  estimate scale ``est_scale`` is an explicit argument (default
    ``1/(s*sqrt(d))``).
R3  causal masking in the estimate is at reshaped-tile level: cell (r, c) is
    allowed iff ``c <= r + o/s`` with ``o = Lk - Lq``; the diagonal tile is
    kept whole.
R5  threshold selection: per row, over allowed blocks ``j <= i + Kh``, order
    by (value desc, index asc); the k-th item is kept iff the float64 sum of
    the items before it, accumulated in that order, is ``< tau * T`` where
    ``T`` is the float64 sum of all allowed items in the same order.
    ``tau >= 1`` keeps every allowed block.
R22 top-k selection (``num_to_choose``, named but unused in the pages' call):
    when it is k > 0 it replaces the threshold: the k largest allowed blocks
    of the row in R5's order are kept (all of them if k >= their count); the
    aggregation, forcing and voting that follow are unchanged.
R6  forced blocks: chunk-vote mode forces the first and last history block
    after voting; per-KV-head mode forces the sink (j = 0) and the diagonal
    block (j = i + Kh).
R7  GQA aggregation ANY (default) or MAJORITY (2*count > G).
R9  the vote runs over history columns only, per sequence.
R10 chunk-vote mode keeps the current chunk dense causal.
R23 sparse-current chunk-vote mode (the current chunk selected per KV head,
    as the GPU-only mode selects over all KV): history columns follow the
    chunk vote exactly as in R9; current-chunk columns follow the per-KV-head
    rule (GQA aggregate of the threshold selection, sink and diagonal
    forced); counts are the per-KV-head statistics over every allowed
    (kv head, q block, block).  With no history it is per-KV-head mode.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

NEG_INF = -np.inf
BLOCK = 128

PER_KVHEAD = "per_kvhead"
CHUNK_VOTE = "chunk_vote"
CHUNK_VOTE_SPARSE = "chunk_vote_sparse"
AGG_ANY = "any"
AGG_MAJORITY = "majority"


# ---------------------------------------------------------------------------
# Layout helpers: varlen and paged addressing ([PAGED] Caminho Varlen,
# Caminho de decodificação).
# ---------------------------------------------------------------------------

def cu_seqlens(lengths):
    """Cumulative lengths with a leading 0 ([PAGED] Caminho Varlen, Exemplo)."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return out


def request_index(cu):
    """Sequence id of every packed token ([PAGED] Caminho Varlen, Exemplo)."""
    idx = []
    for b in range(len(cu) - 1):
        idx.extend([b] * (cu[b + 1] - cu[b]))
    return idx


def paged_location(block_table_row, token, block):
    """(physical block, offset) of a logical token via a block_table row.

    A -1 entry is an unallocated page ([PAGED] Caminho de decodificação,
    Exemplo); touching one is an error.
    """
    phys = int(block_table_row[token // block])
    if phys < 0:
        raise IndexError("token %d maps to an unallocated page" % token)
    return phys, token % block


def gather_paged(cache, block_table_row, length, block=BLOCK):
    """Logical [length, H, d] view of one sequence in a paged cache."""
    out = np.empty((length,) + tuple(cache.shape[2:]), dtype=np.float64)
    for t0 in range(0, length, block):
        phys, _ = paged_location(block_table_row, t0, block)
        n = min(block, length - t0)
        out[t0:t0 + n] = cache[phys, :n]
    return out


# ---------------------------------------------------------------------------
# O1: strided anti-diagonal scores and single-pass block sums
# ([BSA] 核心算法 §1 Step 1 flat_group_gemm_fuse_reshape, Step 2
# softmax_fuse_block_sum).
# ---------------------------------------------------------------------------

def strided_scores(q, k, stride, group):
    """S[h, r, c] = sum_t <q[r*s + s-1-t, h], k[c*s + t, h // group]>  (R1).

    q: [Lq, Hq, d], k: [Lk, Hkv, d].  Returns [Hq, Lq/s, Lk/s].  The GQA head
    map h -> h // group is the repeat_interleave of [BSA] Step 1.
    """
    lq, hq, d = q.shape
    lk = k.shape[0]
    r_n, c_n = lq // stride, lk // stride
    s_out = np.zeros((hq, r_n, c_n))
    for h in range(hq):
        g = h // group
        for t in range(stride):
            qt = q[stride - 1 - t::stride, h, :][:r_n]  # rows r*s + s-1-t
            kt = k[t::stride, g, :][:c_n]  # rows c*s + t
            s_out[h] += qt @ kt.T
    return s_out


def estimate_allowed(r_n, c_n, col_offset):
    """Tile-level causal mask of the reshaped score grid (R3): c <= r + o/s."""
    r = np.arange(r_n)[:, None]
    c = np.arange(c_n)[None, :]
    return c <= r + col_offset


def _block_sum_rows(p, rb):
    """Sum a [R, C] matrix over rb x rb tiles -> [R/rb, C/rb]."""
    r_n, c_n = p.shape
    return p.reshape(r_n // rb, rb, c_n // rb, rb).sum(axis=(1, 3))


def estimate_block_sums(q, k, *, stride, block, est_scale, group):
    """Single-pass definition (O1): row softmax of est_scale*S over allowed
    cells, then sums over (block/s) x (block/s) tiles -> [Hq, Qb, Kb]
    ([BSA] Step 2: reshaped_block_size = block_size / stride)."""
    lq, hq, _ = q.shape
    lk = k.shape[0]
    rb = block // stride
    r_n, c_n = lq // stride, lk // stride
    col_off = (lk - lq) // stride
    allowed = estimate_allowed(r_n, c_n, col_off)
    out = np.zeros((hq, lq // block, lk // block))
    for h in range(hq):
        s_h = strided_scores(q[:, h:h + 1, :], k[:, (h // group):(h // group) + 1, :], stride, 1)[0]
        z = np.where(allowed, est_scale * s_h, NEG_INF)
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        p = e / e.sum(axis=1, keepdims=True)
        out[h] = _block_sum_rows(p, rb)
    return out


# ---------------------------------------------------------------------------
# O2: chunked two-pass estimate ([SYNC] 技术细节, 三阶段 KV Chunking:
# Stage 1 softmax_compute_partial_stats, Stage 2 merge_softmax_stats,
# Stage 3 softmax_normalize_and_block_sum).
# ---------------------------------------------------------------------------

def partial_softmax_stats(z):
    """Stage 1: per row (m, l) over one KV chunk; a row with no allowed cell
    gets m = -inf, l = 0."""
    m = z.max(axis=1)
    l = np.zeros_like(m)
    ok = np.isfinite(m)
    if ok.any():
        l[ok] = np.exp(z[ok] - m[ok, None]).sum(axis=1)
    return m, l


def merge_softmax_stats(ms, ls):
    """Stage 2: m = max_k m_k, l = sum_k l_k * exp(m_k - m)."""
    ms = np.stack(ms)
    ls = np.stack(ls)
    m = ms.max(axis=0)
    l = np.zeros_like(m)
    for mk, lk in zip(ms, ls):
        ok = np.isfinite(mk)
        l[ok] += lk[ok] * np.exp(mk[ok] - m[ok])
    return m, l


def normalize_and_block_sum(z, m, l, rb):
    """Stage 3: P = exp(z - m) / l on allowed cells, then tile sums."""
    p = np.exp(z - m[:, None]) / l[:, None]
    return _block_sum_rows(p, rb)


def estimate_block_sums_chunked(q, k, *, stride, block, est_scale, group, chunk_tokens):
    """Two-pass estimate over KV chunks of ``chunk_tokens`` keys (O2)."""
    lq, hq, _ = q.shape
    lk = k.shape[0]
    rb = block // stride
    r_n = lq // stride
    col_off = (lk - lq) // stride
    if chunk_tokens <= 0:
        chunk_tokens = lk
    bounds = [(a, min(a + chunk_tokens, lk)) for a in range(0, lk, chunk_tokens)]
    out = np.zeros((hq, lq // block, lk // block))
    for h in range(hq):
        g = h // group
        zs, ms, ls = [], [], []
        for a, b in bounds:  # pass 1
            s_h = strided_scores(q[:, h:h + 1, :], k[a:b, g:g + 1, :], stride, 1)[0]
            c0 = a // stride
            allowed = estimate_allowed(r_n, (b - a) // stride, col_off - c0)
            z = np.where(allowed, est_scale * s_h, NEG_INF)
            m_k, l_k = partial_softmax_stats(z)
            zs.append(z)
            ms.append(m_k)
            ls.append(l_k)
        m, l = merge_softmax_stats(ms, ls)
        for (a, b), z in zip(bounds, zs):  # pass 2
            out[h, :, a // block:b // block] = normalize_and_block_sum(z, m, l, rb)
    return out


# ---------------------------------------------------------------------------
# O3: find_blocks_chunked threshold selection ([BSA] 核心算法 §1 Step 3; R5).
# ---------------------------------------------------------------------------

def threshold_select_row(v, tau):
    """Boolean keep-mask over the allowed blocks of one row (R5)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    if n == 0:
        return np.zeros(0, dtype=bool)
    if tau >= 1.0:
        return np.ones(n, dtype=bool)
    order = np.argsort(-v, kind="stable")  # value desc, index asc on ties
    vs = v[order]
    before = np.concatenate([[0.0], np.cumsum(vs)])  # left-to-right float64
    total = before[-1]
    thr = tau * total
    keep = np.zeros(n, dtype=bool)
    keep[order] = before[:n] < thr
    return keep


def topk_select_row(v, k):
    """Boolean keep-mask of the k largest allowed blocks of one row: the
    fixed-count alternative (``num_to_choose``) to the threshold in the
    find_blocks_chunked call ([BSA] 核心算法 §1 Step 3).  Order as in R5
    (value desc, index asc on ties); k >= n keeps every allowed block."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    keep = np.zeros(n, dtype=bool)
    if n == 0 or k <= 0:
        return keep
    order = np.argsort(-v, kind="stable")
    keep[order[:min(k, n)]] = True
    return keep


# ---------------------------------------------------------------------------
# O4-O6: GQA aggregation, forced blocks, majority vote, effective mask
# ([BSA] 核心算法 §1 Step 4) and O9 counts ([BSA] Density 统计 API).
# ---------------------------------------------------------------------------

def select_blocks(bs, *, kh, tau, group, mode, agg=AGG_ANY, num_to_choose=0):
    """bs: [Hq, Qb, Kb] block sums of one sequence.  ``num_to_choose`` > 0
    replaces the threshold rule by the top-k rule (topk_select_row).

    Returns dict(mask_q [Hq,Qb,Kb], mask_kv [Hkv,Qb,Kb] effective attention
    mask, hist_sel [Kb], counts (selected, available)).
    """
    hq, qb, kb = bs.shape
    hkv = hq // group
    allowed = np.arange(kb)[None, :] <= (np.arange(qb)[:, None] + kh)  # [Qb, Kb]
    mask_q = np.zeros((hq, qb, kb), dtype=bool)
    for h in range(hq):
        for i in range(qb):
            n = i + kh + 1
            if num_to_choose > 0:
                mask_q[h, i, :n] = topk_select_row(bs[h, i, :n], num_to_choose)
            else:
                mask_q[h, i, :n] = threshold_select_row(bs[h, i, :n], tau)
    cnt = mask_q.reshape(hkv, group, qb, kb).sum(axis=1)
    if agg == AGG_ANY:
        per_kv = cnt > 0
    elif agg == AGG_MAJORITY:
        per_kv = 2 * cnt > group
    else:
        raise ValueError(agg)
    hist_sel = np.zeros(kb, dtype=bool)
    if mode == PER_KVHEAD:
        eff = per_kv.copy()
        for i in range(qb):
            eff[:, i, 0] = True
            eff[:, i, i + kh] = True
        eff &= allowed[None]
        counts = (int(eff.sum()), int(hkv * allowed.sum()))
    elif mode in (CHUNK_VOTE, CHUNK_VOTE_SPARSE):
        if kh > 0:
            votes = per_kv[:, :, :kh].sum(axis=(0, 1))  # [Kh]
            hist_sel[:kh] = 2 * votes > hkv * qb  # strictly more than half
            hist_sel[0] = True
            hist_sel[kh - 1] = True
        eff = np.zeros((hkv, qb, kb), dtype=bool)
        eff[:, :, :kh] = hist_sel[None, None, :kh]
        if mode == CHUNK_VOTE:
            eff[:, :, kh:] = allowed[None, :, kh:]
            counts = (int(hist_sel.sum()), int(kh))
        else:
            # R23: the current chunk per KV head, sink and diagonal forced
            cur = per_kv.copy()
            for i in range(qb):
                cur[:, i, 0] = True
                cur[:, i, i + kh] = True
            eff[:, :, kh:] = cur[:, :, kh:] & allowed[None, :, kh:]
            counts = (int(eff.sum()), int(hkv * allowed.sum()))
    else:
        raise ValueError(mode)
    return {"mask_q": mask_q, "mask_kv": eff, "hist_sel": hist_sel, "counts": counts}


def density(counts_list):
    """overall density = sum selected / sum available ([BSA] Density 统计 API)."""
    sel = sum(int(c[0]) for c in counts_list)
    avail = sum(int(c[1]) for c in counts_list)
    return sel / avail if avail else float("nan")


# ---------------------------------------------------------------------------
# O7: block-sparse attention with LSE ([BSA] 核心算法 §2
# compute_chunked_prefill, flash_attn_with_lse).
# ---------------------------------------------------------------------------

def sparse_attention(q, k, v, mask, *, softmax_scale, group, block=BLOCK, rows=None,
                     key_range=None, causal=True):
    """Attention of each query over the keys its block mask keeps.

    q: [Lq, Hq, d]; k, v: [Lk, Hkv, d]; mask: [Hkv, Qb, Kb] bool.  Query x
    sits at absolute position o + x (o = Lk - Lq); with ``causal`` a key y is
    visible iff y <= o + x.  ``key_range=(a, b)`` restricts keys to [a, b).
    Returns (out [Lq, Hq, d], lse [Hq, Lq]); rows without any visible key
    get out = 0 and lse = -inf.  ``rows`` limits the work to those query
    indices (others are NaN).
    """
    lq, hq, d = q.shape
    lk = k.shape[0]
    o = lk - lq
    a, b = (0, lk) if key_range is None else key_range
    out = np.full((lq, hq, d), np.nan)
    lse = np.full((hq, lq), np.nan)
    row_set = np.arange(lq) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    for h in range(hq):
        g = h // group
        for i in sorted(set(int(x) // block for x in row_set)):
            xs = row_set[(row_set // block) == i]
            blocks = [j for j in range(mask.shape[2]) if mask[g, i, j]]
            keys = np.concatenate([np.arange(j * block, (j + 1) * block) for j in blocks]) if blocks else np.zeros(0, dtype=np.int64)
            keys = keys[(keys >= a) & (keys < b) & (keys < lk)]
            s = softmax_scale * (q[xs, h, :] @ k[keys, g, :].T)  # [n_rows, n_keys]
            if causal:
                s = np.where(keys[None, :] <= (o + xs)[:, None], s, NEG_INF)
            m = s.max(axis=1, keepdims=True) if keys.size else np.full((xs.size, 1), NEG_INF)
            ok = np.isfinite(m[:, 0])
            e = np.zeros_like(s)
            e[ok] = np.exp(s[ok] - m[ok])
            l = e.sum(axis=1)
            res = np.zeros((xs.size, d))
            res[ok] = (e[ok] @ v[keys, g, :]) / l[ok, None]
            out[xs, h, :] = res
            lse_row = np.full(xs.size, NEG_INF)
            lse_row[ok] = m[ok, 0] + np.log(l[ok])
            lse[h, xs] = lse_row
    return out, lse


# ---------------------------------------------------------------------------
# O8: merge of two partial attentions ([BSA] 核心算法 §2,
# merge_attention_outputs).
# ---------------------------------------------------------------------------

def merge_attention(o_a, lse_a, o_b, lse_b):
    """lse = max + log1p(exp(-|a-b|)); O = e^{a-lse} O_a + e^{b-lse} O_b.

    o_*: [rows, H, d]; lse_*: [H, rows].  A side with lse = -inf adds 0.
    """
    a = np.asarray(lse_a, dtype=np.float64)
    b = np.asarray(lse_b, dtype=np.float64)
    mx = np.maximum(a, b)
    both_inf = ~np.isfinite(mx)
    diff = np.where(both_inf, 0.0, -np.abs(a - b))
    diff = np.where(np.isnan(diff), -np.inf, diff)
    lse = np.where(both_inf, NEG_INF, mx + np.log1p(np.exp(diff)))
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isfinite(a), np.exp(a - lse), 0.0)
        wb = np.where(np.isfinite(b), np.exp(b - lse), 0.0)
    o = wa.T[:, :, None] * np.nan_to_num(o_a) + wb.T[:, :, None] * np.nan_to_num(o_b)
    return o, lse


def chunked_prefill_attention(q, k, v, hist_sel, *, softmax_scale, group, block=BLOCK, rows=None):
    """The pages' chunk order: selected history blocks without a causal mask,
    then the current chunk with one, merged history-first ([BSA] §2)."""
    lq, hq, _ = q.shape
    lk = k.shape[0]
    kh = (lk - lq) // block
    qb = lq // block
    kb = lk // block
    hkv = hq // group
    hist_mask = np.zeros((hkv, qb, kb), dtype=bool)
    hist_mask[:, :, :kh] = np.asarray(hist_sel[:kh], dtype=bool)[None, None, :]
    cur_mask = np.zeros((hkv, qb, kb), dtype=bool)
    cur_mask[:, :, kh:] = True
    o_h, l_h = sparse_attention(q, k, v, hist_mask, softmax_scale=softmax_scale, group=group,
                                block=block, rows=rows, causal=False)
    o_c, l_c = sparse_attention(q, k, v, cur_mask, softmax_scale=softmax_scale, group=group,
                                block=block, rows=rows, causal=True)
    if kh == 0:
        return o_c, l_c
    return merge_attention(o_h, l_h, o_c, l_c)


# ---------------------------------------------------------------------------
# Whole path for a packed / paged batch.
# ---------------------------------------------------------------------------

def to_f64(t):
    """Widen a CPU tensor (fp32 / bf16) or array to a float64 ndarray."""
    if hasattr(t, "detach"):
        import torch  # local: only tensors need it
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def sequence_kv(k, v, cu_k, b, block_table=None, k_cache=None, v_cache=None, block=BLOCK):
    lk = cu_k[b + 1] - cu_k[b]
    if block_table is not None:
        row = np.asarray(block_table[b])
        return gather_paged(k_cache, row, lk, block), gather_paged(v_cache, row, lk, block)
    return k[cu_k[b]:cu_k[b + 1]], v[cu_k[b]:cu_k[b + 1]]


def prefill(q, k, v, cu_q, cu_k, *, num_kv_heads, stride, block=BLOCK, threshold,
            est_scale=None, softmax_scale=None, kv_chunk_tokens=0, mode=PER_KVHEAD,
            agg=AGG_ANY, block_table=None, k_cache=None, v_cache=None, rows=None,
            attention=True, pages_order=False, num_to_choose=0):
    """Estimate -> select -> attend for every sequence of a packed batch.

    q: [total_q, Hq, d]; k, v: [total_k, Hkv, d] (or paged caches via
    ``block_table``).  ``rows``: optional dict b -> query indices to attend.
    ``pages_order`` evaluates chunk-vote attention as history-then-current
    with a merge (identical up to rounding to one masked pass; chunk_vote
    mode only).
    Returns a dict with block_sums [B,Hq,maxQb,maxKb], mask_q, mask_kv
    [B,Hkv,maxQb,maxKb], hist_sel [B,maxKb], counts [B,2], out
    [total_q,Hq,d], lse [Hq,total_q].
    """
    q = to_f64(q)
    if block_table is None:
        k = to_f64(k)
        v = to_f64(v)
    else:
        k_cache = to_f64(k_cache)
        v_cache = to_f64(v_cache)
        block_table = np.asarray(block_table)
    total_q, hq, d = q.shape
    group = hq // num_kv_heads
    if est_scale is None:
        est_scale = 1.0 / (stride * math.sqrt(d))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    nb = len(cu_q) - 1
    lqs = [cu_q[b + 1] - cu_q[b] for b in range(nb)]
    lks = [cu_k[b + 1] - cu_k[b] for b in range(nb)]
    max_qb = max([x // block for x in lqs] + [0])
    max_kb = max([x // block for x in lks] + [0])
    res = {
        "block_sums": np.zeros((nb, hq, max_qb, max_kb)),
        "mask_q": np.zeros((nb, hq, max_qb, max_kb), dtype=bool),
        "mask_kv": np.zeros((nb, num_kv_heads, max_qb, max_kb), dtype=bool),
        "hist_sel": np.zeros((nb, max_kb), dtype=bool),
        "counts": np.zeros((nb, 2), dtype=np.int64),
        "out": np.full((total_q, hq, d), np.nan),
        "lse": np.full((hq, total_q), np.nan),
    }
    for b in range(nb):
        lq, lk = lqs[b], lks[b]
        if lq == 0:
            continue
        qb_, kb_ = lq // block, lk // block
        kh = (lk - lq) // block
        q_b = q[cu_q[b]:cu_q[b + 1]]
        k_b, v_b = sequence_kv(k, v, cu_k, b, block_table, k_cache, v_cache, block)
        if kv_chunk_tokens and kv_chunk_tokens < lk:
            bs = estimate_block_sums_chunked(q_b, k_b, stride=stride, block=block,
                                             est_scale=est_scale, group=group,
                                             chunk_tokens=kv_chunk_tokens)
        else:
            bs = estimate_block_sums(q_b, k_b, stride=stride, block=block,
                                     est_scale=est_scale, group=group)
        sel = select_blocks(bs, kh=kh, tau=threshold, group=group, mode=mode, agg=agg,
                            num_to_choose=num_to_choose)
        res["block_sums"][b, :, :qb_, :kb_] = bs
        res["mask_q"][b, :, :qb_, :kb_] = sel["mask_q"]
        res["mask_kv"][b, :, :qb_, :kb_] = sel["mask_kv"]
        res["hist_sel"][b, :kb_] = sel["hist_sel"]
        res["counts"][b] = sel["counts"]
        if not attention:
            continue
        r_b = None if rows is None else rows.get(b, [])
        if r_b is not None and len(r_b) == 0:
            continue
        if pages_order and mode == CHUNK_VOTE:
            o_b, l_b = chunked_prefill_attention(q_b, k_b, v_b, sel["hist_sel"],
                                                 softmax_scale=softmax_scale, group=group,
                                                 block=block, rows=r_b)
        else:
            o_b, l_b = sparse_attention(q_b, k_b, v_b, sel["mask_kv"], softmax_scale=softmax_scale,
                                        group=group, block=block, rows=r_b)
        res["out"][cu_q[b]:cu_q[b + 1]] = o_b
        res["lse"][:, cu_q[b]:cu_q[b + 1]] = l_b
    return res


def selection_margin(v, tau):
    """Distance of one row's threshold cut from flipping, relative to T.

    min over the cut of (tau*T - C_{k-1})/T, (C_k - tau*T)/T and
    (v_(k) - v_(k+1))/T, where k items are kept.  Large margins mean a
    perturbed estimate still yields the same mask.
    """
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    if n == 0 or tau >= 1.0:
        return np.inf
    order = np.argsort(-v, kind="stable")
    vs = v[order]
    c = np.concatenate([[0.0], np.cumsum(vs)])
    t = c[-1]
    if t <= 0:
        return 0.0
    thr = tau * t
    kept = int((c[:n] < thr).sum())
    cands = []
    if kept >= 1:
        cands.append((thr - c[kept - 1]) / t)
    if kept < n:
        cands.append((c[kept] - thr) / t)
        if kept >= 1:
            cands.append((vs[kept - 1] - vs[kept]) / t)
    return min(cands) if cands else np.inf
