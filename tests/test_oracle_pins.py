"""Pins of the float64 oracle against facts it does not compute itself.

Each pin is chosen so that a plausible slip (a dropped term, a wrong sign or
index, a transposed operand, <= for <) fails it; the ``*_mutant`` tests plant
such slips in copies of oracle functions and check the pin rejects them.
All tests here run on the CPU.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from tests.conftest import GOLDEN


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- O1 scores

def _brute_scores(q, k, stride, group):
    """Dense Q K^T, then gather each s x s tile's anti-diagonal by index."""
    lq, hq, d = q.shape
    lk = k.shape[0]
    out = np.zeros((hq, lq // stride, lk // stride))
    for h in range(hq):
        dense = q[:, h, :] @ k[:, h // group, :].T
        for r in range(lq // stride):
            for c in range(lk // stride):
                acc = 0.0
                for t in range(stride):
                    acc += dense[r * stride + stride - 1 - t, c * stride + t]
                out[h, r, c] = acc
    return out


@pytest.mark.parametrize("stride", [1, 2, 4, 8])
def test_strided_scores_match_bruteforce_antidiagonal(stride):
    q = _rand((32, 4, 8), 1)
    k = _rand((64, 2, 8), 2)
    got = O.strided_scores(q, k, stride, group=2)
    ref = _brute_scores(q, k, stride, group=2)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _main_diagonal_mutant(q, k, stride, group):
    lq, hq, d = q.shape
    lk = k.shape[0]
    out = np.zeros((hq, lq // stride, lk // stride))
    for h in range(hq):
        for t in range(stride):
            out[h] += q[t::stride, h, :] @ k[t::stride, h // group, :].T
    return out


def _wrong_group_mutant(q, k, stride, group):
    # h % Hkv instead of h // group: the other reading of repeat_interleave
    hkv = k.shape[1]
    qq = q.copy()
    out = np.zeros((q.shape[1], q.shape[0] // stride, k.shape[0] // stride))
    for h in range(q.shape[1]):
        out[h] = O.strided_scores(qq[:, h:h + 1], k[:, (h % hkv):(h % hkv) + 1], stride, 1)[0]
    return out


@pytest.mark.parametrize("mutant", [_main_diagonal_mutant, _wrong_group_mutant])
def test_scores_pin_rejects_mutants(mutant):
    q = _rand((32, 4, 8), 3)
    k = _rand((64, 2, 8), 4)
    ref = _brute_scores(q, k, 4, group=2)
    assert not np.allclose(mutant(q, k, 4, 2), ref, rtol=1e-6, atol=1e-6)


def test_constant_vectors_closed_form():
    s, d, a, b = 8, 16, 0.75, -1.5
    q = np.full((64, 1, d), a)
    k = np.full((128, 1, d), b)
    got = O.strided_scores(q, k, s, 1)
    np.testing.assert_allclose(got, s * d * a * b, rtol=0, atol=1e-12)


# ----------------------------------------------------------- O1 block sums

def test_stride1_block_sums_equal_blocked_dense_softmax():
    """s = 1: the estimate is the block-summed causal softmax of q k^T/sqrt(d),
    computed here with torch.softmax (bottom-right causal alignment)."""
    lq, lk, d, blk = 64, 96, 16, 16
    q = _rand((lq, 2, d), 5)
    k = _rand((lk, 1, d), 6)
    scale = 1.0 / math.sqrt(d)
    got = O.estimate_block_sums(q, k, stride=1, block=blk, est_scale=scale, group=2)
    o = lk - lq
    for h in range(2):
        logits = torch.from_numpy(q[:, h, :] @ k[:, 0, :].T * scale)
        mask = torch.arange(lk)[None, :] <= (torch.arange(lq)[:, None] + o)
        p = torch.softmax(logits.masked_fill(~mask, float("-inf")), dim=-1).numpy()
        ref = p.reshape(lq // blk, blk, lk // blk, blk).sum(axis=(1, 3))
        np.testing.assert_allclose(got[h], ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("stride,lq,lk", [(8, 256, 256), (4, 128, 512), (16, 256, 768)])
def test_block_sum_invariants(stride, lq, lk):
    blk = 128
    q = _rand((lq, 2, 32), 7)
    k = _rand((lk, 1, 32), 8)
    bs = O.estimate_block_sums(q, k, stride=stride, block=blk, est_scale=0.05, group=2)
    rb = blk // stride
    kh = (lk - lq) // blk
    np.testing.assert_allclose(bs.sum(axis=2), rb, rtol=1e-12)  # each row: rb rows of prob 1
    assert (bs >= 0).all()
    for i in range(lq // blk):
        assert (bs[:, i, i + kh + 1:] == 0).all()  # blocks beyond the causal diagonal


@pytest.mark.parametrize("chunk", [128, 256, 384, 4096])
def test_chunked_two_pass_equals_single_pass(chunk):
    lq, lk = 256, 1024
    q = _rand((lq, 4, 32), 9)
    k = _rand((lk, 2, 32), 10)
    kw = dict(stride=8, block=128, est_scale=1.0 / (8 * math.sqrt(32)), group=2)
    one = O.estimate_block_sums(q, k, **kw)
    two = O.estimate_block_sums_chunked(q, k, chunk_tokens=chunk, **kw)
    np.testing.assert_allclose(two, one, rtol=1e-12, atol=1e-14)


def test_merge_softmax_stats_mutant_rejected():
    """Dropping the exp(m_k - m) rescale must break the chunked invariant."""
    lq, lk = 128, 512
    q = _rand((lq, 1, 16), 11) * 3
    k = _rand((lk, 1, 16), 12) * 3
    kw = dict(stride=8, block=128, est_scale=0.1, group=1)
    one = O.estimate_block_sums(q, k, **kw)
    orig = O.xattn_oracle.merge_softmax_stats

    def bad(ms, ls):
        ms = np.stack(ms)
        return ms.max(axis=0), np.stack(ls).sum(axis=0)

    O.xattn_oracle.merge_softmax_stats = bad
    try:
        two = O.estimate_block_sums_chunked(q, k, chunk_tokens=128, **kw)
    finally:
        O.xattn_oracle.merge_softmax_stats = orig
    assert not np.allclose(two, one, rtol=1e-6)


# --------------------------------------------------------- O3 threshold

def _brute_min_subset(v, tau):
    n = len(v)
    total = sum(v)
    for size in range(n + 1):
        best = None
        for sub in itertools.combinations(range(n), size):
            if sum(v[j] for j in sub) >= tau * total:
                best = sub
                break
        if best is not None:
            return size
    return n


def test_threshold_select_minimum_cardinality_bruteforce():
    rng = np.random.default_rng(13)
    for trial in range(300):
        n = int(rng.integers(1, 11))
        v = (rng.integers(0, 64, size=n) / 64.0).tolist()  # dyadic: sums are exact
        if sum(v) == 0:
            continue
        tau = float(rng.choice([0.25, 0.5, 0.75, 0.9, 0.95]))
        keep = O.threshold_select_row(v, tau)
        m_star = _brute_min_subset(v, tau)
        assert keep.sum() == m_star, (v, tau)
        assert sum(np.asarray(v)[keep]) >= tau * sum(v)
        # kept items are the m* largest, ties broken toward the lower index
        order = sorted(range(n), key=lambda j: (-v[j], j))
        assert set(np.flatnonzero(keep)) == set(order[:m_star])


def test_threshold_special_cases():
    v = [0.1, 0.4, 0.2, 0.3]
    assert O.threshold_select_row(v, 1.0).all()
    assert O.threshold_select_row(v, 1.5).all()
    assert O.threshold_select_row(v, 1e-9).tolist() == [False, True, False, False]
    # equal values: lower index first
    assert O.threshold_select_row([1.0, 1.0, 1.0, 1.0], 0.5).tolist() == [True, True, False, False]
    # the cut is on the sum strictly before the item
    assert O.threshold_select_row([0.5, 0.25, 0.25], 0.75).tolist() == [True, True, False]


def test_topk_select_bruteforce():
    """Top-k keeps a k-subset of maximum sum; among maximum-sum subsets the
    one whose sorted index list is smallest (ties toward the lower index)."""
    rng = np.random.default_rng(17)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        v = (rng.integers(0, 8, size=n) / 8.0).tolist()  # dyadic, many ties
        k = int(rng.integers(0, n + 3))
        keep = O.topk_select_row(v, k)
        m = min(max(k, 0), n)
        assert keep.sum() == m
        best = max(itertools.combinations(range(n), m), key=lambda sub: (sum(v[j] for j in sub), [-j for j in sub]))
        assert set(np.flatnonzero(keep)) == set(best), (v, k)


def test_topk_special_cases_and_threshold_relation():
    v = [0.1, 0.4, 0.2, 0.3]
    assert O.topk_select_row(v, 0).tolist() == [False] * 4
    assert O.topk_select_row(v, 1).tolist() == [False, True, False, False]
    assert O.topk_select_row(v, 2).tolist() == [False, True, False, True]
    assert O.topk_select_row(v, 9).all()
    assert O.topk_select_row([1.0, 1.0, 1.0], 2).tolist() == [True, True, False]
    # the threshold rule keeps a prefix of the same order: top-k with k = its
    # count reproduces it
    rng = np.random.default_rng(18)
    for trial in range(200):
        w = rng.exponential(size=int(rng.integers(1, 40)))
        tau = float(rng.uniform(0.1, 0.99))
        keep = O.threshold_select_row(w, tau)
        assert (O.topk_select_row(w, int(keep.sum())) == keep).all()
    # top-k mode feeds the same aggregation and forcing as the threshold mode
    bs = np.zeros((2, 2, 4))
    bs[0, 1] = [0.1, 0.2, 0.3, 0.4]
    bs[1, 1] = [0.4, 0.3, 0.2, 0.1]
    sel = O.select_blocks(bs, kh=2, tau=0.9, group=2, mode=O.PER_KVHEAD, num_to_choose=1)
    # row 1: heads pick j=3 and j=0; ANY -> {0, 3}; forced sink 0 and diagonal 3
    assert sel["mask_kv"][0, 1].tolist() == [True, False, False, True]


def test_threshold_mutants_rejected():
    def le_mutant(v, tau):  # <= instead of <
        v = np.asarray(v, float)
        order = np.argsort(-v, kind="stable")
        c = np.concatenate([[0.0], np.cumsum(v[order])])
        keep = np.zeros(len(v), bool)
        keep[order] = c[:-1] <= tau * c[-1]
        return keep

    def asc_mutant(v, tau):  # ascending order
        v = np.asarray(v, float)
        order = np.argsort(v, kind="stable")
        c = np.concatenate([[0.0], np.cumsum(v[order])])
        keep = np.zeros(len(v), bool)
        keep[order] = c[:-1] < tau * c[-1]
        return keep

    v = [0.5, 0.25, 0.25]
    for mut in (le_mutant, asc_mutant):
        assert mut(v, 0.75).tolist() != [True, True, False]


def test_cumsum_is_left_to_right():
    """R5 relies on np.cumsum adding left to right in float64."""
    a = np.random.default_rng(14).random(5000) * np.logspace(-30, 3, 5000)
    s = 0.0
    ref = []
    for x in a:
        s += x
        ref.append(s)
    assert np.array_equal(np.cumsum(a), np.array(ref))


# ---------------------------------------------------- O4-O6 aggregation

def _bs_from_masks(mask_q, kh):
    """Block sums whose tau=0.99 threshold selection reproduces mask_q: the
    kept blocks of a row share 0.999 equally, the dropped ones share 0.001
    (every row must keep at least one block)."""
    hq, qb, kb = mask_q.shape
    bs = np.zeros(mask_q.shape)
    for h in range(hq):
        for i in range(qb):
            n = i + kh + 1
            keep = mask_q[h, i, :n]
            nk, nd = keep.sum(), n - keep.sum()
            assert nk >= 1
            bs[h, i, :n] = np.where(keep, 0.999 / nk, 0.001 / max(nd, 1))
    return bs


TAU_TOY = 0.99


def test_vote_needs_strict_majority():
    # Hkv = 2, G = 1, Qb = 2, Kh = 4: 4 votes per history block, > 2 needed.
    kh, qb = 4, 2
    kb = kh + qb
    mask_q = np.zeros((2, qb, kb), bool)
    # history block 1: 3 of 4 votes; block 2: exactly 2 of 4; block 3: 0; block 0: 1
    mask_q[0, 0, 1] = mask_q[0, 1, 1] = mask_q[1, 0, 1] = True
    mask_q[0, 0, 2] = mask_q[1, 1, 2] = True
    mask_q[1, 0, 0] = True
    for h in range(2):
        for i in range(qb):
            mask_q[h, i, i + kh] = True  # something in the current chunk
    bs = _bs_from_masks(mask_q, kh)
    sel = O.select_blocks(bs, kh=kh, tau=TAU_TOY, group=1, mode=O.CHUNK_VOTE)
    assert (sel["mask_q"] == mask_q).all()
    # block 0 and block Kh-1 = 3 forced; block 1 voted in; block 2 (50%) out
    assert sel["hist_sel"][:kh].tolist() == [True, True, False, True]
    assert sel["counts"] == (3, 4)
    eff = sel["mask_kv"]
    assert (eff[:, :, :kh] == np.array([1, 1, 0, 1], bool)).all()
    for i in range(qb):  # current chunk dense causal
        assert eff[:, i, kh:kh + i + 1].all() and not eff[:, i, kh + i + 1:].any()


def test_gqa_any_and_majority():
    # 2 kv groups of G = 3 q heads; one row (Qb = 1) over 3 allowed blocks
    # (Kh = 2): sink 0 and diagonal 2 are forced, block 1 is the one tested.
    kh, qb, kb = 2, 1, 3
    mask_q = np.zeros((6, qb, kb), bool)
    mask_q[:, 0, 2] = True
    mask_q[0, 0, 1] = True  # group 0: 1 of 3 heads
    mask_q[3, 0, 1] = mask_q[4, 0, 1] = True  # group 1: 2 of 3 heads
    bs = _bs_from_masks(mask_q, kh)
    any_ = O.select_blocks(bs, kh=kh, tau=TAU_TOY, group=3, mode=O.PER_KVHEAD, agg=O.AGG_ANY)
    maj = O.select_blocks(bs, kh=kh, tau=TAU_TOY, group=3, mode=O.PER_KVHEAD, agg=O.AGG_MAJORITY)
    assert (any_["mask_q"] == mask_q).all()
    assert any_["mask_kv"][:, 0, 1].tolist() == [True, True]
    assert maj["mask_kv"][:, 0, 1].tolist() == [False, True]
    assert any_["mask_kv"][:, 0, 0].all() and any_["mask_kv"][:, 0, 2].all()


def test_per_kvhead_forces_sink_and_diagonal():
    kh, qb, kb = 2, 2, 4
    bs = np.zeros((2, qb, kb))
    bs[:, :, 1] = 1.0  # all mass on block 1 (history), tau small -> only block 1 chosen
    for i in range(qb):
        bs[:, i, : i + kh + 1] += 1e-6
    sel = O.select_blocks(bs, kh=kh, tau=0.1, group=2, mode=O.PER_KVHEAD)
    eff = sel["mask_kv"][0]
    assert eff[0].tolist() == [True, True, True, False]  # sink 0, chosen 1, diagonal 2
    assert eff[1].tolist() == [True, True, False, True]  # diagonal 3
    assert sel["counts"] == (6, 3 + 4)


def test_sparse_current_chunk_vote_hand_worked():
    """Sparse-current chunk vote (R23) on a toy worked by hand: Hkv = G = 1,
    Qb = 2, Kh = 4, tau = 0.5.  Row 0 (blocks 0..4) = .05 .6 .05 .05 .25
    keeps block 1 only (the sum before the second-largest is .6 >= .5); row
    1 (blocks 0..5) = .05 .55 .05 .05 .1 .2 keeps block 1 only.  Votes: block
    1 has 2 of 2 (> 1), block 2 has 0; blocks 0 and Kh-1 = 3 are forced ->
    history 1 1 0 1.  Current chunk: row 0 sees block 4, its diagonal
    (forced); row 1 sees blocks 4 and 5: block 4 was not selected (the
    chunk-vote mode would keep it), block 5 is its diagonal."""
    kh, qb, kb = 4, 2, 6
    bs = np.zeros((1, qb, kb))
    bs[0, 0, :5] = [0.05, 0.6, 0.05, 0.05, 0.25]
    bs[0, 1, :6] = [0.05, 0.55, 0.05, 0.05, 0.1, 0.2]
    sel = O.select_blocks(bs, kh=kh, tau=0.5, group=1, mode=O.CHUNK_VOTE_SPARSE)
    assert sel["hist_sel"][:kh].tolist() == [True, True, False, True]
    assert sel["mask_kv"][0, 0].tolist() == [True, True, False, True, True, False]
    assert sel["mask_kv"][0, 1].tolist() == [True, True, False, True, False, True]
    assert sel["counts"] == (8, 11)
    dense = O.select_blocks(bs, kh=kh, tau=0.5, group=1, mode=O.CHUNK_VOTE)
    assert dense["mask_kv"][0, 1].tolist() == [True, True, False, True, True, True]


@pytest.mark.parametrize("agg", [O.AGG_ANY, O.AGG_MAJORITY])
def test_sparse_current_chunk_vote_is_vote_history_plus_kvhead_current(agg):
    """On random block sums: history columns and hist_sel equal the chunk
    vote's, current-chunk columns equal per-KV-head mode's; with no history
    the whole result (mask and counts) is per-KV-head mode's."""
    rng = np.random.default_rng(31)
    for kh, qb, hq, g in ((5, 3, 4, 2), (0, 4, 6, 3), (1, 2, 2, 1), (12, 2, 8, 4)):
        kb = kh + qb
        bs = rng.exponential(1.0, size=(hq, qb, kb))
        for tau in (0.3, 0.8):
            sp = O.select_blocks(bs, kh=kh, tau=tau, group=g, mode=O.CHUNK_VOTE_SPARSE, agg=agg)
            cv = O.select_blocks(bs, kh=kh, tau=tau, group=g, mode=O.CHUNK_VOTE, agg=agg)
            pk = O.select_blocks(bs, kh=kh, tau=tau, group=g, mode=O.PER_KVHEAD, agg=agg)
            assert (sp["hist_sel"] == cv["hist_sel"]).all()
            assert (sp["mask_kv"][:, :, :kh] == cv["mask_kv"][:, :, :kh]).all()
            assert (sp["mask_kv"][:, :, kh:] == pk["mask_kv"][:, :, kh:]).all()
            if kh == 0:
                assert (sp["mask_kv"] == pk["mask_kv"]).all() and sp["counts"] == pk["counts"]
            assert sp["counts"] == (int(sp["mask_kv"].sum()), pk["counts"][1])


# ------------------------------------------------------------ O7 / O8

def _sdpa_causal(q, k, v, scale):
    """torch float64 scaled_dot_product_attention, bottom-right causal, GQA."""
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(g, dim=0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(g, dim=0)
    mask = torch.arange(lk)[None, :] <= (torch.arange(lq)[:, None] + (lk - lq))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    logits = (qt @ kt.transpose(-1, -2)) * scale
    lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=-1)
    return out.permute(1, 0, 2).numpy(), lse.numpy()


@pytest.mark.parametrize("mode", [O.PER_KVHEAD, O.CHUNK_VOTE, O.CHUNK_VOTE_SPARSE])
def test_tau_one_is_full_causal_attention(mode):
    lq, lk, hq, hkv, d = 256, 640, 4, 2, 32
    q = _rand((lq, hq, d), 20)
    k = _rand((lk, hkv, d), 21)
    v = _rand((lk, hkv, d), 22)
    res = O.prefill(q, k, v, [0, lq], [0, lk], num_kv_heads=hkv, stride=8, threshold=1.0,
                    mode=mode, kv_chunk_tokens=256)
    ref_o, ref_l = _sdpa_causal(q, k, v, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(res["out"], ref_o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(res["lse"], ref_l, rtol=1e-12, atol=1e-12)
    assert res["mask_kv"][0].sum() == hkv * sum(i + (lk - lq) // 128 + 1 for i in range(lq // 128))


def test_chunk_vote_without_history_is_dense_causal():
    lq = lk = 384
    q = _rand((lq, 2, 16), 23)
    k = _rand((lk, 1, 16), 24)
    v = _rand((lk, 1, 16), 25)
    res = O.prefill(q, k, v, [0, lq], [0, lk], num_kv_heads=1, stride=8, threshold=0.3,
                    mode=O.CHUNK_VOTE)
    ref_o, _ = _sdpa_causal(q, k, v, 0.25)
    np.testing.assert_allclose(res["out"], ref_o, rtol=1e-10, atol=1e-12)
    assert tuple(res["counts"][0]) == (0, 0)


def test_sparse_attention_matches_masked_sdpa():
    lq, lk, hq, hkv, d = 256, 512, 2, 1, 16
    q = _rand((lq, hq, d), 26)
    k = _rand((lk, hkv, d), 27)
    v = _rand((lk, hkv, d), 28)
    rng = np.random.default_rng(29)
    mask = rng.random((hkv, 2, 4)) < 0.5
    mask[:, 0, 2] = mask[:, 1, 3] = True  # diagonals
    out, lse = O.sparse_attention(q, k, v, mask, softmax_scale=0.3, group=2)
    tok = np.zeros((lq, lk), bool)
    for x in range(lq):
        for y in range(lk):
            tok[x, y] = mask[0, x // 128, y // 128] and y <= x + (lk - lq)
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).expand(hq, -1, -1)
    vt = torch.from_numpy(v).permute(1, 0, 2).expand(hq, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(tok), scale=0.3)
    np.testing.assert_allclose(out, ref.permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_merge_of_disjoint_halves_equals_unsplit():
    lq, lk, d = 128, 512, 16
    q = _rand((lq, 2, d), 30)
    k = _rand((lk, 1, d), 31)
    v = _rand((lk, 1, d), 32)
    full = np.ones((1, 1, 4), bool)
    o_all, l_all = O.sparse_attention(q, k, v, full, softmax_scale=0.25, group=2)
    o_a, l_a = O.sparse_attention(q, k, v, full, softmax_scale=0.25, group=2, key_range=(0, 200))
    o_b, l_b = O.sparse_attention(q, k, v, full, softmax_scale=0.25, group=2, key_range=(200, lk))
    o_m, l_m = O.merge_attention(o_a, l_a, o_b, l_b)
    np.testing.assert_allclose(o_m, o_all, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(l_m, l_all, rtol=1e-12, atol=1e-12)
    # an empty side contributes nothing
    o_e, l_e = O.merge_attention(o_all, l_all, np.zeros_like(o_all), np.full_like(l_all, -np.inf))
    np.testing.assert_allclose(o_e, o_all, rtol=0, atol=0)
    np.testing.assert_allclose(l_e, l_all, rtol=0, atol=0)


def test_pages_order_equals_single_masked_pass():
    lq, lk = 256, 1024
    q = _rand((lq, 4, 16), 33)
    k = _rand((lk, 2, 16), 34)
    v = _rand((lk, 2, 16), 35)
    kw = dict(num_kv_heads=2, stride=8, threshold=0.6, mode=O.CHUNK_VOTE, kv_chunk_tokens=256)
    a = O.prefill(q, k, v, [0, lq], [0, lk], **kw)
    b = O.prefill(q, k, v, [0, lq], [0, lk], pages_order=True, **kw)
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ O9 and layout

def test_density_matches_pages_example():
    with open(os.path.join(GOLDEN, "density_stats_example.json")) as f:
        g = json.load(f)
    ov = g["overall"]
    dens = O.density([(ov["total_selected_blocks"], ov["total_available_blocks"])])
    assert round(dens, 2) == ov["overall_density_2dp"]
    dl = g["debug_line"]
    assert round(100 * O.density([(dl["selected"], dl["available"])]), 1) == dl["chunk_density_percent_1dp"]
    rbk = g["reshaped_block"]
    assert rbk["block_size"] // rbk["stride"] == rbk["reshaped_block_size"]


def test_varlen_and_paged_worked_examples():
    with open(os.path.join(GOLDEN, "paged_attention_examples.json")) as f:
        g = json.load(f)
    vl = g["varlen"]
    cu_q = O.cu_seqlens(vl["q_lengths"])
    cu_k = O.cu_seqlens(vl["k_lengths"])
    assert cu_q == vl["cu_seq_lens_q"] and cu_k == vl["cu_seq_lens_k"]
    assert O.request_index(cu_q) == vl["q_request_index"]
    assert O.request_index(cu_k) == vl["k_request_index"]
    pg = g["paged"]
    bt = pg["block_table"]
    bsz = pg["block_size"]
    for b, n in enumerate(pg["cache_seqlens"]):
        # the cached tokens plus the new one touch exactly the allocated pages
        pages = sorted({O.paged_location(bt[b], t, bsz)[0] for t in range(n + 1)}, key=bt[b].index)
        assert pages == pg["allocated_pages"][str(b)]
        assert O.paged_location(bt[b], n, bsz)[0] == pg["new_token_page"][str(b)]
    with pytest.raises(IndexError):
        O.paged_location(bt[0], 32, bsz)  # -1 page
    # gather through a shuffled table reproduces the logical sequence
    cache = np.arange(7 * bsz, dtype=float).reshape(7, bsz, 1, 1)
    got = O.gather_paged(cache, bt[2], 70, bsz)[:, 0, 0]
    exp = np.concatenate([cache[3, :, 0, 0], cache[5, :, 0, 0], cache[6, :6, 0, 0]])
    assert np.array_equal(got, exp)


def test_well_separated_family_has_wide_margins():
    from workloads import make_well_separated
    w = make_well_separated("ws", seed=101, hq=4, hkv=2, d=64, lq=[512], lk=[1024],
                            dtype=torch.float32)
    res = O.prefill(w.q, w.k, w.v, w.cu_q, w.cu_k, num_kv_heads=2, stride=8, threshold=0.9,
                    attention=False)
    bs = res["block_sums"][0]
    kh = (1024 - 512) // 128
    margins = [O.selection_margin(bs[h, i, : i + kh + 1], 0.9)
               for h in range(bs.shape[0]) for i in range(bs.shape[1])]
    # most rows clear the 5e-3 margin; none is within fp32 rounding of a flip
    assert np.mean(np.array(margins) >= 5e-3) >= 0.7
    assert min(margins) >= 1e-3


def test_selection_margin_hand_computed():
    """selection_margin against values worked out by hand.  v = (1/8, 1/2,
    1/8, 1/4) sorts to 1/2, 1/4, 1/8, 1/8 (indices 1, 3, 0, 2) with
    cumulative sums C = 0, 1/2, 3/4, 7/8, 1 and T = 1."""
    v = [0.125, 0.5, 0.125, 0.25]
    # tau = 0.7: keeps 2 (C1 = 1/2 < 0.7 <= C2 = 3/4); margins 0.2, 0.05 and
    # the gap 1/4 - 1/8 at the cut -> 0.05
    assert O.selection_margin(v, 0.7) == pytest.approx(0.05, abs=1e-12)
    # tau = 0.5: keeps 1; C1 = 1/2 sits exactly on tau*T -> 0
    assert O.selection_margin(v, 0.5) == 0.0
    # tau = 0.3: keeps 1; margins 0.3, 0.2, gap 1/4 -> 0.2
    assert O.selection_margin(v, 0.3) == pytest.approx(0.2, abs=1e-12)
    # equal values at the cut: the order there is a tie -> 0
    assert O.selection_margin([0.25] * 4, 0.6) == 0.0
    # everything kept: only the distance below the threshold counts
    assert O.selection_margin([1.0], 0.9) == pytest.approx(0.9)
    assert O.selection_margin(v, 1.0) == np.inf
    # relative: scaling the row leaves it unchanged
    assert O.selection_margin([8 * x for x in v], 0.7) == pytest.approx(0.05, abs=1e-12)


def test_selection_margin_bounds_every_flip():
    """Any perturbation whose total size sum|dv| stays below half the margin
    times T leaves the kept set unchanged (the property the GPU mask checks
    rely on); moving just over the margin times T from one item to another
    (total size 2.1 m T) changes it, so the bound is tight up to a factor 4."""
    rng = np.random.default_rng(17)
    for trial in range(300):
        n = int(rng.integers(2, 14))
        v = rng.exponential(1.0, size=n)
        tau = float(rng.choice([0.3, 0.5, 0.7, 0.9, 0.95]))
        m = O.selection_margin(v, tau)
        keep = O.threshold_select_row(v, tau)
        t = v.sum()
        for _ in range(20):
            d = rng.standard_normal(n)
            d *= 0.49 * m * t / np.abs(d).sum()
            d = np.maximum(d, -v)  # values stay >= 0
            assert (O.threshold_select_row(v + d, tau) == keep).all(), (v, tau, m)
        if 0 < m < np.inf:
            k = int(keep.sum())
            flipped = False
            for a in range(n):
                for b in range(n):
                    if a == b or v[b] < 1.05 * m * t:
                        continue
                    w = v.copy()
                    w[a] += 1.05 * m * t
                    w[b] -= 1.05 * m * t
                    if not (O.threshold_select_row(w, tau) == keep).all():
                        flipped = True
                        break
                if flipped:
                    break
            assert flipped, (v, tau, m, k)
