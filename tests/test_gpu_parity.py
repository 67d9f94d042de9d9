"""GPU parity of every stage (and the whole path) against the float64 oracle.

All calls go through the C ABI of libxattn.so.  Inputs are the seeded
synthetic workloads; both sides see the identical fp32 / bf16 values.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_strided_amd as X
import oracle as O
from tests import metrics
from tests.gpu_util import (Run, assert_attention_close, assert_block_sums_close, assert_gapped, check_selection,
                            sample_rows, say)
from workloads import make_random, make_well_separated, make_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


EST_CASES = {
    "bf16_s8_d128_varlen": dict(hq=4, hkv=2, d=128, lq=[2048, 384], lk=[4096, 1024], stride=8),
    "bf16_s16_d128_gqa4": dict(hq=4, hkv=1, d=128, lq=[2048], lk=[3072], stride=16),
    "bf16_s4_d64": dict(hq=2, hkv=2, d=64, lq=[1024], lk=[2048], stride=4),
    "bf16_paged_3seq": dict(hq=4, hkv=2, d=128, lq=[512, 256, 128], lk=[2048, 256, 1536], stride=8,
                            paged=True),
    "bf16_empty_seqs": dict(hq=2, hkv=1, d=128, lq=[256, 0, 128, 0], lk=[512, 256, 128, 0], stride=8),
    "f32_s8_d64": dict(hq=2, hkv=1, d=64, lq=[512], lk=[1024], stride=8, dtype=torch.float32),
    # the launcher's table of tiles with work holds up to 64 sequences; 65
    # and more use one workgroup per grid tile
    "bf16_64_seqs": dict(hq=2, hkv=1, d=64, lq=[128 * (1 + i % 2) for i in range(64)],
                         lk=[128 * (2 + i % 3) for i in range(64)], stride=8),
    "bf16_65_seqs": dict(hq=2, hkv=1, d=64, lq=[128 * (1 + i % 2) for i in range(65)],
                         lk=[128 * (2 + i % 3) for i in range(65)], stride=8),
    # large enough (>= 256 tiles of 256 x 256) for the big-tile GEMM path:
    # ragged rows/columns, causal tiles, two sequences
    "bf16_big_s8_varlen": dict(hq=16, hkv=4, d=128, lq=[2432, 640], lk=[8192, 1024], stride=8),
    "bf16_big_s16_d64": dict(hq=16, hkv=8, d=64, lq=[4096], lk=[65536], stride=16),
    # 640-block rows at stride 4: the block-sum kernel that re-reads the partials
    "bf16_s4_long_rows": dict(hq=2, hkv=1, d=64, lq=[256], lk=[81920], stride=4),
    "f32_s16_d128_paged": dict(hq=2, hkv=2, d=128, lq=[256, 128], lk=[512, 384], stride=16,
                               dtype=torch.float32, paged=True),
}


def _make(name, seed=11, **over):
    kw = dict(EST_CASES[name])
    kw.update(over)
    return make_random(name, seed=seed, **kw)


@pytest.mark.parametrize("name", list(EST_CASES))
def test_estimate_block_sums(name):
    w = _make(name)
    r = Run(w)
    say("estimate " + name)
    bs = r.estimate()
    ref = r.oracle(attention=False)["block_sums"]
    assert_block_sums_close(bs, ref, w.stride, name)


def test_estimate_tiny_fp32_workload():
    w = make_workload("tiny_causal_fp32_1k")
    r = Run(w)
    say("estimate tiny fp32")
    bs = r.estimate()
    ref = r.oracle(attention=False)["block_sums"]
    assert_block_sums_close(bs, ref, w.stride, "tiny")


@pytest.mark.parametrize("mode", ["per_kvhead", "chunk_vote", "chunk_vote_sparse"])
@pytest.mark.parametrize("agg", ["any", "majority"])
@pytest.mark.parametrize("tau", [0.0, 0.5, 0.9, 0.95, 1.0])
def test_select_matches_oracle_bit_exact(mode, agg, tau):
    """The select kernels fed the oracle's block sums (rounded to fp32) make
    the same float64 decisions as the oracle on those fp32 values."""
    w = make_random("sel", seed=21, hq=8, hkv=2, d=64, lq=[512, 256, 0], lk=[2048, 256, 384],
                    dtype=torch.float32, stride=8, select_mode=mode, group_agg=agg)
    r = Run(w, threshold=tau)
    bs64 = r.oracle(attention=False)["block_sums"]
    bs32 = bs64.astype(np.float32)
    say("select %s %s %g" % (mode, agg, tau))
    mask, hist, counts = r.select(torch.from_numpy(bs32))
    # oracle selection on the same fp32 values
    for b in range(w.batch):
        lq, lk = w.lens(b)
        qb, kb = lq // 128, lk // 128
        if qb == 0:
            assert (mask[b].cpu() == 0).all()
            assert counts[b].tolist() == [0, 0]
            continue
        sel = O.select_blocks(bs32[b, :, :qb, :kb].astype(np.float64), kh=(lk - lq) // 128, tau=r.tau,
                              group=w.num_q_heads // w.num_kv_heads, mode=mode, agg=agg)
        m = mask[b].cpu().numpy().astype(bool)
        assert (m[:, :qb, :kb] == sel["mask_kv"]).all(), "mask mismatch seq %d" % b
        assert not m[:, qb:, :].any() and not m[:, :, kb:].any()
        assert (hist[b, :kb].cpu().numpy().astype(bool) == sel["hist_sel"]).all()
        assert tuple(counts[b].tolist()) == sel["counts"]


@pytest.mark.parametrize("case", [
    dict(hq=16, hkv=1, lq=[512], lk=[8192]),        # 16 q heads per group: the fused kernel's widest group
    dict(hq=8, hkv=1, lq=[256], lk=[131072]),       # 1024-block rows x 8 heads: two-kernel path (LDS)
    dict(hq=32, hkv=1, lq=[256], lk=[16384]),       # 32 q heads per group: two-kernel path (group size)
    dict(hq=1, hkv=1, lq=[128, 256], lk=[384000, 1024]),  # 3000-block rows: 4096-key sort
])
@pytest.mark.parametrize("mode", ["per_kvhead", "chunk_vote", "chunk_vote_sparse"])
def test_select_wide_rows_and_groups(case, mode):
    """Selection on seeded block sums (exponential, with ties) for row widths
    and group sizes on both sides of the fused kernel's limits."""
    w = make_random("selw", seed=23, d=64, dtype=torch.float32, stride=8, select_mode=mode, **case)
    r = Run(w, threshold=0.9)
    rng = np.random.default_rng(24)
    bs32 = rng.exponential(1.0, size=(r.B, r.hq, r.max_qb, r.max_kb)).astype(np.float32)
    bs32[..., ::7] = bs32[..., 3:4]  # repeated values: index order decides
    say("select wide %s %s" % (case, mode))
    mask, hist, counts = r.select(torch.from_numpy(bs32))
    for b in range(w.batch):
        lq, lk = w.lens(b)
        qb, kb = lq // 128, lk // 128
        sel = O.select_blocks(bs32[b, :, :qb, :kb].astype(np.float64), kh=(lk - lq) // 128, tau=r.tau,
                              group=w.num_q_heads // w.num_kv_heads, mode=mode)
        m = mask[b].cpu().numpy().astype(bool)
        assert (m[:, :qb, :kb] == sel["mask_kv"]).all(), "mask mismatch seq %d" % b
        assert not m[:, qb:, :].any() and not m[:, :, kb:].any()
        assert (hist[b, :kb].cpu().numpy().astype(bool) == sel["hist_sel"]).all()
        assert tuple(counts[b].tolist()) == sel["counts"]


@pytest.mark.parametrize("k", [1, 3, 9, 5000])
@pytest.mark.parametrize("case", [
    dict(hq=8, hkv=2, lq=[512, 256], lk=[2048, 256]),  # fused kernel
    dict(hq=32, hkv=1, lq=[256], lk=[16384]),           # two-kernel path (group size)
])
@pytest.mark.parametrize("mode", ["per_kvhead", "chunk_vote", "chunk_vote_sparse"])
def test_select_topk(k, case, mode):
    """Top-k rule (num_to_choose) on seeded block sums with ties, both
    kernel paths, k below, inside and above the row widths."""
    w = make_random("topk", seed=25, d=64, dtype=torch.float32, stride=8, select_mode=mode, **case)
    r = Run(w, threshold=0.9, num_to_choose=k)
    rng = np.random.default_rng(26)
    bs32 = rng.exponential(1.0, size=(r.B, r.hq, r.max_qb, r.max_kb)).astype(np.float32)
    bs32[..., ::5] = bs32[..., 2:3]
    say("select top-%d %s %s" % (k, case, mode))
    mask, hist, counts = r.select(torch.from_numpy(bs32))
    for b in range(w.batch):
        lq, lk = w.lens(b)
        qb, kb = lq // 128, lk // 128
        sel = O.select_blocks(bs32[b, :, :qb, :kb].astype(np.float64), kh=(lk - lq) // 128, tau=r.tau,
                              group=w.num_q_heads // w.num_kv_heads, mode=mode, num_to_choose=k)
        m = mask[b].cpu().numpy().astype(bool)
        assert (m[:, :qb, :kb] == sel["mask_kv"]).all(), "mask mismatch seq %d" % b
        assert (hist[b, :kb].cpu().numpy().astype(bool) == sel["hist_sel"]).all()
        assert tuple(counts[b].tolist()) == sel["counts"]


def test_select_ties_and_zeros():
    """Equal values (index order decides) and zero blocks."""
    w = make_random("ties", seed=22, hq=2, hkv=1, d=64, lq=[256], lk=[1024], dtype=torch.float32,
                    select_mode="per_kvhead")
    r = Run(w, threshold=0.5)
    bs = np.zeros((1, 2, 2, 8), dtype=np.float32)
    bs[0, 0, 0, :7] = 0.25
    bs[0, 0, 1, :8] = [0.5, 0.0, 0.5, 0.5, 0.0, 1.0, 0.25, 0.25]
    bs[0, 1, 0, :7] = [0.0] * 6 + [1.0]
    bs[0, 1, 1, :8] = 1.0 / 8
    mask, hist, counts = r.select(torch.from_numpy(bs))
    sel = O.select_blocks(bs[0].astype(np.float64), kh=6, tau=r.tau, group=2, mode="per_kvhead")
    assert (mask[0].cpu().numpy().astype(bool) == sel["mask_kv"]).all()
    assert tuple(counts[0].tolist()) == sel["counts"]


ATTN_CASES = {
    "bf16_d128_gqa2_varlen": dict(hq=4, hkv=2, d=128, lq=[512, 256], lk=[1024, 256]),
    "bf16_d64_gqa1": dict(hq=2, hkv=2, d=64, lq=[384], lk=[896]),
    "bf16_d128_gqa2_causal": dict(hq=4, hkv=2, d=128, lq=[1280], lk=[1280]),
    "bf16_d64_gqa2_varlen": dict(hq=4, hkv=2, d=64, lq=[640, 128], lk=[1408, 384]),
    "bf16_paged": dict(hq=4, hkv=1, d=128, lq=[256, 128], lk=[768, 640], paged=True),
    "f32_d64": dict(hq=2, hkv=1, d=64, lq=[256], lk=[512], dtype=torch.float32),
    # 192 (q block, head) rows: each row's key tiles in 5 parts of up to 16
    # tiles (a count that is not a power of two, several tiles per part)
    "f32_d64_gqa3_5parts": dict(hq=6, hkv=2, d=64, lq=[2048, 1024], lk=[2560, 1024], dtype=torch.float32),
}


@pytest.mark.parametrize("name", list(ATTN_CASES))
@pytest.mark.parametrize("mask_kind", ["random", "dense", "diag"])
def test_sparse_attention(name, mask_kind):
    """Single sequences much longer than a CU's share of the launch are split
    into up to 3 parts per row and merged; "diag" (only the diagonal block)
    leaves the leading parts of split rows empty."""
    w = make_random(name, seed=31, **ATTN_CASES[name])
    r = Run(w)
    rng = np.random.default_rng(5)
    mask = np.zeros((r.B, r.hkv, r.max_qb, r.max_kb), dtype=np.uint8)
    for b in range(w.batch):
        lq, lk = w.lens(b)
        kh = (lk - lq) // 128
        for i in range(lq // 128):
            n = i + kh + 1
            if mask_kind == "random":
                row = rng.random((r.hkv, n)) < 0.5
            elif mask_kind == "dense":
                row = np.ones((r.hkv, n), bool)
            else:
                row = np.zeros((r.hkv, n), bool)
            row[:, i + kh] = True
            mask[b, :, i, :n] = row
    mask_t = torch.from_numpy(mask)
    say("attention %s %s" % (name, mask_kind))
    out, lse = r.attend(mask_t)
    ref_o, ref_l = r.oracle_attention(mask_t)
    assert_attention_close(out, lse, ref_o, ref_l, w.dtype, label=name)


@pytest.mark.parametrize("profile", ["rising", "falling", "jump"])
def test_attention_running_max_moves(profile):
    """Keys whose scale changes along the sequence, so that the running max
    of a row moves by large steps on many tiles ("rising": 0.25x to 4x),
    stays at the first tiles' level with later probabilities tiny
    ("falling"), or jumps once in the middle ("jump": 8x over a few blocks,
    0.5x elsewhere); dense causal rows of up to 2560 keys."""
    import dataclasses
    w = make_random("maxmove_" + profile, seed=37, hq=4, hkv=2, d=128, lq=[512], lk=[2560])
    n = w.k.shape[0]
    pos = torch.arange(n, dtype=torch.float32) / n
    if profile == "rising":
        sc = 0.25 + 3.75 * pos
    elif profile == "falling":
        sc = 4.0 - 3.75 * pos
    else:
        sc = torch.where((pos > 0.45) & (pos < 0.5), torch.tensor(8.0), torch.tensor(0.5))
    w = dataclasses.replace(w, k=(w.k.float() * sc[:, None, None]).to(w.dtype))
    r = Run(w)
    mask_t = torch.ones((r.B, r.hkv, r.max_qb, r.max_kb), dtype=torch.uint8)
    say("attention running max %s" % profile)
    out, lse = r.attend(mask_t)
    ref_o, ref_l = r.oracle_attention(mask_t)
    assert_attention_close(out, lse, ref_o, ref_l, w.dtype, label="running max " + profile)


@pytest.mark.parametrize("mask_kind", ["dense", "random", "mixed"])
def test_attention_head_tail_split(mask_kind):
    """Two sequences whose 32 q blocks x 8 kv heads = 256 workgroups fill a
    256-CU launch in one round, rows of 61..86 key blocks.  The head length
    comes from the rows' block lists: 98% of the per-CU share of the listed
    blocks plus two ("dense": 73.5 blocks per CU, 75-block heads); longer
    rows queue the rest as a tail part, which the split merge combines, and
    rows no longer than the head are done whole by their head part
    ("random" keeps 70% of every row: shorter rows and shorter heads;
    "mixed": dense rows beside rows keeping 20%, in one launch).
    Sampled rows (first and last of every q block) against the oracle."""
    w = make_random("head_tail", seed=41, hq=16, hkv=8, d=128, lq=[2048, 2048],
                    lk=[2048 + 128 * 60, 2048 + 128 * 70])
    r = Run(w)
    rng = np.random.default_rng(9)
    mask = np.zeros((r.B, r.hkv, r.max_qb, r.max_kb), dtype=np.uint8)
    for b in range(w.batch):
        lq, lk = w.lens(b)
        kh = (lk - lq) // 128
        for i in range(lq // 128):
            n = i + kh + 1
            if mask_kind == "dense" or (mask_kind == "mixed" and i % 2 == 0):
                row = np.ones((r.hkv, n), bool)
            else:
                row = rng.random((r.hkv, n)) < (0.7 if mask_kind == "random" else 0.2)
            row[:, i + kh] = True
            mask[b, :, i, :n] = row
    mask_t = torch.from_numpy(mask)
    rows, idx = sample_rows(w, per_seq=24)
    say("attention head/tail %s" % mask_kind)
    out, lse = r.attend(mask_t)
    ref_o, ref_l = r.oracle_attention(mask_t, rows=rows)
    assert_attention_close(out, lse, ref_o, ref_l, w.dtype, rows_idx=idx, label="head/tail " + mask_kind)
    # the tails are drawn from a counter the plan clears and each launch
    # resets at its end: three launches on one plan give the same bits
    md = mask_t.to("cuda", torch.uint8).contiguous()
    X.xattn_attn_plan(r.shape, r.params, r.v, md, r.ws)
    for _ in range(3):
        o2 = torch.full_like(r.q, float("nan"))
        l2 = torch.full((r.hq, r.shape.total_q), float("nan"), device="cuda")
        X.xattn_attn_run(r.shape, r.params, r.q, r.k, r.v, md, o2, l2, r.ws)
        torch.cuda.synchronize()
        assert torch.equal(o2.cpu(), out.cpu()) and torch.equal(l2.cpu(), lse.cpu()), "repeated launch differs"


@pytest.mark.parametrize("name", ["bf16_d128_gqa2_varlen", "f32_d64"])
def test_kernel_timing_hook(name):
    """While the hook is on, each attention call records one event pair around
    its attention kernel (not the merges after it); off, nothing is recorded;
    the outputs are those of an untimed call."""
    import block_sparse_attention_strided_amd as X
    w = make_random(name, seed=33, **ATTN_CASES[name])
    r = Run(w)
    mask_t = torch.ones((r.B, r.hkv, r.max_qb, r.max_kb), dtype=torch.uint8)
    out, lse = r.attend(mask_t)
    md = mask_t.to("cuda").contiguous()
    o2 = torch.full_like(r.q, float("nan"))
    l2 = torch.full((r.hq, r.shape.total_q), float("nan"), device="cuda")
    X.xattn_attn_plan(r.shape, r.params, r.v, md, r.ws)
    X.xattn_kernel_timing(True)
    try:
        for _ in range(3):
            X.xattn_attn_run(r.shape, r.params, r.q, r.k, r.v, md, o2, l2, r.ws)
        total, n = X.xattn_kernel_timing_read()
        assert n == 3 and total > 0.0, (total, n)
        assert X.xattn_kernel_timing_read() == (0.0, 0)
    finally:
        X.xattn_kernel_timing(False)
    assert torch.equal(o2.cpu(), out.cpu()) and torch.equal(l2.cpu(), lse.cpu())
    X.xattn_attn_run(r.shape, r.params, r.q, r.k, r.v, md, o2, l2, r.ws)
    torch.cuda.synchronize()
    assert X.xattn_kernel_timing_read() == (0.0, 0)


def test_merge_attention():
    import block_sparse_attention_strided_amd as X
    rng = np.random.default_rng(7)
    rows, heads, d = 300, 3, 128
    oa = rng.standard_normal((rows, heads, d))
    ob = rng.standard_normal((rows, heads, d))
    la = rng.standard_normal((heads, rows)) * 3
    lb = rng.standard_normal((heads, rows)) * 3
    la[0, :10] = -np.inf
    lb[1, :10] = -np.inf
    la[2, :5] = lb[2, :5] = -np.inf
    ref_o, ref_l = O.merge_attention(oa, la, ob, lb)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    o = torch.empty((rows, heads, d), device="cuda")
    l_ = torch.empty((heads, rows), device="cuda")
    say("merge")
    X.xattn_merge_attn(t(oa), t(la), t(ob), t(lb), o, l_)
    torch.cuda.synchronize()
    np.testing.assert_allclose(o.cpu().numpy(), ref_o, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(l_.cpu().numpy(), ref_l, rtol=1e-6, atol=1e-5)


def _prefill_and_check(w, rows=None, rows_idx=None, exact=False, label=""):
    """Whole path against the oracle: block sums within tolerance; masks under
    the margin rule of check_selection (bit-exact everywhere with exact=True);
    attention against the oracle evaluated on the GPU's own mask."""
    r = Run(w)
    say("prefill " + label)
    out, lse, counts, aux = r.prefill()
    ref = r.oracle(attention=False)
    assert_block_sums_close(aux["block_sums"], ref["block_sums"], w.stride, label)
    mism, soft, firm = check_selection(r, ref, aux["block_sums"], aux["mask_kv"], aux["hist_sel"], label)
    say("  mask mismatch fraction %.4g (%d soft / %d firm rows), counts %s vs %s" % (
        mism, soft, firm, counts.tolist(), ref["counts"].tolist()))
    if exact:
        assert mism == 0.0, "%s: mask mismatch fraction %.4g" % (label, mism)
        assert (counts.cpu().numpy() == ref["counts"]).all()
    ref_o, ref_l = r.oracle_attention(aux["mask_kv"], rows=rows)
    do, dl = assert_attention_close(out, lse, ref_o, ref_l, w.dtype, rows_idx=rows_idx, label=label)
    metrics.record("prefill " + label, density=O.density(counts.cpu().tolist()), max_dout=float(do),
                   max_dlse=float(dl))
    return mism, counts, aux


def test_prefill_tiny_fp32():
    _prefill_and_check(make_workload("tiny_causal_fp32_1k"), label="tiny fp32")


def test_prefill_qwen06_4k():
    _prefill_and_check(make_workload("qwen3_0p6b_4k"), label="4k")


def test_prefill_chunk32k_sampled():
    w = make_workload("chunked_prefill_32k")
    rows, idx = sample_rows(w, per_seq=64)
    _prefill_and_check(w, rows=rows, rows_idx=idx, label="32k")


@pytest.mark.parametrize("nseq, mode", [(70, "chunk_vote"), (150, "chunk_vote"), (150, "per_kvhead")])
def test_prefill_many_sequences(nseq, mode):
    """Batches past the planners' tables: more sequences than the estimate's
    per-sequence tile table holds (64; the GEMM then numbers its workgroups
    over the whole grid) and, at 150 sequences, more (sequence, q block) rows
    than the attention's order table (256; the kernel's default order, no
    split rows).  Sequences of 2-3 q blocks over 0-4 history blocks."""
    rng = np.random.default_rng(nseq)
    lq = [128 * int(x) for x in rng.integers(2, 4, nseq)]
    lk = [a + 128 * int(x) for a, x in zip(lq, rng.integers(0, 5, nseq))]
    w = make_random("many%d" % nseq, seed=61 + nseq, hq=4, hkv=2, d=64, lq=lq, lk=lk, select_mode=mode)
    rows, idx = sample_rows(w, per_seq=8)
    _prefill_and_check(w, rows=rows, rows_idx=idx, label="%d sequences %s" % (nseq, mode))


def _random_config(seed):
    """One seeded draw over the path's parameters: heads and group, head
    dim, stride, selection mode, group aggregation, dtype, paging, one to
    three sequences of 1-4 q blocks over 0-8 history blocks, and a threshold
    in [0.5, 0.99]."""
    rng = np.random.default_rng(seed)
    hq, hkv = [(2, 1), (4, 2), (6, 2), (8, 2), (4, 4), (8, 1)][rng.integers(6)]
    nseq = int(rng.integers(1, 4))
    lq = [128 * int(x) for x in rng.integers(1, 5, nseq)]
    lk = [a + 128 * int(x) for a, x in zip(lq, rng.integers(0, 9, nseq))]
    dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
    return dict(hq=hq, hkv=hkv, d=int(rng.choice([64, 128])), lq=lq, lk=lk, dtype=dtype,
                stride=int(rng.choice([4, 8, 16])),
                select_mode=str(rng.choice(["per_kvhead", "chunk_vote", "chunk_vote_sparse"])),
                group_agg=str(rng.choice(["any", "majority"])), paged=bool(rng.random() < 0.4),
                threshold=float(np.round(rng.uniform(0.5, 0.99), 3)))


@pytest.mark.parametrize("seed", list(range(901, 937)))
def test_prefill_random_configs(seed):
    """Whole path against the oracle on seeded random configurations (masks
    under the margin rule, block sums and attention within tolerance)."""
    cfg = _random_config(seed)
    say("random config %d: %s" % (seed, {k: (str(v) if k == "dtype" else v) for k, v in cfg.items()}))
    w = make_random("rand%d" % seed, seed=seed, **cfg)
    _prefill_and_check(w, label="random config %d" % seed)


@pytest.mark.parametrize("seed", list(range(951, 963)))
def test_prefill_random_configs_well_separated(seed):
    """Seeded random configurations on well-separated inputs (block scores
    far apart, shared ranks in the chunk-vote modes so that the vote keeps a
    scattered subset): the selection is genuinely sparse and masks and
    counts must match the oracle exactly."""
    rng = np.random.default_rng(seed)
    cfg = _random_config(seed)
    mode = cfg["select_mode"]
    kw = dict(hq=cfg["hq"], hkv=cfg["hkv"], d=cfg["d"], lq=cfg["lq"], lk=cfg["lk"], dtype=cfg["dtype"],
              stride=cfg["stride"], select_mode=mode, paged=cfg["paged"],
              threshold=float(np.round(rng.uniform(0.8, 0.95), 3)))
    if mode != "per_kvhead":
        kw.update(shared_ranks=True, rank_step=0.05)
    say("well-separated random config %d: %s" % (seed, {k: (str(v) if k == "dtype" else v) for k, v in kw.items()}))
    w = make_well_separated("wsrand%d" % seed, seed=seed, **kw)
    _prefill_and_check(w, exact=True, label="well-separated random config %d" % seed)


def test_prefill_paged_varlen_sampled():
    w = make_workload("paged_varlen_3seq")
    rows, idx = sample_rows(w, per_seq=48)
    _prefill_and_check(w, rows=rows, rows_idx=idx, label="paged varlen")


@pytest.mark.parametrize("case", [
    # the widest rows the library accepts: 4096 key blocks (512K tokens)
    dict(name="max_width_g2", hq=2, hkv=1, d=64, lq=[128], lk=[524288], mode="chunk_vote", tau=0.9),
    dict(name="max_width_g1", hq=1, hkv=1, d=64, lq=[256], lk=[524288], mode="per_kvhead", tau=0.9),
    # tau = 0: no block passes the threshold, only the forced ones remain
    dict(name="tau0_vote", hq=4, hkv=2, d=128, lq=[512], lk=[2048], mode="chunk_vote", tau=0.0),
    dict(name="tau0_kvhead", hq=4, hkv=2, d=128, lq=[512], lk=[2048], mode="per_kvhead", tau=0.0),
    # a lone block, and a batch whose only non-empty sequence is one block
    dict(name="one_block", hq=2, hkv=1, d=128, lq=[128], lk=[128], mode="per_kvhead", tau=0.9),
    dict(name="one_block_in_empties", hq=2, hkv=1, d=128, lq=[0, 128, 0], lk=[0, 256, 128], mode="chunk_vote",
         tau=0.9),
], ids=lambda c: c["name"])
def test_prefill_limits_and_degenerate_cases(case):
    """Whole path at the size limits and in the degenerate cases of the
    method, against the oracle (estimate, masks bit-exact on these inputs,
    attention on every row; the 512K rows on sampled rows)."""
    c = dict(case)
    name, mode, tau = c.pop("name"), c.pop("mode"), c.pop("tau")
    w = make_random(name, seed=61, select_mode=mode, threshold=tau, **c)
    rows = rows_idx = None
    if c["lk"][0] >= 65536:
        rows, rows_idx = sample_rows(w, per_seq=32)
    _prefill_and_check(w, rows=rows, rows_idx=rows_idx, exact=True, label=name)


@pytest.mark.parametrize("mode", ["per_kvhead", "chunk_vote"])
def test_prefill_reusing_another_layers_selection(mode):
    """reuse_selection: layer B attends over layer A's effective mask with no
    estimate or selection of its own -- equal to the oracle's attention of B
    over A's mask; B's block sums and counts are left untouched."""
    kw = dict(hq=8, hkv=2, d=128, lq=[1024, 512], lk=[2048, 512], select_mode=mode)
    wa = make_random("layerA", seed=51, **kw)
    wb = make_random("layerB", seed=52, **kw)
    ra, rb = Run(wa), Run(wb)
    say("reuse %s: layer A full path" % mode)
    _, _, _, aux_a = ra.prefill()
    mask_a = aux_a["mask_kv"]
    out = torch.full_like(rb.q, float("nan"))
    lse = torch.full((rb.hq, rb.shape.total_q), float("nan"), device="cuda")
    counts = torch.full((rb.B, 2), -7, dtype=torch.int32, device="cuda")
    bs = torch.full((rb.B, rb.hq, rb.max_qb, rb.max_kb), -3.0, device="cuda")
    params = X.make_params(stride=wb.stride, threshold=rb.tau, est_scale=rb.est_scale, softmax_scale=rb.softmax_scale,
                           kv_chunk_tokens=wb.kv_chunk_tokens, select_mode=mode, reuse_selection=1)
    say("reuse %s: layer B over layer A's mask" % mode)
    X.xattn_prefill_chunk(rb.shape, params, rb.q, rb.k, rb.v, out, lse, counts, rb.ws,
                          aux={"mask_kv": mask_a, "block_sums": bs})
    torch.cuda.synchronize()
    assert (counts == -7).all() and (bs == -3.0).all()
    ref_o, ref_l = rb.oracle_attention(mask_a)
    assert_attention_close(out, lse, ref_o, ref_l, wb.dtype, label="reuse " + mode)
    with pytest.raises(X.XattnError):
        X.xattn_prefill_chunk(rb.shape, params, rb.q, rb.k, rb.v, out, lse, counts, rb.ws)


@pytest.mark.parametrize("seed", [101, 102, 103])
@pytest.mark.parametrize("mode", ["per_kvhead", "chunk_vote"])
def test_well_separated_masks_bit_exact(seed, mode):
    w = make_well_separated("ws", seed=seed, hq=8, hkv=4, d=128, lq=[1024, 512], lk=[2048, 512],
                            select_mode=mode)
    _prefill_and_check(w, exact=True, label="well-separated %d %s" % (seed, mode))


@pytest.mark.parametrize("case", [
    # chunk vote over 28K of history: the heads agree on a scattered subset
    dict(name="vote_step1", mode="chunk_vote", step=1.0),
    dict(name="vote_step0.1", mode="chunk_vote", step=0.1),
    # per-KV-head rows of about 21 of up to 256 blocks: the attention's row
    # order and splits on short, uneven rows
    dict(name="kvhead_step0.1", mode="per_kvhead", step=0.1),
    # history by the vote, the current chunk per KV head
    dict(name="vote_sparse_cur_step0.1", mode="chunk_vote_sparse", step=0.1),
], ids=lambda c: c["name"])
def test_prefill_32k_sparse_selection(case):
    """The 32K chunk (16 q / 8 kv heads, 4096 queries over 32768 keys, s=8,
    tau=0.9) on well-separated inputs with block ranks shared by the kv
    heads: the selection is genuinely sparse, masks bit-exact, attention on
    sampled rows against the oracle on the GPU's mask."""
    w = make_well_separated("sparse32k_" + case["name"], seed=201, hq=16, hkv=8, d=128, lq=[4096], lk=[32768],
                            stride=8, threshold=0.9, select_mode=case["mode"], kv_chunk_tokens=4096,
                            shared_ranks=True, rank_step=case["step"])
    rows, idx = sample_rows(w, per_seq=48)
    mism, counts, aux = _prefill_and_check(w, rows=rows, rows_idx=idx, exact=True, label=w.name)
    dens = O.density(counts.cpu().tolist())
    assert 0.0 < dens < 0.5, "%s: density %.3g is not sparse" % (w.name, dens)
    if case["mode"] != "per_kvhead":
        assert_gapped(aux["hist_sel"][0], 224, w.name)
    if case["mode"] == "chunk_vote_sparse":
        # the current chunk really is sparse: fewer blocks than dense causal
        cur = aux["mask_kv"][0, :, :, 224:].cpu().numpy().astype(bool)
        assert cur.sum() < 8 * sum(i + 1 for i in range(32))


@pytest.mark.parametrize("mode", ["per_kvhead", "chunk_vote", "chunk_vote_sparse"])
@pytest.mark.parametrize("case", [
    dict(name="paged_3seq", hq=4, hkv=2, d=128, lq=[512, 256, 128], lk=[2048, 256, 1536], paged=True),
    dict(name="varlen_with_empty", hq=4, hkv=2, d=128, lq=[384, 0, 256], lk=[1024, 128, 256]),
    dict(name="causal_2k_gqa2", hq=16, hkv=8, d=128, lq=[2048], lk=[2048]),
], ids=lambda c: c["name"])
def test_prefill_block_lists_match_the_plan_path(case, mode):
    """In the resident prefill the selection kernels write the attention's
    block lists themselves (no plan launch); attending over the same
    effective mask through xattn_sparse_attn (plan kernel) must give the same
    bits, split rows and dynamically drawn tail parts included."""
    c = dict(case)
    name = c.pop("name")
    w = make_random(name, seed=71, select_mode=mode, **c)
    r = Run(w)
    say("block lists %s %s" % (name, mode))
    out, lse, counts, aux = r.prefill()
    out2, lse2 = r.attend(aux["mask_kv"])
    assert torch.equal(out.cpu(), out2.cpu()), "output differs from the plan path"
    assert torch.equal(lse.cpu(), lse2.cpu()), "LSE differs from the plan path"


@pytest.mark.parametrize("case", [
    # every sequence alone still takes the 256 x 256 tiles (>= 256 of them)
    dict(name="big_tiles", hq=32, hkv=8, d=128, lq=[2048, 2432, 512], lk=[16384, 8192, 16384]),
    dict(name="small_tiles", hq=4, hkv=2, d=128, lq=[512, 0, 256, 128], lk=[2048, 256, 256, 1536]),
], ids=lambda c: c["name"])
def test_estimate_batch_matches_per_sequence_launches(case):
    """A launch over several sequences numbers its workgroups over the tiles
    that have work (a per-sequence table of them); a single sequence's launch
    numbers them over its whole tile grid.  Each sequence's block sums must
    come out bit-identical either way."""
    import dataclasses

    c = dict(case)
    name = c.pop("name")
    w = make_random(name, seed=81, **c)
    say("estimate batch vs singles " + name)
    bs = Run(w).estimate().cpu()
    for b in range(w.batch):
        lq, lk = w.lens(b)
        if lq == 0:
            continue
        q0, k0 = w.cu_q[b], w.cu_k[b]
        one = dataclasses.replace(w, q=w.q[q0:q0 + lq].contiguous(), k=w.k[k0:k0 + lk].contiguous(),
                                  v=w.v[k0:k0 + lk].contiguous(), cu_q=[0, lq], cu_k=[0, lk],
                                  block_table=None, k_cache=None, v_cache=None)
        bs1 = Run(one).estimate().cpu()
        qb, kb = lq // 128, lk // 128
        assert torch.equal(bs[b, :, :qb, :kb], bs1[0, :, :qb, :kb]), "sequence %d differs" % b


def test_prefill_paged_cache_beyond_2gib():
    """A paged cache of 33000 pages (2.06 GiB each for K and V at 2 kv heads,
    d = 128) whose used pages lie past the 2^31-byte mark (one page below
    it): K/V spans beyond 31-bit buffer offsets select the register-staged
    estimate (est_partial_bf16) and the single-phase attention with V^T pages
    (attn_mfma) even for an even group.  Against the oracle on the same
    logical K/V."""
    w = make_random("paged2g", seed=93, hq=4, hkv=2, d=128, lq=[256, 128], lk=[768, 640], select_mode="per_kvhead")
    r = Run(w)  # the contiguous twin supplies the oracle inputs
    nphys, page_bytes = 33000, 128 * 2 * 128 * 2
    assert 32768 * page_bytes == 1 << 31
    rng = np.random.default_rng(94)
    nb = [w.lens(b)[1] // 128 for b in range(w.batch)]
    ids = rng.choice(np.arange(32768, nphys), size=sum(nb), replace=False)
    ids[3] = 5
    table = -np.ones((w.batch, max(nb)), dtype=np.int32)
    kc = torch.zeros((nphys, 128, 2, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    n = 0
    for b in range(w.batch):
        for j in range(nb[b]):
            t0 = w.cu_k[b] + j * 128
            kc[int(ids[n])] = r.k[t0:t0 + 128]
            vc[int(ids[n])] = r.v[t0:t0 + 128]
            table[b, j] = ids[n]
            n += 1
    tdev = torch.from_numpy(table).cuda()
    sh = X.Shape(num_q_heads=4, num_kv_heads=2, head_dim=128, dtype=w.dtype, cu_q=w.cu_q, cu_k=w.cu_k,
                 device="cuda", block_table=tdev, num_phys_blocks=nphys)
    ws = X.alloc_workspace(sh, r.params)
    assert ws.numel() > nphys * page_bytes  # V^T pages reserved for the single-phase kernel
    out = torch.full_like(r.q, float("nan"))
    lse = torch.full((r.hq, sh.total_q), float("nan"), device="cuda")
    counts = torch.full((r.B, 2), -1, dtype=torch.int32, device="cuda")
    aux = {"block_sums": torch.empty((r.B, r.hq, r.max_qb, r.max_kb), device="cuda"),
           "mask_kv": torch.empty((r.B, r.hkv, r.max_qb, r.max_kb), dtype=torch.uint8, device="cuda"),
           "hist_sel": torch.empty((r.B, r.max_kb), dtype=torch.uint8, device="cuda")}
    say("paged cache beyond 2 GiB")
    X.xattn_prefill_chunk(sh, r.params, r.q, kc, vc, out, lse, counts, ws, aux=aux)
    torch.cuda.synchronize()
    ref = r.oracle(attention=False)
    assert_block_sums_close(aux["block_sums"], ref["block_sums"], w.stride, "paged 2 GiB")
    check_selection(r, ref, aux["block_sums"], aux["mask_kv"], aux["hist_sel"], "paged 2 GiB")
    ref_o, ref_l = r.oracle_attention(aux["mask_kv"])
    assert_attention_close(out, lse, ref_o, ref_l, w.dtype, label="paged 2 GiB")
    del kc, vc, ws
    torch.cuda.empty_cache()


def test_block_table_entries_outside_the_cache(monkeypatch):
    """XATTN_DEBUG=1: a table entry inside a sequence's key range that is -1
    or names no page of the cache is rejected (INVALID) before any work, by
    every call that takes the table.  Without it such an entry is an absent
    page: an entry one past the cache gives the same bits as -1."""
    w = make_random("badtable", seed=91, hq=4, hkv=2, d=128, lq=[256, 128], lk=[768, 640], paged=True,
                    select_mode="per_kvhead")
    r = Run(w)
    nphys = w.k_cache.shape[0]
    good = w.block_table.clone()
    results = {}
    for bad in (-1, nphys):
        t = good.clone()
        t[0, 2] = bad
        r.table.copy_(t.to("cuda"))
        monkeypatch.setenv("XATTN_DEBUG", "1")
        say("block table entry %d, debug" % bad)
        with pytest.raises(X.XattnError) as ei:
            r.prefill()
        assert ei.value.code == -1 and "block_table entry 2" in str(ei.value), str(ei.value)
        with pytest.raises(X.XattnError):
            r.estimate()
        with pytest.raises(X.XattnError):
            r.attend(torch.ones((r.B, r.hkv, r.max_qb, r.max_kb), dtype=torch.uint8))
        monkeypatch.setenv("XATTN_DEBUG", "0")
        say("block table entry %d, no debug" % bad)
        results[bad] = r.prefill()
    o1, l1, c1, a1 = results[-1]
    o2, l2, c2, a2 = results[nphys]
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(a1["block_sums"], a2["block_sums"])
    r.table.copy_(good.to("cuda"))
    monkeypatch.setenv("XATTN_DEBUG", "1")
    out, lse, counts, aux = r.prefill()  # a valid table passes the check
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("case", [
    dict(name="s8_g2", hq=16, hkv=8, d=128, lq=[2048], lk=[8192], stride=8),
    dict(name="s16_g4", hq=32, hkv=8, d=128, lq=[1024], lk=[16384], stride=16),
    dict(name="s4_g2_d64", hq=4, hkv=2, d=64, lq=[512], lk=[2048], stride=4),
    dict(name="paged_varlen", hq=8, hkv=4, d=128, lq=[512, 0, 256], lk=[2048, 128, 1024], stride=8, paged=True),
    dict(name="g16", hq=16, hkv=1, d=64, lq=[256], lk=[8192], stride=8),
    dict(name="wide_rows", hq=4, hkv=1, d=64, lq=[128], lk=[131072], stride=8),
], ids=lambda c: c["name"])
@pytest.mark.parametrize("mode", ["per_kvhead", "chunk_vote"])
def test_prefill_block_sums_equal_the_estimate_kernel(case, mode):
    """The whole path's block sums (the aux output of xattn_prefill_chunk)
    are bit-identical to xattn_estimate's on the same inputs, for the three
    reshaped block sizes, GQA groups up to 16, paged varlen batches and rows
    too wide for the fused selection kernel."""
    c = dict(case)
    name = c.pop("name")
    w = make_random(name, seed=99, select_mode=mode, **c)
    r = Run(w)
    say("block sums, prefill vs estimate: %s %s" % (name, mode))
    bs_est = r.estimate()
    _, _, _, aux = r.prefill()
    assert torch.equal(aux["block_sums"].cpu(), bs_est.cpu()), "prefill block sums differ from xattn_estimate's"


@pytest.mark.parametrize("k", [3, 9])
@pytest.mark.parametrize("mode", ["per_kvhead", "chunk_vote", "chunk_vote_sparse"])
def test_prefill_topk_end_to_end(k, mode):
    """The top-k rule (num_to_choose) through the whole path on
    well-separated inputs (large value gaps at every row's k-th block):
    masks and counts bit-exact, attention against the oracle on the GPU's
    mask."""
    w = make_well_separated("topk_e2e", seed=105, hq=8, hkv=4, d=128, lq=[1024, 512], lk=[4096, 512],
                            select_mode=mode)
    r = Run(w, num_to_choose=k)
    say("top-%d end to end %s" % (k, mode))
    out, lse, counts, aux = r.prefill()
    ref = r.oracle(attention=False)
    assert_block_sums_close(aux["block_sums"], ref["block_sums"], w.stride, "top-k")
    gm = aux["mask_kv"].cpu().numpy().astype(bool)
    assert (gm == ref["mask_kv"]).all(), "top-%d mask differs from the oracle" % k
    assert (counts.cpu().numpy() == ref["counts"]).all()
    ref_o, ref_l = r.oracle_attention(aux["mask_kv"])
    assert_attention_close(out, lse, ref_o, ref_l, w.dtype, label="top-k e2e")


@pytest.mark.parametrize("spread", ["narrow", "wide"])
@pytest.mark.parametrize("width", [40, 256, 3000])
def test_select_exact_and_serial_scans(spread, width):
    """The selection adds a row's sorted values in float64 with a wave-wide
    scan when every partial sum is exact (values within a narrow exponent
    range: any order gives the same bits), else serially in sorted order.
    narrow: values in [0.5, 1) (exact scan); wide: values 2^-60 .. 1
    (serial scan, where the rounding order matters).  Both bit-exact
    against the oracle's left-to-right cumulative sum."""
    lk = 128 * width
    w = make_random("scan", seed=27, hq=4, hkv=2, d=64, lq=[256], lk=[lk], dtype=torch.float32, stride=8,
                    select_mode="per_kvhead")
    r = Run(w, threshold=0.9)
    rng = np.random.default_rng(28)
    shape = (r.B, r.hq, r.max_qb, r.max_kb)
    if spread == "narrow":
        bs32 = (0.5 + 0.5 * rng.random(shape)).astype(np.float32)
    else:
        bs32 = np.exp2(-60.0 * rng.random(shape)).astype(np.float32)
    say("select scan %s %d" % (spread, width))
    mask, hist, counts = r.select(torch.from_numpy(bs32))
    lq, lk_ = w.lens(0)
    qb, kb = lq // 128, lk_ // 128
    sel = O.select_blocks(bs32[0, :, :qb, :kb].astype(np.float64), kh=(lk_ - lq) // 128, tau=r.tau,
                          group=2, mode="per_kvhead")
    m = mask[0].cpu().numpy().astype(bool)
    assert (m[:, :qb, :kb] == sel["mask_kv"]).all()
    assert tuple(counts[0].tolist()) == sel["counts"]
