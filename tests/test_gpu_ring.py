"""Ring mode of xattn_prefill_chunk: history K/V in pinned host memory,
streamed through device slots on a transfer stream with event ordering.

Checks: agreement with the resident-KV path and with the oracle; bit-equal
results when every slot copy is delayed on the host (a missing wait would
let a kernel read a stale slot); slot reuse with 2 slots; a pageable history
is rejected before any work; the 128K-context workload on sampled rows.

Unless a test says otherwise the inputs are well separated with block ranks
shared by the kv heads, so the chunk vote keeps a scattered tenth of the
history: the slot packing (several runs per slot, block j in slot position
x != j), the gather's skipping of unvoted blocks and the per-slot key windows
all run on gaps.  Each such test asserts that the vote left gaps.
"""

import numpy as np
import pytest
import torch

import block_sparse_attention_strided_amd as X
from tests.gpu_util import (Run, assert_attention_close, assert_block_sums_close, assert_gapped, check_selection,
                            sample_rows, say)
from workloads import make_random, make_well_separated, make_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _ring_inputs(w, pinned=True):
    lq, lk = w.lens(0)
    kh = (lk - lq) // 128
    hkv, d = w.num_kv_heads, w.head_dim
    kh_t = w.k[: lk - lq].reshape(kh, 128, hkv, d)
    vh_t = w.v[: lk - lq].reshape(kh, 128, hkv, d)
    if pinned:
        k_hist = torch.empty(kh_t.shape, dtype=w.dtype, pin_memory=True)
        v_hist = torch.empty(vh_t.shape, dtype=w.dtype, pin_memory=True)
        k_hist.copy_(kh_t)
        v_hist.copy_(vh_t)
    else:
        k_hist, v_hist = kh_t.contiguous(), vh_t.contiguous()
    k_cur = w.k[lk - lq:].cuda()
    v_cur = w.v[lk - lq:].cuda()
    return k_hist, v_hist, k_cur, v_cur, kh


def _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh):
    out = torch.full_like(r.q, float("nan"))
    lse = torch.full((r.hq, r.shape.total_q), float("nan"), device="cuda")
    counts = torch.full((1, 2), -1, dtype=torch.int32, device="cuda")
    aux = {
        "block_sums": torch.empty((1, r.hq, r.max_qb, r.max_kb), device="cuda"),
        "mask_kv": torch.empty((1, r.hkv, r.max_qb, r.max_kb), dtype=torch.uint8, device="cuda"),
        "hist_sel": torch.empty((1, r.max_kb), dtype=torch.uint8, device="cuda"),
    }
    X.xattn_prefill_chunk(r.shape, r.params, r.q, k_cur, v_cur, out, lse, counts, r.ws, aux=aux, ring=ring,
                          k_hist=k_hist, v_hist=v_hist, hist_blocks=kh)
    torch.cuda.synchronize()
    return out, lse, counts, aux


SMALL = dict(d=128, lq=[1024], lk=[16384], stride=16, threshold=0.95, select_mode="chunk_vote",
             kv_chunk_tokens=1024)


def _small(kind="sparse", hq=8, hkv=2, seed=41, lk=None, mode="chunk_vote"):
    """1024 queries over 16K keys (120 history blocks), s=16, tau=0.95.
    sparse: well-separated shared ranks, step 0.3 (the vote keeps 12 of 120
    history blocks in 11 runs); gaussian: planted Gaussian inputs (the vote
    keeps every block)."""
    kw = dict(SMALL, hq=hq, hkv=hkv, select_mode=mode)
    if lk is not None:
        kw["lk"] = [lk]
    if kind == "gaussian":
        return make_random("ring_small_gauss", seed=seed, **kw)
    return make_well_separated("ring_small_sparse", seed=seed, shared_ranks=True, rank_step=0.3, **kw)


@pytest.mark.parametrize("kind,hq,slots,mode", [
    ("sparse", 8, 4, "chunk_vote"), ("sparse", 8, 2, "chunk_vote"), ("sparse", 6, 4, "chunk_vote"),
    ("gaussian", 8, 4, "chunk_vote"), ("sparse", 8, 4, "chunk_vote_sparse")],
    ids=["sparse-g4-4slots", "sparse-g4-2slots", "sparse-g3-4slots", "gaussian-g4-4slots", "sparse-cur-g4-4slots"])
def test_ring_matches_resident_path_and_oracle(kind, hq, slots, mode):
    """Group 3 (hq=6, hkv=2) runs the single-phase attention kernel, which
    reads V^T pages of each slot; chunk_vote_sparse also selects inside the
    resident current chunk."""
    w = _small(kind, hq=hq, mode=mode)
    r = Run(w)
    k_hist, v_hist, k_cur, v_cur, kh = _ring_inputs(w)
    ring = X.Ring(slots, 8, w.num_kv_heads, w.head_dim, w.dtype)
    say("ring small %s hq=%d slots=%d: resident path" % (kind, hq, slots))
    o_res, l_res, c_res, aux_res = r.prefill()
    say("ring small: ring path")
    o_ring, l_ring, c_ring, aux_ring = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    ring.close()
    if kind == "sparse":
        assert_gapped(aux_ring["hist_sel"][0], kh, "ring %s hq=%d slots=%d" % (kind, hq, slots))
    # the estimate and the selection see bit-identical inputs either way
    assert torch.equal(aux_res["block_sums"], aux_ring["block_sums"])
    assert torch.equal(aux_res["mask_kv"], aux_ring["mask_kv"])
    assert torch.equal(c_res, c_ring)
    assert (o_res.float() - o_ring.float()).abs().max().item() <= 2e-2
    ref = r.oracle(attention=False)
    assert_block_sums_close(aux_ring["block_sums"], ref["block_sums"], w.stride, "ring small")
    check_selection(r, ref, aux_ring["block_sums"], aux_ring["mask_kv"], aux_ring["hist_sel"],
                    "ring small %s hq=%d" % (kind, hq))
    if kind == "sparse":
        assert torch.equal(aux_ring["hist_sel"][0, :kh].cpu(), torch.from_numpy(ref["hist_sel"][0, :kh]).to(torch.uint8))
    ref_o, ref_l = r.oracle_attention(aux_ring["mask_kv"])
    assert_attention_close(o_ring, l_ring, ref_o, ref_l, w.dtype, label="ring small")


@pytest.mark.parametrize("slots", [2, 4])
def test_ring_delayed_copies_give_identical_results(slots):
    """A host callback sleeps 2 ms before every slot copy on the transfer
    stream; with correct event ordering the result is bit-identical."""
    w = _small()
    r = Run(w)
    k_hist, v_hist, k_cur, v_cur, kh = _ring_inputs(w)
    ring = X.Ring(slots, 8, w.num_kv_heads, w.head_dim, w.dtype)
    say("ring delay test slots=%d: no delay" % slots)
    o0, l0, c0, a0 = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    assert_gapped(a0["hist_sel"][0], kh, "ring delay slots=%d" % slots)
    ring.set_copy_delay_us(2000)
    say("ring delay test slots=%d: 2 ms delay per copy" % slots)
    o1, l1, c1, a1 = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    ring.set_copy_delay_us(0)
    say("ring delay test slots=%d: back to back" % slots)
    o2, l2, c2, a2 = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    ring.close()
    for o, l_, c, a in ((o1, l1, c1, a1), (o2, l2, c2, a2)):
        assert torch.equal(a["block_sums"], a0["block_sums"])
        assert torch.equal(a["mask_kv"], a0["mask_kv"])
        assert torch.equal(c, c0)
        assert torch.equal(o, o0)
        assert torch.equal(l_, l0)


def _write_back_pair(seed_chunk2, seed_chunk1, L=16384, lq=1024):
    """Chunk 2 (the last lq of L keys) and chunk 1 (the lq before it) of one
    well-separated sequence: chunk 1's keys are chunk 2's first L - lq."""
    kw = dict(hq=8, hkv=2, d=128, stride=16, threshold=0.95, select_mode="chunk_vote", kv_chunk_tokens=1024,
              shared_ranks=True, rank_step=0.3)
    w2 = make_well_separated("wb2", seed=seed_chunk2, lq=[lq], lk=[L], **kw)
    w1 = make_well_separated("wb1", seed=seed_chunk1, lq=[lq], lk=[L - lq], **kw)
    w1.k = w2.k[: L - lq].clone()
    w1.v = w2.v[: L - lq].clone()
    return w1, w2


def test_ring_write_back_feeds_the_next_chunk():
    """Chunk 1's K/V, written back into the pinned history on the ring's
    offload stream (every copy delayed 2 ms by a host callback), are read by
    chunk 2's ring prefill: its estimate, selection and output equal chunk 2
    with all K/V resident, and the host history holds chunk 1's K/V."""
    L, lq = 16384, 1024
    w1, w2 = _write_back_pair(43, 43)
    r1, r2 = Run(w1), Run(w2)
    hkv, d = w2.num_kv_heads, w2.head_dim
    nh, h1 = (L - lq) // 128, (L - 2 * lq) // 128
    k_host = torch.empty((nh, 128, hkv, d), dtype=w2.dtype, pin_memory=True).fill_(float("nan"))
    v_host = torch.empty((nh, 128, hkv, d), dtype=w2.dtype, pin_memory=True).fill_(float("nan"))
    k_host[:h1].copy_(w2.k[: L - 2 * lq].reshape(h1, 128, hkv, d))
    v_host[:h1].copy_(w2.v[: L - 2 * lq].reshape(h1, 128, hkv, d))
    ring = X.Ring(4, 8, hkv, d, w2.dtype)
    ring.set_copy_delay_us(2000)
    k1, v1 = w2.k[L - 2 * lq: L - lq].cuda(), w2.v[L - 2 * lq: L - lq].cuda()
    say("write-back: chunk 1 through the ring")
    _, _, _, a1 = _run_ring(r1, w1, ring, k_host[:h1], v_host[:h1], k1, v1, h1)
    assert_gapped(a1["hist_sel"][0], h1, "write-back chunk 1")
    say("write-back: chunk 1 K/V to host blocks %d..%d" % (h1, nh))
    ring.offload_chunk(k1, v1, k_host[h1:], v_host[h1:], lq // 128)
    k2, v2 = w2.k[L - lq:].cuda(), w2.v[L - lq:].cuda()
    say("write-back: chunk 2 through the ring")
    o2, l2, c2, a2 = _run_ring(r2, w2, ring, k_host, v_host, k2, v2, nh)
    ring.offload_wait()
    torch.cuda.synchronize()
    ring.close()
    assert_gapped(a2["hist_sel"][0], nh, "write-back chunk 2")
    assert torch.equal(k_host.reshape(-1, hkv, d), w2.k[: L - lq])
    assert torch.equal(v_host.reshape(-1, hkv, d), w2.v[: L - lq])
    say("write-back: chunk 2 resident")
    o_res, l_res, c_res, a_res = r2.prefill()
    assert torch.equal(a2["block_sums"], a_res["block_sums"])
    assert torch.equal(a2["mask_kv"], a_res["mask_kv"])
    assert torch.equal(c2, c_res)
    assert (o2.float() - o_res.float()).abs().max().item() <= 2e-2


def test_ring_reusing_a_selection_skips_the_estimate():
    """reuse_selection in ring mode: the selection of a first ring call
    (mask_kv and hist_sel) drives a second call that streams no history K for
    an estimate; same output, block sums untouched."""
    w = _small()
    r = Run(w)
    k_hist, v_hist, k_cur, v_cur, kh = _ring_inputs(w)
    ring = X.Ring(4, 8, w.num_kv_heads, w.head_dim, w.dtype)
    say("ring reuse: full path")
    o0, l0, c0, a0 = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    assert_gapped(a0["hist_sel"][0], kh, "ring reuse")
    params = X.make_params(stride=w.stride, threshold=r.tau, est_scale=r.est_scale, softmax_scale=r.softmax_scale,
                           kv_chunk_tokens=w.kv_chunk_tokens, select_mode=w.select_mode, reuse_selection=1)
    out = torch.full_like(r.q, float("nan"))
    lse = torch.full((r.hq, r.shape.total_q), float("nan"), device="cuda")
    bs = torch.full_like(a0["block_sums"], -3.0)
    say("ring reuse: reusing the selection")
    X.xattn_prefill_chunk(r.shape, params, r.q, k_cur, v_cur, out, lse, None, r.ws,
                          aux={"mask_kv": a0["mask_kv"], "hist_sel": a0["hist_sel"], "block_sums": bs},
                          ring=ring, k_hist=k_hist, v_hist=v_hist, hist_blocks=kh)
    torch.cuda.synchronize()
    ring.close()
    assert (bs == -3.0).all()
    assert torch.equal(out, o0)
    assert torch.equal(lse, l0)


@pytest.mark.parametrize("hq,mode", [(8, "chunk_vote"), (6, "chunk_vote"), (8, "chunk_vote_sparse")],
                         ids=["g4", "g3", "g4-sparse-cur"])
def test_staged_ring_matches_resident_path(hq, mode):
    """Staged ring (history K in chunks, device-driven gather of the voted V
    blocks from mapped pinned memory, chunked attention with merges):
    estimate and selection bit-identical to the resident path, output within
    the bf16 tolerance of it and of the oracle; bit-identical to itself with
    every copy delayed 2 ms and with a reused selection.  hq=6 (group 3) runs
    the single-phase kernel, which reads V^T pages transposed per launch.
    The 20K history spans two staging chunks of 128 blocks."""
    w = _small(hq=hq, lk=20480, mode=mode)
    r = Run(w)
    k_hist, v_hist, k_cur, v_cur, kh = _ring_inputs(w)
    lq, lk = w.lens(0)
    ring = X.Ring(1, lk // 128, w.num_kv_heads, w.head_dim, w.dtype, staged=True)
    say("staged ring hq=%d %s: resident path" % (hq, mode))
    o_res, l_res, c_res, a_res = r.prefill()
    say("staged ring: staged path")
    o_st, l_st, c_st, a_st = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    runs = assert_gapped(a_st["hist_sel"][0], kh, "staged hq=%d" % hq)
    assert any(j < 128 for j, _ in runs) and any(j + n > 128 for j, n in runs), runs
    for a in ("block_sums", "mask_kv", "hist_sel"):
        assert torch.equal(a_st[a], a_res[a]), a
    assert torch.equal(c_st, c_res)
    assert (o_st.float() - o_res.float()).abs().max().item() <= 2e-2
    ref_o, ref_l = r.oracle_attention(a_st["mask_kv"])
    assert_attention_close(o_st, l_st, ref_o, ref_l, w.dtype, label="staged ring")
    ring.set_copy_delay_us(2000)
    say("staged ring: 2 ms delay per copy")
    o_d, l_d, c_d, a_d = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    ring.set_copy_delay_us(0)
    assert torch.equal(o_d, o_st) and torch.equal(a_d["block_sums"], a_res["block_sums"])
    params = X.make_params(stride=w.stride, threshold=r.tau, est_scale=r.est_scale, softmax_scale=r.softmax_scale,
                           kv_chunk_tokens=w.kv_chunk_tokens, select_mode=w.select_mode, reuse_selection=1)
    out = torch.full_like(r.q, float("nan"))
    lse = torch.full((r.hq, r.shape.total_q), float("nan"), device="cuda")
    say("staged ring: reused selection")
    X.xattn_prefill_chunk(r.shape, params, r.q, k_cur, v_cur, out, lse, None, r.ws,
                          aux={"mask_kv": a_res["mask_kv"], "hist_sel": a_res["hist_sel"]},
                          ring=ring, k_hist=k_hist, v_hist=v_hist, hist_blocks=kh)
    torch.cuda.synchronize()
    ring.close()
    assert torch.equal(out, o_st) and torch.equal(lse, l_st)
    small = X.Ring(1, lk // 128 - 1, w.num_kv_heads, w.head_dim, w.dtype, staged=True)
    with pytest.raises(X.XattnError):
        _run_ring(r, w, small, k_hist, v_hist, k_cur, v_cur, kh)
    small.close()


def test_staged_ring_write_back_feeds_the_next_chunk():
    """Chunk 1 through the staged ring, its K/V written back (delayed 2 ms per
    copy) into the pinned history, chunk 2 through the staged ring: equal to
    chunk 2 with all K/V resident."""
    L, lq = 16384, 1024
    w1, w2 = _write_back_pair(45, 45)
    r1, r2 = Run(w1), Run(w2)
    hkv, d = w2.num_kv_heads, w2.head_dim
    nh, h1 = (L - lq) // 128, (L - 2 * lq) // 128
    k_host = torch.empty((nh, 128, hkv, d), dtype=w2.dtype, pin_memory=True).fill_(float("nan"))
    v_host = torch.empty((nh, 128, hkv, d), dtype=w2.dtype, pin_memory=True).fill_(float("nan"))
    k_host[:h1].copy_(w2.k[: L - 2 * lq].reshape(h1, 128, hkv, d))
    v_host[:h1].copy_(w2.v[: L - 2 * lq].reshape(h1, 128, hkv, d))
    ring = X.Ring(1, L // 128, hkv, d, w2.dtype, staged=True)
    ring.set_copy_delay_us(2000)
    k1, v1 = w2.k[L - 2 * lq: L - lq].cuda(), w2.v[L - 2 * lq: L - lq].cuda()
    say("staged write-back: chunk 1")
    _run_ring(r1, w1, ring, k_host[:h1], v_host[:h1], k1, v1, h1)
    ring.offload_chunk(k1, v1, k_host[h1:], v_host[h1:], lq // 128)
    k2, v2 = w2.k[L - lq:].cuda(), w2.v[L - lq:].cuda()
    say("staged write-back: chunk 2")
    o2, l2, c2, a2 = _run_ring(r2, w2, ring, k_host, v_host, k2, v2, nh)
    ring.offload_wait()
    torch.cuda.synchronize()
    ring.close()
    assert_gapped(a2["hist_sel"][0], nh, "staged write-back chunk 2")
    o_res, l_res, c_res, a_res = r2.prefill()
    assert torch.equal(a2["block_sums"], a_res["block_sums"])
    assert torch.equal(a2["mask_kv"], a_res["mask_kv"])
    assert (o2.float() - o_res.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("seed", list(range(1001, 1013)))
def test_ring_random_configs(seed):
    """Seeded random ring configurations: slot ring (2 or 4 slots of 4-16
    blocks) or staged ring, heads and group, d, stride, chunk-vote mode,
    dtype, well-separated (gapped vote) or Gaussian inputs.  Block sums,
    masks, history vote and counts bit-identical to the resident path, the
    output within the dtype's tolerance of it, the selection under the
    margin rule against the oracle."""
    rng = np.random.default_rng(seed)
    hq, hkv = [(2, 1), (4, 2), (6, 2), (8, 2), (4, 4)][rng.integers(5)]
    lq = 128 * int(rng.integers(2, 9))
    lk = lq + 128 * int(rng.integers(8, 64))
    dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
    kw = dict(hq=hq, hkv=hkv, d=int(rng.choice([64, 128])), lq=[lq], lk=[lk], dtype=dtype,
              stride=int(rng.choice([4, 8, 16])), select_mode=str(rng.choice(["chunk_vote", "chunk_vote_sparse"])),
              threshold=float(np.round(rng.uniform(0.8, 0.95), 3)), kv_chunk_tokens=int(rng.choice([1024, 4096])))
    staged = bool(rng.random() < 0.4)
    slots, slot_blocks = int(rng.choice([2, 4])), int(rng.choice([4, 8, 16]))
    if rng.random() < 0.7:
        w = make_well_separated("ring_rand%d" % seed, seed=seed, shared_ranks=True, rank_step=0.3, **kw)
    else:
        w = make_random("ring_rand%d" % seed, seed=seed, **kw)
    say("ring random config %d: staged=%s slots=%d x %d %s" % (seed, staged, slots, slot_blocks,
                                                             {k: (str(v) if k == "dtype" else v) for k, v in kw.items()}))
    r = Run(w)
    k_hist, v_hist, k_cur, v_cur, kh = _ring_inputs(w)
    ring = (X.Ring(1, lk // 128, hkv, w.head_dim, dtype, staged=True) if staged
            else X.Ring(slots, slot_blocks, hkv, w.head_dim, dtype))
    o_res, l_res, c_res, a_res = r.prefill()
    o_ring, l_ring, c_ring, a_ring = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    ring.close()
    for a in ("block_sums", "mask_kv"):
        assert torch.equal(a_res[a], a_ring[a]), a
    assert torch.equal(a_res["hist_sel"][:, :kh], a_ring["hist_sel"][:, :kh])
    assert torch.equal(c_res, c_ring)
    tol = 2e-2 if dtype == torch.bfloat16 else 1e-4
    assert (o_res.float() - o_ring.float()).abs().max().item() <= tol
    ref = r.oracle(attention=False)
    assert_block_sums_close(a_ring["block_sums"], ref["block_sums"], w.stride, "ring random %d" % seed)
    check_selection(r, ref, a_ring["block_sums"], a_ring["mask_kv"], a_ring["hist_sel"], "ring random %d" % seed)


def test_ring_write_back_rejects_pageable_destination():
    ring = X.Ring(2, 2, 1, 128, torch.bfloat16)
    k = torch.zeros((128, 1, 128), dtype=torch.bfloat16, device="cuda")
    dst = torch.zeros((1, 128, 1, 128), dtype=torch.bfloat16)
    with pytest.raises(X.XattnError) as ei:
        ring.offload_chunk(k, k, dst, dst, 1)
    assert ei.value.code == -5
    with pytest.raises(X.XattnError):
        ring.offload_chunk(k, k, dst, dst, -1)
    ring.close()


def test_ring_rejects_pageable_history():
    w = make_random("ring_err", seed=42, hq=2, hkv=1, d=128, lq=[256], lk=[1024], stride=8,
                    select_mode="chunk_vote")
    r = Run(w)
    k_hist, v_hist, k_cur, v_cur, kh = _ring_inputs(w, pinned=False)
    ring = X.Ring(2, 2, 1, 128, w.dtype)
    with pytest.raises(X.XattnError) as ei:
        _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    assert ei.value.code == -5
    ring.close()


def _ring_128k_check(w, staged=False):
    r = Run(w)
    k_hist, v_hist, k_cur, v_cur, kh = _ring_inputs(w)
    if staged:
        ring = X.Ring(1, w.lens(0)[1] // 128, w.num_kv_heads, w.head_dim, w.dtype, staged=True)
    else:
        ring = X.Ring(w.ring_slots, w.ring_slot_blocks, w.num_kv_heads, w.head_dim, w.dtype)
    say("ring 128K %s: %s path" % (w.name, "staged" if staged else "slot"))
    out, lse, counts, aux = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    ring.close()
    ref = r.oracle(attention=False)
    assert_block_sums_close(aux["block_sums"], ref["block_sums"], w.stride, "128K")
    mism, soft, firm = check_selection(r, ref, aux["block_sums"], aux["mask_kv"], aux["hist_sel"],
                                       "128K %s %s" % (w.name, "staged" if staged else "slots"))
    say("  mask mismatch %.4g (%d soft / %d firm rows) counts %s vs %s" % (
        mism, soft, firm, counts.tolist(), ref["counts"].tolist()))
    rng = np.random.default_rng(3)
    blocks = sorted(rng.choice(32, size=3, replace=False).tolist())
    rows = {0: sorted({b * 128 + int(x) for b in blocks for x in rng.choice(128, 16, replace=False)} |
                      {b * 128 for b in blocks} | {b * 128 + 127 for b in blocks})}
    ref_o, ref_l = r.oracle_attention(aux["mask_kv"], rows=rows)
    assert_attention_close(out, lse, ref_o, ref_l, w.dtype, rows_idx=np.asarray(rows[0]), label="128K")
    return aux, ref, kh


def test_ring_qwen3_4b_128k_sampled():
    _ring_128k_check(make_workload("qwen3_4b_128k_ring"))


@pytest.mark.parametrize("staged", [False, True], ids=["slots", "staged"])
def test_ring_128k_sparse_vote(staged):
    """The 128K ring shape (32 q / 8 kv heads, s=16, tau=0.95, 4 slots of 32
    blocks) on well-separated inputs with shared ranks, step 0.05: the vote
    keeps about 6% of the 992 history blocks in about 50 runs, which the
    slot ring packs several runs to a slot and the staged ring gathers."""
    w = make_well_separated("ring128k_sparse", seed=202, hq=32, hkv=8, d=128, lq=[4096], lk=[131072], stride=16,
                            threshold=0.95, select_mode="chunk_vote", kv_chunk_tokens=4096, shared_ranks=True,
                            rank_step=0.05, ring=True)
    aux, ref, kh = _ring_128k_check(w, staged=staged)
    runs = assert_gapped(aux["hist_sel"][0], kh, "128K sparse %s" % ("staged" if staged else "slots"))
    assert len(runs) >= 10
    assert torch.equal(aux["hist_sel"][0, :kh].cpu(), torch.from_numpy(ref["hist_sel"][0, :kh]).to(torch.uint8))


def test_ring_fp32_matches_resident_path_and_oracle():
    """fp32 K/V through the slot ring (4 slots of 2 blocks) on a gapped vote:
    selection bit-identical to the resident path, outputs within the fp32
    tolerance of it and of the oracle."""
    w = make_well_separated("ring_f32", seed=47, hq=2, hkv=1, d=64, lq=[256], lk=[4096], dtype=torch.float32,
                            stride=8, threshold=0.9, select_mode="chunk_vote", kv_chunk_tokens=512,
                            shared_ranks=True, rank_step=0.3)
    r = Run(w)
    k_hist, v_hist, k_cur, v_cur, kh = _ring_inputs(w)
    ring = X.Ring(4, 2, w.num_kv_heads, w.head_dim, w.dtype)
    say("ring fp32: resident path")
    o_res, l_res, c_res, a_res = r.prefill()
    say("ring fp32: ring path")
    o_ring, l_ring, c_ring, a_ring = _run_ring(r, w, ring, k_hist, v_hist, k_cur, v_cur, kh)
    ring.close()
    assert_gapped(a_ring["hist_sel"][0], kh, "ring fp32")
    assert torch.equal(a_res["block_sums"], a_ring["block_sums"])
    assert torch.equal(a_res["mask_kv"], a_ring["mask_kv"])
    assert (o_res - o_ring).abs().max().item() <= 1e-4
    ref_o, ref_l = r.oracle_attention(a_ring["mask_kv"])
    assert_attention_close(o_ring, l_ring, ref_o, ref_l, w.dtype, label="ring fp32")
