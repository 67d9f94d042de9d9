"""Shared plumbing for the GPU parity tests: move a workload to the device,
run the library's stages through the C ABI, and run the oracle on the same
inputs with the same float32-rounded parameters."""

import math
import sys

import numpy as np
import torch

import block_sparse_attention_strided_amd as X
import oracle as O
from tests import metrics

# Tolerances (floating point): block sums |g-o| <= 1e-3*|o| + 1e-7*rb;
# attention bf16 out 2e-2 abs / lse 1e-3 abs; fp32 out 1e-4 / lse 1e-5.
BS_RTOL = 1e-3
OUT_ATOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
LSE_ATOL = {torch.bfloat16: 1e-3, torch.float32: 1e-5}


def f32(x):
    return float(np.float32(x))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Run:
    """A workload resident on the GPU with its C-ABI shape/params/workspace."""

    def __init__(self, w, *, threshold=None, select_mode=None, group_agg=None, num_to_choose=0, device="cuda"):
        self.w = w
        self.paged = w.block_table is not None
        d = w.head_dim
        self.tau = f32(w.threshold if threshold is None else threshold)
        self.mode = w.select_mode if select_mode is None else select_mode
        self.agg = w.group_agg if group_agg is None else group_agg
        self.num_to_choose = num_to_choose
        self.est_scale = f32(1.0 / (w.stride * math.sqrt(d)))
        self.softmax_scale = f32(1.0 / math.sqrt(d))
        self.q = w.q.to(device)
        if self.paged:
            self.k = w.k_cache.to(device)
            self.v = w.v_cache.to(device)
            self.table = w.block_table.to(device).contiguous()
            self.shape = X.Shape(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=d,
                                 dtype=w.dtype, cu_q=w.cu_q, cu_k=w.cu_k, device=device,
                                 block_table=self.table, num_phys_blocks=w.k_cache.shape[0])
        else:
            self.k = w.k.to(device)
            self.v = w.v.to(device)
            self.shape = X.Shape(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=d,
                                 dtype=w.dtype, cu_q=w.cu_q, cu_k=w.cu_k, device=device)
        self.params = X.make_params(stride=w.stride, threshold=self.tau, est_scale=self.est_scale,
                                    softmax_scale=self.softmax_scale, kv_chunk_tokens=w.kv_chunk_tokens,
                                    select_mode=self.mode, group_agg=self.agg, num_to_choose=num_to_choose)
        self.ws = X.alloc_workspace(self.shape, self.params, device)
        sh = self.shape
        self.B, self.hq, self.hkv = sh.batch, sh.num_q_heads, sh.num_kv_heads
        self.max_qb, self.max_kb = sh.max_qb, sh.max_kb
        self.device = device

    # ---- GPU stages
    def estimate(self):
        bs = torch.full((self.B, self.hq, self.max_qb, self.max_kb), float("nan"), device=self.device)
        X.xattn_estimate(self.shape, self.params, self.q, self.k, bs, self.ws)
        torch.cuda.synchronize()
        return bs

    def select(self, bs):
        mask = torch.full((self.B, self.hkv, self.max_qb, self.max_kb), 7, dtype=torch.uint8, device=self.device)
        hist = torch.full((self.B, max(self.max_kb, 1)), 7, dtype=torch.uint8, device=self.device)
        counts = torch.full((self.B, 2), -1, dtype=torch.int32, device=self.device)
        X.xattn_select(self.shape, self.params, bs.to(self.device).contiguous(), mask, hist, counts, self.ws)
        torch.cuda.synchronize()
        return mask, hist, counts

    def attend(self, mask):
        out = torch.full_like(self.q, float("nan"))
        lse = torch.full((self.hq, self.shape.total_q), float("nan"), device=self.device)
        X.xattn_sparse_attn(self.shape, self.params, self.q, self.k, self.v,
                            mask.to(self.device, torch.uint8).contiguous(), out, lse, self.ws)
        torch.cuda.synchronize()
        return out, lse

    def prefill(self):
        out = torch.full_like(self.q, float("nan"))
        lse = torch.full((self.hq, self.shape.total_q), float("nan"), device=self.device)
        counts = torch.full((self.B, 2), -1, dtype=torch.int32, device=self.device)
        aux = {
            "block_sums": torch.empty((self.B, self.hq, self.max_qb, self.max_kb), device=self.device),
            "mask_kv": torch.empty((self.B, self.hkv, self.max_qb, self.max_kb), dtype=torch.uint8,
                                   device=self.device),
            "hist_sel": torch.empty((self.B, max(self.max_kb, 1)), dtype=torch.uint8, device=self.device),
        }
        X.xattn_prefill_chunk(self.shape, self.params, self.q, self.k, self.v, out, lse, counts, self.ws,
                              aux=aux)
        torch.cuda.synchronize()
        return out, lse, counts, aux

    # ---- oracle on the same inputs
    def oracle(self, attention=True, rows=None):
        w = self.w
        kw = dict(num_kv_heads=w.num_kv_heads, stride=w.stride, threshold=self.tau,
                  est_scale=self.est_scale, softmax_scale=self.softmax_scale,
                  kv_chunk_tokens=w.kv_chunk_tokens, mode=self.mode, agg=self.agg,
                  attention=attention, rows=rows, num_to_choose=self.num_to_choose)
        if self.paged:
            return O.prefill(w.q, None, None, w.cu_q, w.cu_k, block_table=w.block_table.numpy(),
                             k_cache=w.k_cache, v_cache=w.v_cache, **kw)
        return O.prefill(w.q, w.k, w.v, w.cu_q, w.cu_k, **kw)

    def oracle_attention(self, mask, rows=None):
        """Oracle O7 on a given effective mask [B,Hkv,maxQb,maxKb]."""
        w = self.w
        q = O.to_f64(w.q)
        out = np.full(q.shape, np.nan)
        lse = np.full((w.num_q_heads, q.shape[0]), np.nan)
        k = v = None
        if not self.paged:
            k = O.to_f64(w.k)
            v = O.to_f64(w.v)
        kc = O.to_f64(w.k_cache) if self.paged else None
        vc = O.to_f64(w.v_cache) if self.paged else None
        m = np.asarray(mask.cpu().numpy(), dtype=bool)
        for b in range(w.batch):
            lq, lk = w.lens(b)
            if lq == 0:
                continue
            kb_, vb_ = O.sequence_kv(k, v, w.cu_k, b, None if not self.paged else w.block_table.numpy(),
                                     kc, vc)
            r_b = None if rows is None else rows.get(b, [])
            if r_b is not None and len(r_b) == 0:
                continue
            o_b, l_b = O.sparse_attention(q[w.cu_q[b]:w.cu_q[b + 1]], kb_, vb_,
                                          m[b, :, :lq // 128, :lk // 128],
                                          softmax_scale=self.softmax_scale,
                                          group=w.num_q_heads // w.num_kv_heads, rows=r_b)
            out[w.cu_q[b]:w.cu_q[b + 1]] = o_b
            lse[:, w.cu_q[b]:w.cu_q[b + 1]] = l_b
        return out, lse


def assert_block_sums_close(gpu, ref, stride, label=""):
    g = gpu.detach().cpu().double().numpy()
    rb = 128 // stride
    err = np.abs(g - ref)
    tol = BS_RTOL * np.abs(ref) + 1e-7 * rb
    bad = err > tol
    assert not np.isnan(g).any(), label + ": NaN in block sums"
    assert not bad.any(), "%s: %d/%d block sums out of tolerance; worst rel %.3g" % (
        label, int(bad.sum()), bad.size, float((err / np.maximum(np.abs(ref), 1e-30)).max()))


def assert_attention_close(out, lse, ref_out, ref_lse, dtype, rows_idx=None, label=""):
    o = out.detach().float().cpu().double().numpy()
    l_ = lse.detach().cpu().double().numpy()
    if rows_idx is not None:
        o = o[rows_idx]
        ref_out = ref_out[rows_idx]
        l_ = l_[:, rows_idx]
        ref_lse = ref_lse[:, rows_idx]
    assert np.isfinite(o).all(), label + ": non-finite output"
    do = np.abs(o - ref_out).max()
    dl = np.abs(l_ - ref_lse).max()
    assert do <= OUT_ATOL[dtype], "%s: max |out - oracle| = %.3g" % (label, do)
    assert dl <= LSE_ATOL[dtype], "%s: max |lse - oracle| = %.3g" % (label, dl)
    return do, dl


def sample_rows(w, per_seq=96, seed=0):
    """Query rows spread over every q block of every sequence (first, last and
    random rows of each block)."""
    rng = np.random.default_rng(seed)
    rows = {}
    flat = []
    for b in range(w.batch):
        lq, _ = w.lens(b)
        if lq == 0:
            rows[b] = []
            continue
        picks = set()
        for i in range(lq // 128):
            picks.update({i * 128, i * 128 + 127})
        picks.update(int(x) for x in rng.choice(lq, size=min(per_seq, lq), replace=False))
        rows[b] = sorted(picks)
        flat.extend(w.cu_q[b] + x for x in rows[b])
    return rows, np.asarray(flat)


# Acceptance of masks on inputs whose threshold cuts may sit arbitrarily close
# to a flip: a (q head, q block) row is FIRM when its oracle selection margin
# (oracle.selection_margin) is at least MARGIN_DELTA = 5e-3, or exceeds twice
# the row's measured block-sum error sum_j |gpu - oracle| / T.  The second
# bound is a proof, not a heuristic: every cumulative sum and the total move
# by at most that error, so neither a "before < tau*T" test nor the order of
# the two items at the cut can change.  Firm rows must select bit-exactly;
# the others are counted and reported.
MARGIN_DELTA = 5e-3


def check_selection(r, ref, gpu_bs, gpu_mask, gpu_hist=None, label=""):
    """Compare the GPU's effective mask (and history vote) with the oracle's
    under the rule above; returns (mismatch fraction, soft rows, firm rows).

    Per-KV-head mode: a (kv head, q block) row must match when all q-head
    rows of its group are firm.  Chunk-vote modes: with U kv rows holding a
    soft q-head row, history block j's vote can move by at most U, so
    hist_sel[j] must match unless that can cross the strict majority; the
    current chunk must always match when dense causal (chunk_vote) and on
    firm rows when selected per KV head (chunk_vote_sparse)."""
    w = r.w
    group = w.num_q_heads // w.num_kv_heads
    hkv = w.num_kv_heads
    g_bs = gpu_bs.detach().cpu().double().numpy()
    g_mask = gpu_mask.detach().cpu().numpy().astype(bool)
    g_hist = None if gpu_hist is None else gpu_hist.detach().cpu().numpy().astype(bool)
    mism_el = tot_el = 0
    soft_rows = firm_rows = 0
    for b in range(w.batch):
        lq, lk = w.lens(b)
        qb, kb = lq // 128, lk // 128
        if qb == 0:
            continue
        kh = kb - qb
        firm = np.zeros((w.num_q_heads, qb), dtype=bool)
        for h in range(w.num_q_heads):
            for i in range(qb):
                ro = ref["block_sums"][b, h, i, :i + kh + 1]
                rg = g_bs[b, h, i, :i + kh + 1]
                t = ro.sum()
                err = np.abs(rg - ro).sum() / t if t > 0 else np.inf
                m = O.selection_margin(ro, r.tau)
                firm[h, i] = (m >= MARGIN_DELTA) or (m > 2.0 * err * 1.001 + 1e-12)
        soft_rows += int((~firm).sum())
        firm_rows += int(firm.sum())
        kv_firm = firm.reshape(hkv, group, qb).all(axis=1)  # [Hkv, Qb]
        gm = g_mask[b, :, :qb, :kb]
        om = ref["mask_kv"][b, :, :qb, :kb]
        mism_el += int((gm != om).sum())
        tot_el += gm.size
        if r.mode == "per_kvhead":
            bad = (gm != om).any(axis=2) & kv_firm
            assert not bad.any(), "%s: seq %d: %d firm (kv head, q block) rows differ" % (label, b, int(bad.sum()))
        else:
            if r.mode == "chunk_vote":
                # current chunk: dense causal on both sides
                assert (gm[:, :, kh:] == om[:, :, kh:]).all(), "%s: seq %d: current-chunk mask differs" % (label, b)
            else:
                # current chunk per KV head: firm rows must match
                bad = (gm[:, :, kh:] != om[:, :, kh:]).any(axis=2) & kv_firm
                assert not bad.any(), "%s: seq %d: %d firm current-chunk rows differ" % (label, b, int(bad.sum()))
            if kh > 0:
                u = int((~kv_firm).sum())
                votes = ref["mask_q"][b, :, :qb, :kh].reshape(hkv, group, qb, kh)
                per_kv = votes.any(axis=1) if r.agg == "any" else (2 * votes.sum(axis=1) > group)
                v = per_kv.sum(axis=(0, 1))
                n = hkv * qb
                firm_j = (2 * (v - u) > n) | (2 * (v + u) <= n)
                firm_j[0] = firm_j[kh - 1] = True  # forced
                oh = ref["hist_sel"][b, :kh]
                gh = gm[0, 0, :kh] if g_hist is None else g_hist[b, :kh]
                bad = (gh != oh) & firm_j
                assert not bad.any(), "%s: seq %d: %d firm history votes differ" % (label, b, int(bad.sum()))
                bad = (gm[:, :, :kh] != oh[None, None, :]) & firm_j[None, None, :]
                assert not bad.any(), "%s: seq %d: effective history mask differs on firm votes" % (label, b)
    frac = mism_el / max(tot_el, 1)
    metrics.record("mask " + label, mismatch=frac, soft_rows=soft_rows, firm_rows=firm_rows)
    return frac, soft_rows, firm_rows


def runs_of(sel):
    """(first, count) runs of consecutive selected blocks."""
    sel = np.asarray(sel, dtype=bool)
    runs = []
    for j, x in enumerate(sel):
        if x and (j == 0 or not sel[j - 1]):
            runs.append([j, 0])
        if x:
            runs[-1][1] += 1
    return runs


def assert_gapped(hist, kh, label=""):
    """The voted history is a proper, non-contiguous subset: 0 < density < 1
    with at least two runs, so a test on it exercises the sparse paths."""
    h = hist.detach().cpu().numpy()[:kh].astype(bool) if hasattr(hist, "detach") else np.asarray(hist)[:kh]
    n = int(h.sum())
    runs = runs_of(h)
    metrics.record("history " + label, selected=n, of=kh, runs=len(runs))
    assert 0 < n < kh, "%s: %d of %d history blocks voted in" % (label, n, kh)
    assert len(runs) >= 2, "%s: the voted history is one run %s" % (label, runs)
    return runs
