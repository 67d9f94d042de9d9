"""xattn_prefill_chunk_static: the resident prefill on the library's static
per-device scratch (no workspace argument, no device allocation), checked
against xattn_prefill_chunk on a caller workspace.  Both run the same kernels,
so every output must be bit-identical; two calls in a row, the second with a
smaller input, show that nothing left in the shared scratch by a call leaks
into the next."""

import pytest
import torch

import block_sparse_attention_strided_amd as X
from tests.gpu_util import Run, say
from workloads import make_random, make_workload

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _static(r, with_aux):
    out = torch.full_like(r.q, float("nan"))
    lse = torch.full((r.hq, r.shape.total_q), float("nan"), device="cuda")
    counts = torch.full((r.B, 2), -1, dtype=torch.int32, device="cuda")
    aux = None
    if with_aux:
        aux = {"block_sums": torch.empty((r.B, r.hq, r.max_qb, r.max_kb), device="cuda"),
               "mask_kv": torch.empty((r.B, r.hkv, r.max_qb, r.max_kb), dtype=torch.uint8, device="cuda"),
               "hist_sel": torch.empty((r.B, max(r.max_kb, 1)), dtype=torch.uint8, device="cuda")}
    X.xattn_prefill_chunk_static(r.shape, r.params, r.q, r.k, r.v, out, lse, counts, aux=aux)
    torch.cuda.synchronize()
    return out, lse, counts, aux


def _compare(w, with_aux):
    r = Run(w)
    say("static scratch: %s, workspace %d MiB" % (w.name, r.ws.numel() >> 20))
    assert r.ws.numel() <= 256 << 20
    o0, l0, c0, a0 = r.prefill()
    o1, l1, c1, a1 = _static(r, with_aux)
    assert torch.equal(o0, o1), w.name
    assert torch.equal(l0, l1), w.name
    assert torch.equal(c0, c1), w.name
    if with_aux:
        for key in ("block_sums", "mask_kv", "hist_sel"):
            assert torch.equal(a0[key], a1[key]), key


def test_static_scratch_matches_the_workspace_path_on_consecutive_calls():
    # 1: the 32K chunk (about 105 MiB of scratch); 2: a smaller paged varlen
    # batch with an empty sequence, its masks left in the scratch
    _compare(make_workload("chunked_prefill_32k"), with_aux=True)
    _compare(make_random("static_small", seed=97, hq=8, hkv=4, d=128, lq=[512, 0, 256], lk=[1024, 128, 2048],
                         paged=True, select_mode="per_kvhead"), with_aux=False)


def test_static_scratch_rejects_a_call_that_does_not_fit():
    w = make_random("static_big", seed=98, hq=32, hkv=8, d=128, lq=[8192], lk=[16384], select_mode="chunk_vote")
    sh = X.Shape(num_q_heads=32, num_kv_heads=8, head_dim=128, dtype=w.dtype, cu_q=w.cu_q, cu_k=w.cu_k,
                 device="cuda")
    pr = X.make_params()
    assert X.xattn_workspace_size(sh, pr) > 256 << 20
    q = torch.empty((8192, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(X.XattnError) as ei:
        X.xattn_prefill_chunk_static(sh, pr, q, q, q, q, None, None)
    assert ei.value.code == -2 and "static scratch" in str(ei.value)
