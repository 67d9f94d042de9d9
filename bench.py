"""Throughput of the XAttention block-sparse prefill path on one MI355X.

One step = one whole pass of the hot path (strided estimate + block-sum,
threshold/GQA/vote selection, block-sparse attention with LSE) over one
prefill chunk of the 32K-context workload: a 4096-token chunk of a
Qwen3-0.6B-shaped layer (16 q heads / 8 kv heads, d = 128, bf16) over 28K
tokens of history, stride 8, block 128, threshold 0.9, chunk-vote selection.
Inputs are synthetic (seeded Gaussian Q/K/V with planted peaked keys) and
resident in HBM before the timed region starts.

Prints one JSON line (rank 0).  The roofline entry is for the dominant
kernel (the sparse attention), timed alone with HIP events on the stream it
is launched on; algorithmic flops = 4*d per visible selected (query, key)
pair per q head.  The cpu_baseline entry times the float64 oracle on a
bounded sample of the same workload on the host cores.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse prefill query-tokens/s at 32K ctx (estimate+select+attn); % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="chunked_prefill_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=96,
                    help="query rows of the oracle attention sample (scaled to the chunk)")
    ap.add_argument("--stages", action="store_true", help="also print per-stage timings to stderr")
    return ap.parse_args()


def attention_flops(mask, cu_q, cu_k, group, d):
    """4*d per visible (query, key) pair over the selected blocks, per q head."""
    import numpy as np

    m = mask.cpu().numpy().astype(bool)
    pairs = 0
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        qb, kh = lq // 128, (lk - lq) // 128
        for i in range(qb):
            sel = m[b, :, i, : i + kh + 1]  # [hkv, n]
            full = sel[:, : i + kh].sum()
            diag = sel[:, i + kh].sum()
            pairs += int(full) * 128 * 128 + int(diag) * (128 * 129 // 2)
    return 4.0 * d * pairs * group


def block_sum_bytes(cu_q, cu_k, hq, stride):
    """Algorithmic bytes of the block-sum kernel: each allowed per-block
    partial read once, the block sums written once."""
    rb = 128 // stride
    tot = 0
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        qb, kh, kb = lq // 128, (lk - lq) // 128, lk // 128
        for i in range(qb):
            tot += (i + kh + 1) * rb * 4 + kb * 4
    return tot * hq


def time_region(fn, steps, stream):
    import torch

    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record(stream)
    for _ in range(steps):
        fn()
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


def cpu_baseline(w, sample_rows):
    import numpy as np

    import oracle as O

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = int(os.environ.get("OMP_NUM_THREADS", "1"))
    t0 = time.perf_counter()
    res = O.prefill(w.q, w.k, w.v, w.cu_q, w.cu_k, num_kv_heads=w.num_kv_heads, stride=w.stride,
                    threshold=w.threshold, kv_chunk_tokens=w.kv_chunk_tokens, mode=w.select_mode,
                    attention=False)
    t_es = time.perf_counter() - t0
    lq = w.cu_q[1] - w.cu_q[0]
    rng = np.random.default_rng(0)
    rows = sorted(int(x) for x in rng.choice(lq, size=min(sample_rows, lq), replace=False))
    kh = (w.cu_k[1] - w.cu_k[0] - lq) // 128
    t1 = time.perf_counter()
    O.sparse_attention(O.to_f64(w.q), O.to_f64(w.k), O.to_f64(w.v), res["mask_kv"][0][:, : lq // 128, :],
                       softmax_scale=1.0 / math.sqrt(w.head_dim), group=w.num_q_heads // w.num_kv_heads,
                       rows=rows)
    t_at = time.perf_counter() - t1
    t_total = t_es + t_at * lq / len(rows)
    return {
        "value": lq / t_total,
        "unit": "query-tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "float64 oracle: estimate+select over the full chunk (%.1f s) + attention for %d of %d "
                  "query rows (%.1f s), attention scaled to all rows; history blocks %d" % (
                      t_es, len(rows), lq, t_at, kh),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_sparse_attention_strided_amd as X
    from workloads import make_workload

    w = make_workload(args.workload)
    dev = "cuda"
    q, k, v = w.q.to(dev), w.k.to(dev), w.v.to(dev)
    sh = X.Shape(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, dtype=w.dtype,
                 cu_q=w.cu_q, cu_k=w.cu_k, device=dev)
    pr = X.make_params(stride=w.stride, threshold=w.threshold, kv_chunk_tokens=w.kv_chunk_tokens,
                       select_mode=w.select_mode, group_agg=w.group_agg)
    ws = X.alloc_workspace(sh, pr, dev)
    B, hq, hkv = sh.batch, sh.num_q_heads, sh.num_kv_heads
    out = torch.empty_like(q)
    lse = torch.empty((hq, sh.total_q), device=dev)
    counts = torch.empty((B, 2), dtype=torch.int32, device=dev)
    bs = torch.empty((B, hq, sh.max_qb, sh.max_kb), device=dev)
    mask = torch.empty((B, hkv, sh.max_qb, sh.max_kb), dtype=torch.uint8, device=dev)
    hist = torch.empty((B, sh.max_kb), dtype=torch.uint8, device=dev)
    aux = {"block_sums": bs, "mask_kv": mask, "hist_sel": hist}
    stream = torch.cuda.current_stream()

    def step():
        X.xattn_prefill_chunk(sh, pr, q, k, v, out, lse, counts, ws, aux=aux)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms = time_region(step, args.steps, stream)

    # dominant kernel alone: sparse attention over the mask this step selected
    def attn():
        X.xattn_sparse_attn(sh, pr, q, k, v, mask, out, lse, ws)

    def est():
        X.xattn_estimate(sh, pr, q, k, bs, ws)

    def sel():
        X.xattn_select(sh, pr, bs, mask, hist, counts, ws)

    attn()
    ms_attn = time_region(attn, args.steps, stream)
    ms_est = time_region(est, args.steps, stream)
    ms_sel = time_region(sel, args.steps, stream)
    flops = attention_flops(mask, w.cu_q, w.cu_k, hq // hkv, w.head_dim)
    achieved = flops / (ms_attn * 1e-3) / 1e12
    cnt = counts.cpu().tolist()
    total_q = sh.total_q
    res = {
        "metric": METRIC,
        "value": total_q / (ms * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian Q/K/V, 8 planted peaked keys per kv head)",
        "config": {
            "workload": w.name,
            "q_heads": hq, "kv_heads": hkv, "head_dim": w.head_dim,
            "chunk_tokens": total_q, "context_tokens": w.cu_k[-1],
            "stride": w.stride, "block": 128, "threshold": w.threshold, "select_mode": w.select_mode,
            "density": [c[0] / c[1] if c[1] else None for c in cnt],
        },
        "stages_ms": {"estimate": ms_est, "select": ms_sel, "attention": ms_attn},
        "roofline": {
            "kernel": "attn_bf16 (block-sparse flash attention)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": None,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
