"""Throughput of the XAttention block-sparse prefill path on one MI355X.

One step = one whole pass of the hot path (strided estimate + block sums,
threshold / GQA / vote selection, block-sparse attention with LSE) over one
prefill chunk.  Default workload: the 32K-context chunk -- the last 4096
tokens of a Qwen3-0.6B-shaped layer (16 q heads / 8 kv heads, d = 128,
bf16) over 28K tokens of history, stride 8, block 128, threshold 0.9,
chunk-vote selection.  Inputs are synthetic (seeded Gaussian Q/K/V with
planted peaked keys) and resident in HBM before the timed region starts.
Other workloads (--workload) are the 4K layer, the paged varlen batch and the
128K context streamed from pinned host memory through the 4-slot ring.

Prints one JSON line.  "roofline" is for the dominant kernel, the bf16 sparse
attention (attn_pp), timed alone (xattn_attn_run) with HIP events on the
stream it is launched on; algorithmic flops = 4*d per visible selected
(query, key) pair per q head.  "achievable" states what this machine reaches on
a large bf16 GEMM (hipBLASLt through torch.matmul) and on a device copy, next
to the published peaks.  "cpu_baseline" times the float64 oracle on a
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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="chunked_prefill_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-rows", type=int, default=3072,
                    help="query rows of the oracle attention sample (scaled to the chunk)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy kernel (reference for PMC byte counters)")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the large-GEMM and copy rate measurement")
    return ap.parse_args()


def attention_flops(mask, cu_q, cu_k, group, d):
    """4*d per visible (query, key) pair over the selected blocks, per q head."""
    m = mask.cpu().numpy().astype(bool)
    pairs = 0
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        qb, kh = lq // 128, (lk - lq) // 128
        for i in range(qb):
            sel = m[b, :, i, : i + kh + 1]
            pairs += int(sel[:, : i + kh].sum()) * 128 * 128 + int(sel[:, i + kh].sum()) * (128 * 129 // 2)
    return 4.0 * d * pairs * group


def estimate_flops(cu_q, cu_k, hq, stride, d):
    """2*s*d per allowed reshaped score cell (c <= r + (Lk-Lq)/s)."""
    tot = 0
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        r_n, o_s = lq // stride, (lk - lq) // stride
        tot += sum(min(lk // stride, r + o_s + 1) for r in range(r_n))
    return 2.0 * stride * d * tot * hq


def profiled_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 summary of
    this workload, or None if the attention source changed since then."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "kernels_%s.md" % workload)
    src = os.path.join(ROOT, "block_sparse_attention_strided_amd", "csrc", "attention.hip")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    text = open(path).read()
    if ("attention.hip %s" % h) not in text:
        return None
    for line in text.splitlines():
        if line.startswith("attention traffic_bytes_per_launch:"):
            return int(line.split(":")[1])
    return None


def achievable_rates(dev):
    """This box's rates on a large bf16 GEMM (8192^3, hipBLASLt via
    torch.matmul) and a 512 MiB device copy, timed with HIP events."""
    import torch

    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    ms_g = time_region(lambda: torch.matmul(a, b, out=c), 10, torch.cuda.current_stream())
    x = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    ms_c = time_region(lambda: y.copy_(x), 10, torch.cuda.current_stream())
    del a, b, c, x, y
    gemm = 2.0 * n ** 3 / (ms_g * 1e-3) / 1e12
    copy = 2.0 * (512 << 20) / (ms_c * 1e-3) / 1e9
    return {"gemm_bf16_tflops": gemm, "gemm_frac_of_peak": gemm / PEAK_BF16_TFLOPS,
            "copy_gbs": copy, "copy_frac_of_peak": copy / PEAK_HBM_GBS,
            "gemm": "bf16 8192x8192x8192 torch.matmul (hipBLASLt), 10 launches",
            "copy": "512 MiB device-to-device copy_, 10 launches, read+write bytes"}


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
    """float64 oracle on the host: estimate + select over the whole chunk,
    attention on a sample of query rows scaled to all rows."""
    import numpy as np

    import oracle as O

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = int(os.environ.get("OMP_NUM_THREADS", "1"))
    kw = dict(num_kv_heads=w.num_kv_heads, stride=w.stride, threshold=w.threshold,
              kv_chunk_tokens=w.kv_chunk_tokens, mode=w.select_mode)
    t0 = time.perf_counter()
    if w.block_table is not None:
        res = O.prefill(w.q, None, None, w.cu_q, w.cu_k, block_table=w.block_table.numpy(), k_cache=w.k_cache,
                        v_cache=w.v_cache, attention=False, **kw)
    else:
        res = O.prefill(w.q, w.k, w.v, w.cu_q, w.cu_k, attention=False, **kw)
    t_es = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    total_q = w.total_q
    n_s = min(sample_rows, total_q)
    flat = sorted(int(x) for x in rng.choice(total_q, size=n_s, replace=False))
    q = O.to_f64(w.q)
    k = v = kc = vc = None
    if w.block_table is None:
        k, v = O.to_f64(w.k), O.to_f64(w.v)
    else:
        kc, vc = O.to_f64(w.k_cache), O.to_f64(w.v_cache)
    t1 = time.perf_counter()
    for b in range(w.batch):
        rows = [x - w.cu_q[b] for x in flat if w.cu_q[b] <= x < w.cu_q[b + 1]]
        if not rows:
            continue
        lq, lk = w.lens(b)
        kb_, vb_ = O.sequence_kv(k, v, w.cu_k, b, None if w.block_table is None else w.block_table.numpy(), kc, vc)
        O.sparse_attention(q[w.cu_q[b]:w.cu_q[b + 1]], kb_, vb_, res["mask_kv"][b][:, : lq // 128, : lk // 128],
                           softmax_scale=1.0 / math.sqrt(w.head_dim), group=w.num_q_heads // w.num_kv_heads,
                           rows=rows)
    t_at = time.perf_counter() - t1
    t_total = t_es + t_at * total_q / n_s
    return {
        "value": total_q / t_total,
        "unit": "query-tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "float64 NumPy oracle on the same inputs: estimate+select over all %d query rows (%.1f s) + "
                  "attention for %d sampled rows (%.1f s) scaled to all rows" % (total_q, t_es, n_s, t_at),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_sparse_attention_strided_amd as X
    from workloads import make_workload

    w = make_workload(args.workload)
    dev = "cuda"
    ring = None
    q = w.q.to(dev)
    lq0, lk0 = w.lens(0)
    if w.ring:
        kh = (lk0 - lq0) // 128
        k_hist = torch.empty((kh, 128, w.num_kv_heads, w.head_dim), dtype=w.dtype, pin_memory=True)
        v_hist = torch.empty_like(k_hist, pin_memory=True)
        k_hist.copy_(w.k[: lk0 - lq0].reshape(k_hist.shape))
        v_hist.copy_(w.v[: lk0 - lq0].reshape(v_hist.shape))
        k, v = w.k[lk0 - lq0:].to(dev), w.v[lk0 - lq0:].to(dev)
        ring = X.Ring(w.ring_slots, w.ring_slot_blocks, w.num_kv_heads, w.head_dim, w.dtype)
        table = None
    elif w.block_table is not None:
        k, v = w.k_cache.to(dev), w.v_cache.to(dev)
        table = w.block_table.to(dev).contiguous()
    else:
        k, v = w.k.to(dev), w.v.to(dev)
        table = None
    sh = X.Shape(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, dtype=w.dtype,
                 cu_q=w.cu_q, cu_k=w.cu_k, device=dev, block_table=table,
                 num_phys_blocks=0 if table is None else w.k_cache.shape[0])
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
        if ring is None:
            X.xattn_prefill_chunk(sh, pr, q, k, v, out, lse, counts, ws, aux=aux)
        else:
            X.xattn_prefill_chunk(sh, pr, q, k, v, out, lse, counts, ws, aux=aux, ring=ring,
                                  k_hist=k_hist, v_hist=v_hist, hist_blocks=(lk0 - lq0) // 128)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms = time_region(step, args.steps, stream)
    cnt = counts.cpu().tolist()

    stages = {}
    # the same step reusing this step's selection (another layer sharing it):
    # no estimate, no selection, and in ring mode no history K streamed for them
    pr_reuse = X.make_params(stride=w.stride, threshold=w.threshold, kv_chunk_tokens=w.kv_chunk_tokens,
                             select_mode=w.select_mode, group_agg=w.group_agg, reuse_selection=1)
    aux_reuse = {"mask_kv": mask, "hist_sel": hist}

    def step_reuse():
        if ring is None:
            X.xattn_prefill_chunk(sh, pr_reuse, q, k, v, out, lse, None, ws, aux=aux_reuse)
        else:
            X.xattn_prefill_chunk(sh, pr_reuse, q, k, v, out, lse, None, ws, aux=aux_reuse, ring=ring,
                                  k_hist=k_hist, v_hist=v_hist, hist_blocks=(lk0 - lq0) // 128)

    step_reuse()
    torch.cuda.synchronize()
    stages["reuse_selection_step_ms"] = time_region(step_reuse, max(1, min(args.steps, 10)), stream)
    step()
    torch.cuda.synchronize()
    roofline = None
    if ring is None:
        def est():
            X.xattn_estimate(sh, pr, q, k, bs, ws)

        def sel():
            X.xattn_select(sh, pr, bs, mask, hist, counts, ws)

        def plan():
            X.xattn_attn_plan(sh, pr, v, mask, ws)

        def run():
            X.xattn_attn_run(sh, pr, q, k, v, mask, out, lse, ws)

        stages["estimate_ms"] = time_region(est, args.steps, stream)
        stages["select_ms"] = time_region(sel, args.steps, stream)
        stages["attn_plan_ms"] = time_region(plan, args.steps, stream)
        plan()
        ms_attn = time_region(run, args.steps, stream)
        stages["attn_kernel_ms"] = ms_attn
        flops = attention_flops(mask, w.cu_q, w.cu_k, hq // hkv, w.head_dim)
        achieved = flops / (ms_attn * 1e-3) / 1e12
        e_fl = estimate_flops(w.cu_q, w.cu_k, hq, w.stride, w.head_dim)
        stages["estimate_flops"] = e_fl
        stages["estimate_tflops"] = e_fl / (stages["estimate_ms"] * 1e-3) / 1e12
        roofline = {
            "kernel": "attn_pp (block-sparse flash attention, bf16 MFMA, ping-pong)",
            "bound": "mfma",
            "achieved": achieved,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": profiled_traffic(w.name),
            "flops_per_launch": flops,
        }
        step()
        torch.cuda.synchronize()
    res = {
        "metric": METRIC,
        "value": sh.total_q / (ms * 1e-3),
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
            "query_tokens": sh.total_q, "context_tokens": [w.cu_k[b + 1] - w.cu_k[b] for b in range(B)],
            "stride": w.stride, "block": 128, "threshold": w.threshold, "select_mode": w.select_mode,
            "kv": "ring (pinned host history, %d x %d-block slots)" % (w.ring_slots, w.ring_slot_blocks)
                  if ring is not None else ("paged" if table is not None else "contiguous"),
            "density": [c[0] / c[1] if c[1] else None for c in cnt],
        },
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if args.copy_calibration:
        x = torch.empty(512 << 20, dtype=torch.uint8, device=dev).view(torch.float32)
        y = torch.empty_like(x)
        x.fill_(1.0)
        for _ in range(5):
            torch.mul(x, 1.0, out=y)
        torch.cuda.synchronize()
        res["copy_calibration"] = {"bytes_read": x.numel() * 4, "bytes_written": y.numel() * 4,
                                   "kernel": "elementwise mul by 1.0 (torch), 5 launches"}
    if ring is not None:
        # write-back of the chunk's K/V to pinned host memory (offload stream),
        # timed alone: D2H link rate of the step after the path
        nb = lq0 // 128
        k_dst = torch.empty((nb, 128, hkv, w.head_dim), dtype=w.dtype, pin_memory=True)
        v_dst = torch.empty_like(k_dst, pin_memory=True)

        def wb():
            ring.offload_chunk(k, v, k_dst, v_dst, nb)
            ring.offload_wait()

        wb()
        torch.cuda.synchronize()
        wb_ms = time_region(wb, 5, stream)
        res["stages"]["writeback_ms"] = wb_ms
        res["stages"]["writeback_gbs"] = 2 * k_dst.numel() * k_dst.element_size() / (wb_ms * 1e-3) / 1e9
        ring.close()
        # the same step through a staged ring: history K in one bulk copy,
        # voted V blocks gathered from mapped pinned memory by a kernel
        staged = X.Ring(1, lk0 // 128, w.num_kv_heads, w.head_dim, w.dtype, staged=True)

        def step_staged():
            X.xattn_prefill_chunk(sh, pr, q, k, v, out, lse, counts, ws, aux=aux, ring=staged,
                                  k_hist=k_hist, v_hist=v_hist, hist_blocks=(lk0 - lq0) // 128)

        step_staged()
        torch.cuda.synchronize()
        res["stages"]["staged_step_ms"] = time_region(step_staged, max(1, min(args.steps, 10)), stream)
        staged.close()
    if not args.no_achievable:
        res["achievable"] = achievable_rates(dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_rows)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
