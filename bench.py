"""Throughput of the XAttention block-sparse prefill path on one MI355X.

One step = one whole pass of the hot path (strided estimate + block sums,
threshold / GQA / vote selection, block-sparse attention with LSE) over one
prefill chunk.  Default workload: the 32K-context chunk -- the last 4096
tokens of a Qwen3-0.6B-shaped layer (16 q heads / 8 kv heads, d = 128,
bf16) over 28K tokens of history, stride 8, block 128, threshold 0.9,
chunk-vote selection.  Inputs are synthetic (seeded Gaussian Q/K/V with
planted peaked keys) and resident in HBM before the timed region starts.
Other workloads (--workload) are the 4K layer, the paged varlen batch, the
128K context streamed from pinned host memory through the 4-slot ring, the
tiny fp32 layer, and two sparse regimes at the 32K shape.

Prints one JSON line.  "ms_per_step" is the whole timed region over the
steps; "step_ms" gives the median and minimum of per-step event pairs
recorded inside it.  "roofline" is for the dominant kernel, the bf16 sparse
attention kernel, timed alone by the library's event pairs around each of its
launches (xattn_kernel_timing) on the stream it is launched on, while
xattn_attn_run runs ("attn_call_ms" is the whole call: the kernel, then the
merge of split rows); algorithmic flops = 4*d per visible selected (query, key) pair
per q head.  "sparse_regimes" repeats the step and the attention roofline on
the 32K shape with inputs whose selection is genuinely sparse.
"other_configs" gives the step time of the other workloads (the tiny fp32
layer, the 4K layer, the paged batch, the 128K ring) measured in the same
run.  "achievable" states what this machine reaches on a large bf16 GEMM (hipBLASLt
through torch.matmul) and on a device copy, next to the published peaks.
"cpu_baseline" times the float64 oracle on a bounded sample of the same
workload on the host cores.

``--summarize-profile DIR`` instead reduces the rocprofv3 CSV output of one
workload (the commands are listed in the summary) to
profiles/kernels_<workload>.md.
"""

import argparse
import csv
import glob
import hashlib
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
PEAK_FP32_VALU_TFLOPS = 157.3  # 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (dual issue) x 2.4 GHz
CSRC = os.path.join(ROOT, "block_sparse_attention_strided_amd", "csrc")
SPARSE_STAGES = ("chunked_prefill_32k_sparse_vote", "chunked_prefill_32k_sparse_kvhead")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="chunked_prefill_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sparse-stages", action="store_true",
                    help="skip the sparse-regime stages measured next to the 32K headline")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the step time of the other workloads measured next to the 32K headline")
    ap.add_argument("--cpu-sample-rows", type=int, default=3072,
                    help="query rows of the oracle attention sample (scaled to the chunk)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy kernel (reference for PMC byte counters)")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the large-GEMM and copy rate measurement")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="write profiles/kernels_<workload>.md from rocprofv3 output under DIR and exit")
    return ap.parse_args()


def source_hash(name):
    return hashlib.sha256(open(os.path.join(CSRC, name), "rb").read()).hexdigest()[:16]


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


def dense_attention_flops(cu_q, cu_k, hq, d):
    """The same count for every causal-allowed block (density 1)."""
    pairs = 0
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        qb, kh = lq // 128, (lk - lq) // 128
        pairs += sum((i + kh) * 128 * 128 + 128 * 129 // 2 for i in range(qb))
    return 4.0 * d * pairs * hq


def estimate_flops(cu_q, cu_k, hq, stride, d):
    """2*s*d per allowed reshaped score cell (c <= r + (Lk-Lq)/s)."""
    tot = 0
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        r_n, o_s = lq // stride, (lk - lq) // stride
        tot += sum(min(lk // stride, r + o_s + 1) for r in range(r_n))
    return 2.0 * stride * d * tot * hq


def profiled_traffic(workload, profiles_dir=None):
    """HBM bytes per attention launch from the committed rocprofv3 summary of
    this workload, or None if the attention source changed since then."""
    path = os.path.join(profiles_dir or os.path.join(ROOT, "profiles"), "kernels_%s.md" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if ("attention.hip %s" % source_hash("attention.hip")) not in text:
        return None
    for line in text.splitlines():
        if line.startswith("attention traffic_bytes_per_launch:"):
            return int(line.split(":")[1])
    return None


def time_region(fn, steps, stream):
    """Mean ms per call over one event pair around `steps` calls."""
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


def time_steps(fn, steps, stream):
    """(whole-region ms per step, per-step ms list): one event pair around the
    region, and one event recorded between consecutive steps inside it."""
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for x in range(steps):
        fn()
        ev[x + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[x].elapsed_time(ev[x + 1]) for x in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, per


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


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


def cpu_baseline(w, sample_rows):
    """float64 oracle on the host: estimate + select over the whole chunk,
    attention on a sample of query rows scaled to all rows.  BLAS threads are
    set to the cores this process may run on."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O

    cores = len(os.sched_getaffinity(0))
    kw = dict(num_kv_heads=w.num_kv_heads, stride=w.stride, threshold=w.threshold,
              kv_chunk_tokens=w.kv_chunk_tokens, mode=w.select_mode)
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] + [1])
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
            kb_, vb_ = O.sequence_kv(k, v, w.cu_k, b, None if w.block_table is None else w.block_table.numpy(),
                                     kc, vc)
            O.sparse_attention(q[w.cu_q[b]:w.cu_q[b + 1]], kb_, vb_, res["mask_kv"][b][:, : lq // 128, : lk // 128],
                               softmax_scale=1.0 / math.sqrt(w.head_dim), group=w.num_q_heads // w.num_kv_heads,
                               rows=rows)
        t_at = time.perf_counter() - t1
    t_total = t_es + t_at * total_q / n_s
    return {
        "value": total_q / t_total,
        "unit": "query-tokens/s",
        "cores": used,
        "affinity_cores": cores,
        "kind": "oracle",
        "sample": "float64 NumPy oracle on the same inputs: estimate+select over all %d query rows (%.1f s) + "
                  "attention for %d sampled rows (%.1f s) scaled to all rows" % (total_q, t_es, n_s, t_at),
    }


class Case:
    """A workload resident on the device with its C-ABI objects and the
    outputs of one step."""

    def __init__(self, w, dev):
        import torch

        import block_sparse_attention_strided_amd as X

        self.X, self.w, self.dev = X, w, dev
        self.ring = None
        self.q = w.q.to(dev)
        lq0, lk0 = w.lens(0)
        self.hist_blocks = (lk0 - lq0) // 128
        table = None
        if w.ring:
            kh = self.hist_blocks
            self.k_hist = torch.empty((kh, 128, w.num_kv_heads, w.head_dim), dtype=w.dtype, pin_memory=True)
            self.v_hist = torch.empty_like(self.k_hist, pin_memory=True)
            self.k_hist.copy_(w.k[: lk0 - lq0].reshape(self.k_hist.shape))
            self.v_hist.copy_(w.v[: lk0 - lq0].reshape(self.v_hist.shape))
            self.k, self.v = w.k[lk0 - lq0:].to(dev), w.v[lk0 - lq0:].to(dev)
            self.ring = X.Ring(w.ring_slots, w.ring_slot_blocks, w.num_kv_heads, w.head_dim, w.dtype)
        elif w.block_table is not None:
            self.k, self.v = w.k_cache.to(dev), w.v_cache.to(dev)
            table = w.block_table.to(dev).contiguous()
        else:
            self.k, self.v = w.k.to(dev), w.v.to(dev)
        self.table = table
        self.sh = X.Shape(num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, dtype=w.dtype,
                          cu_q=w.cu_q, cu_k=w.cu_k, device=dev, block_table=table,
                          num_phys_blocks=0 if table is None else w.k_cache.shape[0])
        self.pr = X.make_params(stride=w.stride, threshold=w.threshold, kv_chunk_tokens=w.kv_chunk_tokens,
                                select_mode=w.select_mode, group_agg=w.group_agg)
        self.ws = X.alloc_workspace(self.sh, self.pr, dev)
        sh = self.sh
        B, hq, hkv = sh.batch, sh.num_q_heads, sh.num_kv_heads
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((hq, sh.total_q), device=dev)
        self.counts = torch.empty((B, 2), dtype=torch.int32, device=dev)
        self.bs = torch.empty((B, hq, sh.max_qb, sh.max_kb), device=dev)
        self.mask = torch.empty((B, hkv, sh.max_qb, sh.max_kb), dtype=torch.uint8, device=dev)
        self.hist = torch.empty((B, sh.max_kb), dtype=torch.uint8, device=dev)
        self.aux = {"block_sums": self.bs, "mask_kv": self.mask, "hist_sel": self.hist}

    def step(self, params=None, aux=None, counts="default"):
        X = self.X
        pr = self.pr if params is None else params
        aux = self.aux if aux is None else aux
        counts = self.counts if counts == "default" else counts
        if self.ring is None:
            X.xattn_prefill_chunk(self.sh, pr, self.q, self.k, self.v, self.out, self.lse, counts, self.ws, aux=aux)
        else:
            X.xattn_prefill_chunk(self.sh, pr, self.q, self.k, self.v, self.out, self.lse, counts, self.ws, aux=aux,
                                  ring=self.ring, k_hist=self.k_hist, v_hist=self.v_hist,
                                  hist_blocks=self.hist_blocks)

    def density(self):
        return [c[0] / c[1] if c[1] else None for c in self.counts.cpu().tolist()]

    def kernel_stages(self, steps, stream):
        """Each stage alone (resident K/V only), and the attention roofline
        over the selected pairs of the current mask."""
        X, w = self.X, self.w
        st = {}
        st["estimate_ms"] = time_region(lambda: X.xattn_estimate(self.sh, self.pr, self.q, self.k, self.bs, self.ws),
                                        steps, stream)
        st["select_ms"] = time_region(
            lambda: X.xattn_select(self.sh, self.pr, self.bs, self.mask, self.hist, self.counts, self.ws), steps, stream)
        st["attn_plan_ms"] = time_region(lambda: X.xattn_attn_plan(self.sh, self.pr, self.v, self.mask, self.ws),
                                         steps, stream)
        X.xattn_attn_plan(self.sh, self.pr, self.v, self.mask, self.ws)
        run = lambda: X.xattn_attn_run(self.sh, self.pr, self.q, self.k, self.v, self.mask, self.out, self.lse,
                                       self.ws)
        # the whole call (the attention kernel, then the merge of split rows)
        st["attn_call_ms"] = time_region(run, steps, stream)
        # the attention kernel alone: the library's event pairs around each of
        # its launches, on the stream it is launched on
        X.xattn_kernel_timing(True)
        try:
            time_region(run, steps, stream)
            total_ms, launches = X.xattn_kernel_timing_read()
        finally:
            X.xattn_kernel_timing(False)
        ms_attn = total_ms / max(1, launches)
        st["attn_kernel_ms"] = ms_attn
        hq, hkv = self.sh.num_q_heads, self.sh.num_kv_heads
        flops = attention_flops(self.mask, w.cu_q, w.cu_k, hq // hkv, w.head_dim)
        e_fl = estimate_flops(w.cu_q, w.cu_k, hq, w.stride, w.head_dim)
        st["estimate_flops"] = e_fl
        st["estimate_tflops"] = e_fl / (st["estimate_ms"] * 1e-3) / 1e12
        st["estimate_frac"] = st["estimate_tflops"] / PEAK_BF16_TFLOPS
        st["attn_flops"] = flops
        st["attn_pair_density"] = flops / dense_attention_flops(w.cu_q, w.cu_k, hq, w.head_dim)
        achieved = flops / (ms_attn * 1e-3) / 1e12
        bf16 = w.dtype.itemsize == 2
        peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_VALU_TFLOPS
        roofline = {
            "kernel": "attn_pp (block-sparse flash attention, bf16 MFMA, ping-pong)" if bf16
                      else "attn_f32 (block-sparse flash attention, fp32 VALU)",
            "bound": "mfma" if bf16 else "alu",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": profiled_traffic(w.name),
            "flops_per_launch": flops,
        }
        # leave this case's step outputs in place
        self.step()
        return st, roofline

    def close(self):
        if self.ring is not None:
            self.ring.close()
            self.ring = None


def sparse_regime(name, steps, warmup, dev, stream):
    """Step and attention roofline of one sparse-regime workload."""
    from workloads import make_workload

    w = make_workload(name)
    c = Case(w, dev)
    for _ in range(warmup):
        c.step()
    ms, per = time_steps(c.step, steps, stream)
    dens = c.density()
    st, roof = c.kernel_stages(steps, stream)
    c.close()
    return {
        "workload": name,
        "description": w.description,
        "select_mode": w.select_mode,
        "density": dens,
        "attn_pair_density": st["attn_pair_density"],
        "ms_per_step": ms,
        "step_ms_median": median(per),
        "step_ms_min": min(per),
        "query_tokens_per_s": w.total_q / (ms * 1e-3),
        "estimate_ms": st["estimate_ms"],
        "select_ms": st["select_ms"],
        "attn_kernel_ms": st["attn_kernel_ms"],
        "attn_call_ms": st["attn_call_ms"],
        "attn_roofline": {k: roof[k] for k in ("achieved", "peak", "unit", "frac", "flops_per_launch")},
    }


# The other workloads, each timed briefly next to the 32K headline.
OTHER_CONFIGS = ("tiny_causal_fp32_1k", "qwen3_0p6b_4k", "paged_varlen_3seq", "qwen3_4b_128k_ring")


def other_config(name, steps, warmup, dev, stream):
    """Whole-step time of one more workload (its own warmup, then `steps`)."""
    from workloads import make_workload

    w = make_workload(name)
    c = Case(w, dev)
    for _ in range(warmup):
        c.step()
    ms, per = time_steps(c.step, steps, stream)
    dens = c.density()
    c.close()
    return {
        "workload": name,
        "ms_per_step": ms,
        "step_ms_median": median(per),
        "query_tokens_per_s": w.total_q / (ms * 1e-3),
        "steps": steps,
        "density": dens,
        "kv": "ring (pinned host history)" if w.ring else ("paged" if w.block_table is not None else "contiguous"),
    }


def reuse_accuracy(dev, mixes=(0.0, 0.2, 0.5, 1.0)):
    """Selection reuse across layers measured against the layer's own
    selection: synthetic layer pairs at the 32K shape whose block ranks
    partly agree (a fraction `mix` of the blocks trade ranks), layer B run
    once on its own estimate and once on layer A's mask."""
    import torch

    from workloads import make_layer_pair

    kw = dict(hq=16, hkv=8, d=128, lq=[4096], lk=[32768], stride=8, threshold=0.9, select_mode="chunk_vote",
              kv_chunk_tokens=4096, rank_step=0.04)
    rows = []
    for mix in mixes:
        wa, wb = make_layer_pair(203, mix, **kw)
        ca, cb = Case(wa, dev), Case(wb, dev)
        ca.step()
        cb.step()
        torch.cuda.synchronize()
        own_out, own_lse, own_mask = cb.out.float().clone(), cb.lse.clone(), cb.mask.clone()
        reuse = cb.X.make_params(stride=wb.stride, threshold=wb.threshold, kv_chunk_tokens=wb.kv_chunk_tokens,
                                 select_mode=wb.select_mode, reuse_selection=1)
        cb.step(reuse, {"mask_kv": ca.mask, "hist_sel": ca.hist}, None)
        torch.cuda.synchronize()
        err = cb.out.float() - own_out
        rows.append({
            "mix": mix,
            "mask_mismatch": float((ca.mask != own_mask).float().mean()),
            "density_own": cb.density()[0],
            "density_reused": ca.density()[0],
            "out_max_abs_err": float(err.abs().max()),
            "out_rel_err": float(err.norm() / own_out.norm()),
            "lse_max_abs_err": float((cb.lse - own_lse).abs().max()),
        })
        ca.close()
        cb.close()
        del ca, cb
    return {"workload": "layer pairs at the 32K chunk's shape (well-separated, shared ranks, step 0.04; "
                        "chunk vote); layer B on its own selection vs on layer A's", "pairs": rows}


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X (got --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch

    import block_sparse_attention_strided_amd as X
    from workloads import make_workload

    w = make_workload(args.workload)
    dev = "cuda"
    c = Case(w, dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        c.step()
    torch.cuda.synchronize()
    ms, per = time_steps(c.step, args.steps, stream)
    dens = c.density()

    stages = {"step_ms_median": median(per), "step_ms_min": min(per)}
    # the same step reusing this step's selection (another layer sharing it):
    # no estimate, no selection, and in ring mode no history K streamed for them
    pr_reuse = X.make_params(stride=w.stride, threshold=w.threshold, kv_chunk_tokens=w.kv_chunk_tokens,
                             select_mode=w.select_mode, group_agg=w.group_agg, reuse_selection=1)
    aux_reuse = {"mask_kv": c.mask, "hist_sel": c.hist}
    c.step(pr_reuse, aux_reuse, None)
    torch.cuda.synchronize()
    stages["reuse_selection_step_ms"] = time_region(lambda: c.step(pr_reuse, aux_reuse, None),
                                                    max(1, min(args.steps, 10)), stream)
    c.step()
    torch.cuda.synchronize()
    roofline = None
    if c.ring is None:
        st, roofline = c.kernel_stages(args.steps, stream)
        stages.update(st)
    res = {
        "metric": METRIC,
        "value": c.sh.total_q / (ms * 1e-3),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded Gaussian Q/K/V, 8 planted peaked keys per kv head)"
                if not w.name.startswith("chunked_prefill_32k_sparse") else "synthetic (" + w.description + ")",
        "config": {
            "workload": w.name,
            "q_heads": c.sh.num_q_heads, "kv_heads": c.sh.num_kv_heads, "head_dim": w.head_dim,
            "query_tokens": c.sh.total_q, "context_tokens": [w.cu_k[b + 1] - w.cu_k[b] for b in range(c.sh.batch)],
            "stride": w.stride, "block": 128, "threshold": w.threshold, "select_mode": w.select_mode,
            "kv": "ring (pinned host history, %d x %d-block slots)" % (w.ring_slots, w.ring_slot_blocks)
                  if c.ring is not None else ("paged" if c.table is not None else "contiguous"),
            "density": dens,
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
    if c.ring is not None:
        # write-back of the chunk's K/V to pinned host memory (offload stream),
        # timed alone: D2H link rate of the step after the path
        lq0, lk0 = w.lens(0)
        nb = lq0 // 128
        hkv = c.sh.num_kv_heads
        k_dst = torch.empty((nb, 128, hkv, w.head_dim), dtype=w.dtype, pin_memory=True)
        v_dst = torch.empty_like(k_dst, pin_memory=True)

        def wb():
            c.ring.offload_chunk(c.k, c.v, k_dst, v_dst, nb)
            c.ring.offload_wait()

        wb()
        torch.cuda.synchronize()
        wb_ms = time_region(wb, 5, stream)
        res["stages"]["writeback_ms"] = wb_ms
        res["stages"]["writeback_gbs"] = 2 * k_dst.numel() * k_dst.element_size() / (wb_ms * 1e-3) / 1e9
        c.close()
        # the same step through a staged ring: history K in one bulk copy,
        # voted V blocks gathered from mapped pinned memory by a kernel
        staged = X.Ring(1, lk0 // 128, w.num_kv_heads, w.head_dim, w.dtype, staged=True)

        def step_staged():
            X.xattn_prefill_chunk(c.sh, c.pr, c.q, c.k, c.v, c.out, c.lse, c.counts, c.ws, aux=c.aux, ring=staged,
                                  k_hist=c.k_hist, v_hist=c.v_hist, hist_blocks=c.hist_blocks)

        step_staged()
        torch.cuda.synchronize()
        res["stages"]["staged_step_ms"] = time_region(step_staged, max(1, min(args.steps, 10)), stream)
        staged.close()
    if w.name == "chunked_prefill_32k" and not args.no_sparse_stages:
        res["sparse_regimes"] = [sparse_regime(n, min(args.steps, 50), min(args.warmup, 10), dev, stream)
                                 for n in SPARSE_STAGES]
        res["reuse_accuracy"] = reuse_accuracy(dev)
    if w.name == "chunked_prefill_32k" and not args.no_other_configs:
        del c
        res["other_configs"] = [
            other_config(n, min(args.steps, 5) if "ring" in n else min(args.steps, 50),
                         min(args.warmup, 2) if "ring" in n else min(args.warmup, 10), dev, stream)
            for n in OTHER_CONFIGS]
    if not args.no_achievable:
        res["achievable"] = achievable_rates(dev)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_rows)
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------------------
# rocprofv3 summary: profiles/kernels_<workload>.md
# ---------------------------------------------------------------------------

PROFILE_COMMANDS = [
    "rocprofv3 --kernel-trace --stats -f csv -d DIR/prof_{wl} -o trace -- python3 bench.py --workload {wl} "
    "--steps 100 --warmup 20 --no-cpu-baseline --no-achievable --no-sparse-stages --no-other-configs > DIR/prof_{wl}.json",
    "rocprofv3 --pmc FETCH_SIZE -f csv -d DIR/pmc_fetch_{wl} -o pmc -- python3 bench.py --workload {wl} "
    "--steps 3 --warmup 1 --no-cpu-baseline --no-achievable --no-sparse-stages --no-other-configs --copy-calibration",
    "rocprofv3 --pmc WRITE_SIZE -f csv -d DIR/pmc_write_{wl} -o pmc -- python3 bench.py --workload {wl} "
    "--steps 3 --warmup 1 --no-cpu-baseline --no-achievable --no-sparse-stages --no-other-configs --copy-calibration",
    "rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 -f csv -d DIR/pmc_mfma_{wl} -o pmc -- python3 bench.py "
    "--workload {wl} --steps 3 --warmup 1 --no-cpu-baseline --no-achievable --no-sparse-stages --no-other-configs",
    "rocprofv3 --pmc SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE -f csv "
    "-d DIR/pmc_lds_{wl} -o pmc -- python3 bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline "
    "--no-achievable --no-sparse-stages --no-other-configs",
    "python3 bench.py --summarize-profile DIR --workload {wl}",
]


def _one(base, pattern):
    f = sorted(glob.glob(os.path.join(base, pattern), recursive=True))
    return f[0] if f else None


def _short(n):
    return n.replace("xattn::(anonymous namespace)::", "").replace("void ", "").split("(")[0]


NUM_XCDS = 8      # MI355X: XCDs, each with its own clock domain counter
NUM_SIMDS = 1024  # 256 CUs x 4 SIMDs


def _per_kernel(path, counter=None):
    out = {}
    for r in csv.DictReader(open(path)):
        if counter and r.get("Counter_Name") != counter:
            continue
        out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def summarize_profile(base, wl, out_dir=None):
    """Kernel durations (trace), copy-calibrated HBM bytes (FETCH_SIZE,
    WRITE_SIZE) and executed MFMA flops per dispatch for one workload,
    written to <out_dir or profiles/>/kernels_<wl>.md."""
    stats_csv = _one(base, "prof_%s/**/*kernel_stats.csv" % wl)
    if stats_csv is None:
        sys.exit("no kernel_stats.csv under %s/prof_%s" % (base, wl))
    bench = json.loads(open(os.path.join(base, "prof_%s.json" % wl)).read().strip().splitlines()[-1])
    stats = list(csv.DictReader(open(stats_csv)))
    fetch_csv = _one(base, "pmc_fetch_%s/**/*counter_collection.csv" % wl)
    write_csv = _one(base, "pmc_write_%s/**/*counter_collection.csv" % wl)
    mfma_csv = _one(base, "pmc_mfma_%s/**/*counter_collection.csv" % wl)
    st = bench.get("stages", {})
    roof = bench.get("roofline") or {}
    flops = {"attn_pp": roof.get("flops_per_launch"), "attn_mfma": roof.get("flops_per_launch"),
             "est_gemm_bf16": st.get("estimate_flops"), "est_partial_bf16": st.get("estimate_flops")}
    L = ["# rocprofv3 kernel summary: %s" % wl, "",
         "Commands (repo root, on the MI355X box, TMPDIR=/tmp; DIR = the output folder):", ""]
    L += ["    " + c.format(wl=wl) for c in PROFILE_COMMANDS]
    L += ["", "source sha256[:16]: attention.hip %s estimate.hip %s select.hip %s" % (
        source_hash("attention.hip"), source_hash("estimate.hip"), source_hash("select.hip")), ""]
    line = "Bench line of the traced run: %.4f ms per step (median %.4f), %.4g query-tokens/s" % (
        bench["ms_per_step"], st.get("step_ms_median", float("nan")), bench["value"])
    if "attn_kernel_ms" in st:
        line += "; attention kernel alone %.4f ms, estimate alone %.4f ms" % (st["attn_kernel_ms"], st["estimate_ms"])
    L += [line + "; density %s." % bench["config"].get("density"), "",
          "## Kernel durations (kernel trace, all dispatches of the run)", "",
          "| kernel | calls | avg us | min us | max us | share |", "|---|---|---|---|---|---|"]
    avg = {}
    for r in stats:
        n = _short(r["Name"])
        avg[n] = float(r["AverageNs"]) / 1e3
        L.append("| %s | %s | %.1f | %.1f | %.1f | %.1f%% |" % (n, r["Calls"], avg[n], float(r["MinNs"]) / 1e3,
                                                             float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    traffic = None
    if fetch_csv and write_csv:
        fetch, write = _per_kernel(fetch_csv), _per_kernel(write_csv)
        calib = [k for k in fetch if "MulFunctor" in k]
        if calib:
            fv, wv = max(fetch[calib[0]]), max(write[calib[0]])
            ff, wf = (512 << 20) / (fv * 1024), (512 << 20) / (wv * 1024)
            L += ["", "## HBM traffic and rates per dispatch", "",
                  "Calibration: a plain elementwise copy (`torch.mul(x, 1.0, out=y)`, 512 MiB read + 512 MiB "
                  "written) reads FETCH_SIZE %.0f KiB and WRITE_SIZE %.0f KiB, so FETCH_SIZE is scaled by %.3f and "
                  "WRITE_SIZE by %.3f. Rates use the average trace duration above; MFMA rates count the method's "
                  "algorithmic flops (attention 4*d per visible selected (query, key) pair, estimate 2*s*d per "
                  "allowed reshaped score cell) against 2500 TFLOP/s, HBM rates against 8000 GB/s." % (fv, wv, ff, wf),
                  "",
                  "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | read MiB | written MiB | HBM GB/s | HBM frac | "
                  "algorithmic TFLOP/s | MFMA frac |", "|---|---|---|---|---|---|---|---|---|"]
            for k in fetch:
                if k in calib or "rocclr" in k or "FillFunctor" in k:
                    continue
                n = _short(k)
                fm = sum(fetch[k]) / len(fetch[k])
                wlist = write.get(k, [0.0])
                wm = sum(wlist) / len(wlist)
                rb, wb = fm * 1024 * ff, wm * 1024 * wf
                t = avg.get(n)
                gbs = (rb + wb) / (t * 1e-6) / 1e9 if t else float("nan")
                fl = flops.get(n.split("<")[0])
                tf = fl / (t * 1e-6) / 1e12 if (fl and t) else None
                L.append("| %s | %.0f | %.0f | %.1f | %.1f | %.0f | %.3f | %s | %s |" % (
                    n, fm, wm, rb / 2 ** 20, wb / 2 ** 20, gbs, gbs / PEAK_HBM_GBS,
                    "%.0f" % tf if tf else "-", "%.3f" % (tf / PEAK_BF16_TFLOPS) if tf else "-"))
                if n.split("<")[0] in ("attn_pp", "attn_mfma"):
                    traffic = rb + wb
    if mfma_csv:
        mops = _per_kernel(mfma_csv, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        L += ["", "## MFMA counters per dispatch", "",
              "Executed bf16 MFMA flops = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 (the counter counts 512-flop units; "
              "the attention executes the masked halves of its diagonal blocks too); executed TFLOP/s divides them "
              "by the average trace duration above.", "",
              "| kernel | executed GFLOP | algorithmic GFLOP | executed TFLOP/s | frac of 2500 |",
              "|---|---|---|---|---|"]
        for k, v in mops.items():
            if not v or max(v) == 0:
                continue
            n = _short(k)
            ex = sum(v) / len(v) * 512
            t = avg.get(n)
            fl = flops.get(n.split("<")[0])
            L.append("| %s | %.1f | %s | %s | %s |" % (
                n, ex / 1e9, "%.1f" % (fl / 1e9) if fl else "-", "%.0f" % (ex / (t * 1e-6) / 1e12) if t else "-",
                "%.3f" % (ex / (t * 1e-6) / 1e12 / PEAK_BF16_TFLOPS) if t else "-"))
    lds_csv = _one(base, "pmc_lds_%s/**/*counter_collection.csv" % wl)
    if lds_csv:
        cnt = {c: _per_kernel(lds_csv, c) for c in ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
                                                     "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")}
        L += ["", "## LDS and MFMA busy cycles per dispatch", "",
              "SQ_VALU_MFMA_BUSY_CYCLES sums the MFMA pipe's busy cycles over all SIMDs (it equals the executed "
              "MFMA count times each instruction's cycles). GRBM_GUI_ACTIVE sums the GPU's active clock cycles "
              "over its %d XCDs, so GRBM_GUI_ACTIVE / %d is the dispatch's length in shader clocks (which includes "
              "launch overhead, so it reads long for dispatches of a few microseconds). The MFMA busy fraction "
              "divides the first by %d SIMDs times that length; the clock column divides that length by the trace "
              "duration. Bank-conflict stalls are given as a share of the LDS's active cycles." % (
                  NUM_XCDS, NUM_XCDS, NUM_SIMDS), "",
              "| kernel | LDS active cycles | bank-conflict cycles | conflict share | MFMA busy cycles | "
              "shader clocks | clock GHz | MFMA busy frac |", "|---|---|---|---|---|---|---|---|"]

        def mean(c, k):
            v = cnt[c].get(k, [])
            return sum(v) / len(v) if v else 0.0

        for k in cnt["SQ_LDS_IDX_ACTIVE"]:
            if "rocclr" in k or "Functor" in k:
                continue
            n = _short(k)
            a_, bc = mean("SQ_LDS_IDX_ACTIVE", k), mean("SQ_LDS_BANK_CONFLICT", k)
            mb, clocks = mean("SQ_VALU_MFMA_BUSY_CYCLES", k), mean("GRBM_GUI_ACTIVE", k) / NUM_XCDS
            t = avg.get(n)
            L.append("| %s | %.4g | %.4g | %s | %.4g | %.4g | %s | %s |" % (
                n, a_, bc, "%.3f" % (bc / a_) if a_ else "-", mb, clocks,
                "%.2f" % (clocks / (t * 1e3)) if t else "-",
                "%.3f" % (mb / (NUM_SIMDS * clocks)) if (clocks and mb) else "-"))
    if traffic is not None:
        L += ["", "attention traffic_bytes_per_launch: %d" % int(traffic)]
    out = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "kernels_%s.md" % wl)
    with open(out, "w") as f:
        f.write("\n".join(L) + "\n")
    print(out)


if __name__ == "__main__":
    main()
