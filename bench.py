"""Benchmark: absorbed MLA decode on one MI355X.

One step = the whole absorbed path over one batch of the DeepSeek-V3-shaped
decode workload (B=64 sequences, H=128 heads, 4096 cached rows each in a
contiguous bf16 latent cache [64, 4096, 576], one query token, seeded Gaussian
inputs): absorb W_UK into the queries, scan the latent cache (split-T), then
merge the splits and project back through W_UV in one fused pass.  Inputs are resident in HBM before the
timed region; each step reads a different one of three cache copies so the
256 MB last-level cache cannot serve a step from the previous one.

Prints one JSON line.  ``value`` is the step's algorithmic TFLOP/s; the line
also carries the algorithmic HBM GB/s, tokens/s, the roofline of the dominant
kernel (the split-T latent scan, timed with HIP events on the stream it runs
on) and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# the split-T kernel's sources: a traffic figure taken with hardware counters
# holds only for the code it was taken on
# the sources of each split-T kernel: a counter summary stays valid while
# the digest of its kernel's sources is unchanged
SHARED_SOURCES = ("head_latent_attention_mla_amd/csrc/mla_plan.h",
                  "head_latent_attention_mla_amd/csrc/mla_common.h",
                  "head_latent_attention_mla_amd/csrc/mla_internal.h",
                  "head_latent_attention_mla_amd/csrc/mla_split_store.h")
KERNEL_SOURCES = {"bf16": ("head_latent_attention_mla_amd/csrc/mla_decode.hip",) + SHARED_SOURCES,
                  "fp8math": ("head_latent_attention_mla_amd/csrc/mla_decode_f8.hip",) + SHARED_SOURCES}
COPY_BYTES = 1 << 30         # read (and written) by the copy-kernel calibration run
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
N_COPIES = 3
PART_DTYPE_NAME = "bf16"     # split partials of the decode step: half the fp32 partial traffic


def algorithmic_counts(B, s_q, H, seqlens, causal, cache_elem_bytes=2, scale_bytes=0):
    """FLOPs and bytes by the pages' counting rule: 2 per multiply-add over the
    causally visible (query, cached row) pairs, 2*576 + 2*512 per head and pair;
    a cached row is read once, the latent query read once and the latent output
    written once (split partials are implementation overhead, not counted)."""
    pairs = 0
    rows = 0
    for T in seqlens:
        rows += T
        for j in range(s_q):
            pairs += (T - s_q + j + 1) if causal else T
    f_scan = pairs * H * (2 * 576 + 2 * 512)
    f_absorb = 2 * (2 * B * s_q * H * 128 * 512)
    by_cache = rows * (576 * cache_elem_bytes + scale_bytes)
    by_qlat = B * s_q * H * 576 * 2
    by_olat = B * s_q * H * 512 * 2        # the latent output at its narrowest width (bf16)
    by_weights = 2 * H * 128 * 512 * 2
    by_q, by_out = B * s_q * H * 192 * 2, B * s_q * H * 128 * 2
    return dict(flops_scan=f_scan, flops_step=f_scan + f_absorb,
                bytes_scan=by_cache + by_qlat + by_olat, bytes_cache=by_cache,
                bytes_step=by_cache + by_weights + by_q + by_out)


def kernel_source_digest(kind: str = "bf16") -> str:
    """Digest of the sources of the split-T kernel: "bf16" (decode_split_kernel,
    every workload's scan but the FP8-arithmetic one) or "fp8math"."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the split-T kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration),
    or None when there is none or the kernel has changed since."""
    path = os.path.join(ROOT, "profiles", f"decode_split_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9]+)", text)
    d = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    kind = "fp8math" if workload.endswith("_fp8math") else "bf16"
    if not t or not d or d.group(1) != kernel_source_digest(kind):
        return None
    return int(t.group(1))


def copy_calibration(steps: int):
    """A plain elementwise copy of COPY_BYTES (fp32 negation, one read and one
    write per element), the known-size kernel that scales the HBM counters."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.randn(COPY_BYTES // 4, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    print(json.dumps({"calibration": "copy", "bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                      "us_per_launch": round(us, 2), "copy_gbs": round(2 * COPY_BYTES / us / 1e3, 1)}), flush=True)


def blas_info(pools):
    """The BLAS library numpy runs on (vendor, version, threads in use)."""
    blas = [p for p in pools if p.get("user_api") == "blas"] or list(pools)
    if not blas:
        return {"vendor": "unknown", "threads": 1}
    b = blas[0]
    return {"vendor": b.get("internal_api", "unknown"), "version": b.get("version"),
            "threads": int(b.get("num_threads", 1))}


def measured_peaks(dev):
    """Achievable peaks measured on this GPU: HBM bandwidth of a plain copy
    (read + write of 1 GiB) and dense bf16 matrix throughput of an
    8192^3 library GEMM; the roofline fractions are also quoted against
    these."""
    import torch
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    out = {}
    for name, fn, work in (("hbm_copy_gbs", lambda: dst.copy_(src), 2 * COPY_BYTES / 1e9),
                           ("bf16_gemm_tflops", lambda: torch.mm(a, b), 2 * 8192 ** 3 / 1e12)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(work * 10 / (e0.elapsed_time(e1) * 1e-3), 1)
    del src, dst, a, b
    return out


def cpu_baseline(inp, scale, seconds_target=15.0, selection=None):
    """The fp64 oracle (naive expand-then-attend) on a bounded sample of (b, h)
    pairs of the same workload, scaled to the step's metric: the absorbed-path
    FLOPs of the sampled pairs (the same counting rule as the GPU figure) per
    second of oracle time."""
    import numpy as np
    from threadpoolctl import threadpool_info
    import oracle

    w = inp["workload"]
    rng = np.random.default_rng(0)
    flops, done, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds_target:
        pairs = [(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(4)]
        if selection is None:
            oracle.naive_decode(inp, scale, pairs=pairs)
        else:
            oracle.sparse_decode(inp, selection[0], selection[1], scale, pairs=pairs)
        for b, _ in pairs:
            T = int(inp["seqlens"][b]) if selection is None else int(selection[1][b])
            vis = sum((T - w.s_q + j + 1) if (w.causal and selection is None) else T for j in range(w.s_q))
            flops += vis * (2 * 576 + 2 * 512) + 2 * 2 * 128 * 512 * w.s_q
        done += len(pairs)
    dt = time.perf_counter() - t0
    blas = blas_info(threadpool_info())
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": blas["threads"],
        "host_cores": len(os.sched_getaffinity(0)),
        "blas": blas,
        "kind": "oracle",
        "sample": f"{done} random (sequence, head) pairs of the {w.name} workload (B={w.B} H={w.H} "
                  f"s_q={w.s_q} T={w.T or w.T_range}{'' if selection is None else f' top-{w.topk}'}), "
                  f"fp64 numpy {'naive' if selection is None else 'sparse'} expand-then-attend, {dt:.1f} s; "
                  f"value = absorbed-path FLOPs of those pairs per second",
        "tokens_per_s": done / w.H * w.s_q / dt,
    }


def append_main(args, w):
    """The latent append step alone: N tokens projected through the
    [576, d_model] weight, rotated and stored into the cache.  HBM-bound on
    the weight; the weight rotates over enough copies that the 256 MB
    last-level cache cannot hold them."""
    import torch
    from head_latent_attention_mla_amd import workloads as W
    from head_latent_attention_mla_amd import mla

    print(f"[bench] generating {w}", file=sys.stderr, flush=True)
    inp = W.generate_append(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fp8 = w.cache_dtype == "fp8"

    def bf16(a):
        return torch.from_numpy(a.view("int16")).view(torch.bfloat16).to(dev)

    x = bf16(inp["x"])
    w_bytes = 576 * w.d_model * 2
    n_w = max(2, -(-320 * 2 ** 20 // w_bytes))
    weights = [bf16(inp["w_dkr"])]
    weights += [weights[0].clone() for _ in range(n_w - 1)]
    seq_id = torch.from_numpy(inp["seq_id"]).to(dev)
    pos = torch.from_numpy(inp["pos"]).to(dev)
    n_rows = w.B * w.T_cap
    if w.paged:
        rows = torch.zeros((n_rows // 64, 64, 576), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
        table = torch.arange(n_rows // 64, dtype=torch.int32, device=dev).view(w.B, w.T_cap // 64)
    else:
        rows = torch.zeros((w.B, w.T_cap, 576), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
        table = None
    scale_t = torch.zeros(rows.shape[:2], dtype=torch.float32, device=dev) if fp8 else None
    cache = mla.LatentCache(rows=rows, seqlens=torch.full((w.B,), w.T_cap, dtype=torch.int32, device=dev),
                            max_seqlen=w.T_cap, row_scale=scale_t, block_table=table)
    ws = torch.empty(mla.append_workspace_bytes(w.N, w.d_model), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        mla.latent_append(x, weights[i % n_w], seq_id, pos, cache, 10000.0, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # a call is a few microseconds of GPU work, less than the Python call
    # takes: the timed calls (one per weight copy) are captured once in a HIP
    # graph and replayed, so the GPU, not the host, sets the pace
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n_w):
            step(i)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-args.steps // n_w))
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    n_calls = reps * n_w
    ms = t0.elapsed_time(t1) / n_calls
    s = ms * 1e-3
    row_bytes = 576 * (1 if fp8 else 2) + (4 if fp8 else 0)
    alg_bytes = w_bytes + w.N * w.d_model * 2 + w.N * row_bytes + 8 * w.N
    flops = 2 * w.N * w.d_model * 576
    gbs = alg_bytes / s / 1e9
    rec = {
        "metric": "latent append HBM GB/s (% roofline)",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n_calls,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: N={w.N} tokens, d_model={w.d_model}, W_DKV|W_KR [576, {w.d_model}] bf16, "
                               f"{'paged' if w.paged else 'contiguous'} {w.cache_dtype} cache of {w.B} x {w.T_cap} "
                               f"slots, seed {w.seed}",
                   "global_batch": w.N, "seq_len": w.T_cap, "parallelism": "single GPU"},
        "tokens_per_s": round(w.N / s, 1),
        "roofline": {
            "kernel": "latent append (append_project_kernel + append_finalize_kernel, one call)",
            "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": alg_bytes, "algorithmic_flops_per_launch": flops,
            "avg_launch_us": round(ms * 1e3, 2), "achieved_tflops": round(flops / s / 1e12, 2),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        from threadpoolctl import threadpool_info
        from oracle import latent_append as oracle_append
        from oracle import mla_oracle as oracle
        xs = oracle.bf16_to_f64(inp["x"])
        wd = oracle.bf16_to_f64(inp["w_dkr"])
        done, t_start = 0, time.perf_counter()
        while time.perf_counter() - t_start < min(args.cpu_seconds, 10.0) or done == 0:
            oracle_append.append_rows(xs, wd, inp["pos"], 10000.0)
            done += 1
        dt = time.perf_counter() - t_start
        rec["cpu_baseline"] = {
            "value": round(done * alg_bytes / dt / 1e9, 3), "unit": "GB/s",
            "cores": blas_info(threadpool_info())["threads"], "host_cores": len(os.sched_getaffinity(0)),
            "blas": blas_info(threadpool_info()), "kind": "oracle",
            "sample": f"{done} full calls of the fp64 numpy latent-append oracle on the same {w.N} tokens, {dt:.1f} s",
        }
    print(json.dumps(rec), flush=True)


def prefill_flops(w, seqlens):
    """Expand-path FLOPs of one call: the per-head expansion of every cached
    row (2 T H d_c (d_k + d_v)) and 2 (192 + 128) per head and visible
    (query, row) pair."""
    expand = sum(2 * int(T) * w.H * 512 * 256 for T in seqlens)
    pairs = 0
    for T in seqlens:
        T = int(T)
        if w.causal:
            pairs += sum(T - w.s_q + j + 1 for j in range(w.s_q))
        else:
            pairs += w.s_q * T
    return expand, pairs * w.H * 2 * (192 + 128)


def prefill_main(args, w):
    """The expand (prefill) path alone: one call expands every cached row per
    head and runs causal attention for all s_q query tokens.  MFMA-bound."""
    import torch
    from head_latent_attention_mla_amd import workloads as W
    from head_latent_attention_mla_amd import mla

    scale = 1.0 / math.sqrt(192.0)
    print(f"[bench] generating {w}", file=sys.stderr, flush=True)
    inp = W.generate(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, w_uk, w_uv, cache = W.to_torch(inp, dev)
    out = torch.empty((w.B, w.s_q, w.H, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.prefill_workspace_bytes(w.B, w.s_q, w.H, cache.max_seqlen), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        mla.prefill_expand(q, cache, w_uk, w_uv, scale, causal=w.causal, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    s = ms * 1e-3
    f_expand, f_attn = prefill_flops(w, inp["seqlens"])
    flops = f_expand + f_attn
    tflops = flops / s / 1e12
    rec = {
        "metric": "MLA prefill (expand path) TFLOP/s (% MFMA roofline)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} prompts of {w.s_q} tokens, H={w.H}, "
                               f"{'causal' if w.causal else 'non-causal'}, contiguous {w.cache_dtype} latent cache, "
                               f"seed {w.seed}",
                   "global_batch": w.B, "seq_len": w.s_q, "parallelism": "single GPU"},
        "tokens_per_s": round(w.B * w.s_q / s, 1),
        "roofline": {
            "kernel": "prefill expand path (transpose_wuv + expand_kv_kernel + prefill_attn_kernel, one call)",
            "bound": "mfma", "achieved": round(tflops, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": None,
            "algorithmic_flops_per_launch": flops, "expand_flops": f_expand, "attention_flops": f_attn,
            "avg_launch_us": round(ms * 1e3, 2),
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        import numpy as np
        from threadpoolctl import threadpool_info
        import oracle
        rng = np.random.default_rng(0)
        done, fl, t_start = 0, 0, time.perf_counter()
        while time.perf_counter() - t_start < min(args.cpu_seconds, 20.0) or done == 0:
            b, h = int(rng.integers(w.B)), int(rng.integers(w.H))
            oracle.naive_decode(inp, scale, causal=w.causal, pairs=[(b, h)])
            one = w.with_(B=1, H=1)
            e1, a1 = prefill_flops(one, [inp["seqlens"][b]])
            fl += e1 + a1
            done += 1
        dt = time.perf_counter() - t_start
        rec["cpu_baseline"] = {
            "value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": blas_info(threadpool_info())["threads"], "host_cores": len(os.sched_getaffinity(0)),
            "blas": blas_info(threadpool_info()), "kind": "oracle",
            "sample": f"{done} random (sequence, head) pairs of the {w.name} workload, fp64 numpy expand-then-attend, "
                      f"{dt:.1f} s; value = expand-path FLOPs of those pairs per second",
        }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps from a HIP graph (measured: the same step time as eager "
                         "launches, the gaps between kernels are on the GPU side)")
    ap.add_argument("--fp8-math", action="store_true",
                    help="FP8 caches: run the scan with E4M3 matrix arithmetic (mla_decode_partial_fp8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--naive-steps", type=int, default=3,
                    help="calls of the naive expand-then-attend ablation to time (0: skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run the known-size copy kernel that scales the HBM byte counters")
    ap.add_argument("--kernel-digest", action="store_true",
                    help="print the source digest of the split-T kernel (of the FP8-arithmetic one with --fp8-math)")
    args = ap.parse_args()
    if args.kernel_digest:
        print(kernel_source_digest("fp8math" if args.fp8_math else "bf16"))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this build has no "
              "multi-GPU path; data-parallel attention would shard whole sequences per GPU.", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        copy_calibration(max(args.steps, 1))
        return

    import torch
    from head_latent_attention_mla_amd import workloads as W
    from head_latent_attention_mla_amd import mla

    if args.workload in W.APPEND_WORKLOADS:
        append_main(args, W.APPEND_WORKLOADS[args.workload])
        return
    w = W.WORKLOADS[args.workload]
    if w.name == "prefill":
        prefill_main(args, w)
        return
    scale = 1.0 / math.sqrt(192.0)
    print(f"[bench] generating {w}", file=sys.stderr, flush=True)
    inp = W.generate(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, w_uk, w_uv, cache0 = W.to_torch(inp, dev)
    caches = [cache0]
    for _ in range(N_COPIES - 1):
        caches.append(mla.LatentCache(rows=cache0.rows.clone(), seqlens=cache0.seqlens, max_seqlen=cache0.max_seqlen,
                                      row_scale=None if cache0.row_scale is None else cache0.row_scale.clone(),
                                      block_table=cache0.block_table))
    B, s_q, H = w.B, w.s_q, w.H
    N = B * s_q
    sparse = w.topk is not None
    f8m = bool(args.fp8_math)
    if f8m and (w.cache_dtype != "fp8" or sparse):
        print("--fp8-math needs a dense FP8-cache workload (fp8_cache)", file=sys.stderr)
        sys.exit(2)
    selection = W.generate_selection(inp) if sparse else None
    q_lat = torch.empty((B, s_q, H, 576), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B, s_q, H, 128), dtype=torch.bfloat16, device=dev)
    if sparse:
        sel_idx = torch.from_numpy(selection[0]).to(dev)
        sel_count = torch.from_numpy(selection[1]).to(dev)
        scan_len = int(sel_idx.shape[1])
        ws = torch.empty(mla.sparse_workspace_bytes(B, s_q, H, scan_len, fp8=cache0.fp8), dtype=torch.uint8,
                         device=dev)
    else:
        scan_len = cache0.max_seqlen
        ws = torch.empty(mla.decode_workspace_bytes(B, s_q, H, scan_len), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    PART_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}[PART_DTYPE_NAME]

    def step(i, ev=None, part_dtype=PART_DTYPE):
        c = caches[i % N_COPIES]
        if ev is not None:
            ev[0].record(stream)
        mla.absorb_q(q.view(N, H, -1), w_uk, out=q_lat.view(N, H, -1))
        if ev is not None:
            ev[1].record(stream)
        if sparse:
            mla.sparse_decode_partial(q_lat, c, sel_idx, sel_count, scale, workspace=ws, part_dtype=part_dtype)
        else:
            mla.decode_partial(q_lat, c, scale, w.causal, workspace=ws, fp8_math=f8m, part_dtype=part_dtype)
        if ev is not None:
            ev[2].record(stream)
        mla.decode_combine_out(ws, w_uv, B, s_q, H, scan_len, out=out.view(N, H, -1), part_dtype=part_dtype)
        if ev is not None:
            ev[3].record(stream)

    def keep_host_ahead():
        # a short spin on the GPU lets the host queue the next launches before
        # the GPU reaches them, so that no timed span holds host launch time
        torch.cuda._sleep(2_000_000)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps, launched one by one; with --graph the steps
    # (one per cache copy) are captured once in a HIP graph and replayed
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    n_timed = args.steps
    if not args.graph:
        torch.cuda.synchronize()
        keep_host_ahead()
        t0.record(stream)
        for i in range(args.steps):
            step(i)
        t1.record(stream)
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(N_COPIES):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, -(-args.steps // N_COPIES))
        n_timed = reps * N_COPIES
        keep_host_ahead()
        t0.record(stream)
        for _ in range(reps):
            graph.replay()
        t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / n_timed

    # statistics pass: at least 50 steps with HIP events on the launch stream
    # at every kernel boundary (recorded back to back, read after one
    # synchronisation): per-step median / p10 / p90 and per-kernel durations
    fused_gather = sparse and not cache0.paged and not cache0.fp8
    scan_name = ("decode_split (gather fused)" if fused_gather else "sparse_gather+decode_split") if sparse \
        else "decode_split"
    names = ["absorb_q", scan_name, "combine_out"]
    n_stats = max(args.steps, 50)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(n_stats)]
    torch.cuda.synchronize()
    keep_host_ahead()
    for i in range(n_stats):
        step(i, evs[i])
    torch.cuda.synchronize()
    spans = {n: [evs[i][k].elapsed_time(evs[i][k + 1]) * 1e3 for i in range(n_stats)] for k, n in enumerate(names)}
    step_ms = [evs[i][0].elapsed_time(evs[i][len(names)]) for i in range(n_stats)]

    def pct(v, q):
        v = sorted(v)
        return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]

    kern_us = {n: sum(v) / len(v) for n, v in spans.items()}
    step_stats = {"steps": n_stats, "median_ms": round(pct(step_ms, 0.5), 5), "p10_ms": round(pct(step_ms, 0.1), 5),
                  "p90_ms": round(pct(step_ms, 0.9), 5),
                  "kernel_median_us": {n: round(pct(v, 0.5), 2) for n, v in spans.items()},
                  "kernel_p10_us": {n: round(pct(v, 0.1), 2) for n, v in spans.items()},
                  "kernel_p90_us": {n: round(pct(v, 0.9), 2) for n, v in spans.items()}}

    # the same step with fp32 split partials (the scope's default precision)
    if True:
        torch.cuda.synchronize()
        for i in range(3):
            step(i, part_dtype=torch.float32)
        torch.cuda.synchronize()
        keep_host_ahead()
        t0.record(stream)
        for i in range(args.steps):
            step(i, part_dtype=torch.float32)
        t1.record(stream)
        torch.cuda.synchronize()
        fp32_step_ms = t0.elapsed_time(t1) / args.steps

    fp8 = w.cache_dtype == "fp8"
    peak_mfma = FP8_PEAK_TFLOPS if f8m else BF16_PEAK_TFLOPS
    rows_read = [int(x) for x in (selection[1] if sparse else inp["seqlens"])]
    cnt = algorithmic_counts(B, s_q, H, rows_read, w.causal and not sparse,
                             cache_elem_bytes=1 if fp8 else 2, scale_bytes=4 if fp8 else 0)
    s = ms_per_step * 1e-3
    tflops = cnt["flops_step"] / s / 1e12
    split_s = kern_us[names[1]] * 1e-6
    scan_gbs = cnt["bytes_scan"] / split_s / 1e9
    scan_tflops = cnt["flops_scan"] / split_s / 1e12
    # the path at s_q = 1 with a bf16 cache sits below the bf16 ridge (HBM-bound);
    # more query tokens per cached row or an fp8 cache push it past (MFMA-bound)
    hbm_bound = (not fp8) and s_q == 1
    roofline = {
        "kernel": ("split-T scan gathering the selected rows (counted once)" if fused_gather
                   else "sparse gather + split-T scan (selected rows counted once)" if sparse
                   else "decode_split_f8 (split-T latent scan, E4M3 arithmetic)" if f8m
                   else "decode_split (split-T latent scan)"),
        "bound": "hbm" if hbm_bound else "mfma",
        "achieved": round(scan_gbs if hbm_bound else scan_tflops, 1),
        "peak": HBM_PEAK_GBS if hbm_bound else peak_mfma,
        "unit": "GB/s" if hbm_bound else "TFLOP/s",
        "frac": round((scan_gbs / HBM_PEAK_GBS) if hbm_bound else (scan_tflops / peak_mfma), 4),
        "traffic": measured_traffic(w.name + ("_fp8math" if f8m else "")),
        "algorithmic_bytes_per_launch": cnt["bytes_scan"],
        "algorithmic_flops_per_launch": cnt["flops_scan"],
        "avg_launch_us": round(kern_us[names[1]], 2),
        "median_launch_us": step_stats["kernel_median_us"][names[1]],
        "achieved_tflops": round(scan_tflops, 1),
        "achieved_gbs": round(scan_gbs, 1),
    }
    peaks = measured_peaks(dev)
    meas = peaks["hbm_copy_gbs"] if hbm_bound else (None if f8m else peaks["bf16_gemm_tflops"])
    roofline["peak_measured"] = meas
    roofline["peak_measured_how"] = ("1 GiB device copy (read + write)" if hbm_bound
                                     else None if f8m else "8192^3 bf16 library GEMM")
    roofline["frac_of_measured"] = round(roofline["achieved"] / meas, 4) if meas else None
    rec = {
        "metric": "absorbed MLA decode TFLOP/s + HBM GB/s (% roofline), H=128 B=64 T=4096",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": n_timed,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if f8m else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}{' (E4M3 arithmetic)' if f8m else ''}: B={B} H={H} s_q={s_q} T={w.T or w.T_range}"
                               f"{f' top-{w.topk} selected' if sparse else ''} "
                               f"{'paged' if w.paged else 'contiguous'} {w.cache_dtype} latent cache [*, 576], "
                               f"{'causal' if w.causal else 'non-causal'}, {PART_DTYPE_NAME} split partials, "
                               f"seed {w.seed}",
                   "global_batch": B, "seq_len": w.max_T, "parallelism": "single GPU"},
        "step_gbs": round(cnt["bytes_step"] / s / 1e9, 1),
        "tokens_per_s": round(N / s, 1),
        "kernel_us": {k: round(v, 2) for k, v in kern_us.items()},
        "step_stats": step_stats,
        "ms_per_step_fp32_partials": round(fp32_step_ms, 5),
        "measured_peaks": peaks,
        "roofline": roofline,
    }
    if args.naive_steps > 0 and not sparse:
        # the ablation: same inputs and output, every cached row expanded per head
        nws = torch.empty(mla.naive_workspace_bytes(B, s_q, H, cache0.max_seqlen), dtype=torch.uint8, device=dev)
        out_n = torch.empty_like(out)
        mla.naive_decode(q, cache0, w_uk, w_uv, scale, w.causal, out=out_n, workspace=nws)
        torch.cuda.synchronize()
        n0, n1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n0.record(stream)
        for i in range(args.naive_steps):
            mla.naive_decode(q, caches[i % N_COPIES], w_uk, w_uv, scale, w.causal, out=out_n, workspace=nws)
        n1.record(stream)
        torch.cuda.synchronize()
        naive_ms = n0.elapsed_time(n1) / args.naive_steps
        naive_flops = cnt["flops_scan"] // (2 * 576 + 2 * 512) * (2 * 192 + 2 * 128) + \
            sum(int(x) for x in inp["seqlens"]) * H * 2 * (2 * 512 * 128)
        naive_tflops = naive_flops / (naive_ms * 1e-3) / 1e12
        rec["naive_ablation"] = {
            "ms_per_step": round(naive_ms, 4),
            "absorbed_speedup": round(naive_ms / ms_per_step, 2),
            "naive_algorithmic_tflops": round(naive_tflops, 1),
            # the speedup says little unless read beside how close the naive
            # kernel itself runs to its own (bf16 MFMA) roofline
            "naive_frac_of_bf16_peak": round(naive_tflops / BF16_PEAK_TFLOPS, 4),
            "flop_ratio_naive_over_absorbed": round(naive_flops / cnt["flops_scan"], 1),
            "naive_flops": naive_flops,
        }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(inp, scale, args.cpu_seconds, selection)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
