#!/usr/bin/env python3
"""Benchmark of the paged KV-cache attention hot path on one MI355X.

One step = the whole hot path over one batch: the block copies the step's
copy-on-write needs, the slot_mapping scatter of the step's new K/V
(pa_cache_write), then attention over the paged cache (pa_decode:
partition kernel then log-sum-exp merge, or pa_varlen).  The block tables
and slot mapping come from the library's host block manager before timing.

Inputs are seeded synthetic tensors resident in HBM before the timed
region.  To keep the 256 MB Infinity Cache from serving KV reads that a
real step would take from HBM, the timed steps rotate over R identical
copies of the KV pool, R chosen so that R x (KV bytes read per step)
exceeds four times the cache.

Prints one JSON line on stdout (details on stderr).  `value` is the
whole-step KV-read throughput in GB/s: algorithmic KV bytes per step
(every context token's K and V row, each unique physical slot once) x
steps / timed seconds, the K steps launched back to back between one pair
of HIP events.  `roofline` prices the partition kernel alone (for a varlen
step, the whole pa_varlen call), from a second timed region of K
back-to-back launches over the same rotating pools between one pair of
HIP events on the stream they run on, against the 8 TB/s HBM peak; its `traffic` comes from the committed rocprofv3 FETCH_SIZE /
WRITE_SIZE summary of the same kernel and workload, and is null when the
kernel source has changed since those counters were taken.
`cpu_baseline` times the CPU oracle on a bounded sample of the same
workload.  A varlen step made of prefill chunks only (mixed_varlen_prefill)
is a contraction: its line reports TFLOP/s of causal QK^T and PV and prices
the pa_varlen call against the dense bf16 matrix-core peak.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 matrix-core peak of one MI355X
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="gqa_decode_b32",
                   choices=["tiny_f32_decode", "gqa_decode_b32", "long_ctx_decode",
                            "parallel_sampling_cow", "mixed_varlen",
                            "gqa_decode_b32_fp8", "long_ctx_decode_fp8", "beam_search",
                            "prefix_cache", "mixed_varlen_prefill", "mixed_varlen_fp8",
                            "chunked_prefill_long", "parallel_sampling_cow_1020",
                            "long_ctx_decode_tp8_share"])
    p.add_argument("--layout", default="rotated", choices=["rotated", "plain"],
                   help="KV head order inside a cache slot (pa_layout)")
    p.add_argument("--partition", type=int, default=-1,
                   help="split-K partition size (0: library choice; -1: the workload's)")
    p.add_argument("--rotate", type=int, default=0, help="KV pool copies (0: automatic)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time for the oracle baseline (0 disables it)")
    p.add_argument("--json-out", default="", help="also write the JSON line to this file")
    p.add_argument("--print-source-hash", action="store_true",
                   help="print the decode kernel source hash used to match counter summaries")
    p.add_argument("--mode", default="step", choices=["step", "copy", "swap"],
                   help="copy: time pa_copy_blocks over a known byte count (counter "
                        "calibration); swap: pa_swap_blocks between the GPU pool and pinned "
                        "host memory, against plain host-link copies of the same bytes")
    return p.parse_args()


def kernel_source_hash():
    """Hash of the decode kernels' sources (kernel, device code, helpers)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("decode.hip", "decode_body.h", "decode_mfma.h", "common.h", "kernels.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_158_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_kernel_name(w):
    """The decode partition kernel a workload's step launches: the
    matrix-core one for bf16 / FP8 caches, head dim 128 and 4..16 query
    heads per KV head, the vector one otherwise."""
    g = w.num_heads // w.num_kv_heads
    mfma = w.dtype == "bf16" and w.head_dim == 128 and 4 <= g <= 16
    return "decode_mfma_kernel" if mfma else "decode_partition_kernel"


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed counter summary, if still current."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("decode_hip_sha256_16") != kernel_source_hash():
        return None
    return int(t["traffic_bytes_per_launch"])


def unique_kv_bytes(tables, lens, B, hkv, D, elem):
    import numpy as np
    slots = []
    for r in range(len(lens)):
        L = int(lens[r])
        if L == 0:
            continue
        t = np.arange(L)
        slots.append(tables[r, t // B].astype(np.int64) * B + t % B)
    if not slots:
        return 0, 0
    allv = np.concatenate(slots)
    uniq = np.unique(allv).size
    return uniq * 2 * hkv * D * elem, allv.size * 2 * hkv * D * elem


def cpu_baseline(w, seconds):
    """Time the CPU oracle (as written, untuned) on the first n sequences of the batch."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention, run as orun
    st = orun.run_script(w)  # cache fill: setup, not timed
    slots = st.step_slots[-1]
    n_all = len(w.batch)
    per_tok = 2 * w.num_kv_heads * w.head_dim * w.cache_elem_bytes
    fp8 = w.kv_dtype == "fp8"

    def timed(n):
        kc, vc = st.k_cache.copy(), st.v_cache.copy()
        t0 = time.perf_counter()
        if fp8:
            attention.cache_write_fp8(w.final.k[:n], w.final.v[:n], slots[:n], kc, vc,
                                      w.k_scale, w.v_scale)
            attention.decode(w.q[:n], kc, vc, st.block_tables[:n], st.context_lens[:n], w.scale,
                             w.dtype, w.num_kv_heads, cache_dtype="fp8", k_scale=w.k_scale,
                             v_scale=w.v_scale)
        else:
            attention.cache_write(w.final.k[:n], w.final.v[:n], slots[:n], kc, vc)
            attention.decode(w.q[:n], kc, vc, st.block_tables[:n], st.context_lens[:n], w.scale,
                             w.dtype, w.num_kv_heads)
        return time.perf_counter() - t0

    def sample(threads, budget):
        with threadpool_limits(limits=threads):
            t1 = timed(1)
            n = max(1, min(n_all, int(budget / max(t1, 1e-6))))
            reps, dt = 0, 0.0
            while reps == 0 or dt < budget:  # the whole sample, repeated to fill the budget
                dt += timed(n)
                reps += 1
        return n, reps, dt

    # one BLAS thread, and every core this process may use; the oracle's
    # per-head NumPy calls are small, so more threads need not be faster:
    # the faster of the two is the baseline, with the threads it used
    runs = []
    for threads in sorted({1, max(1, len(os.sched_getaffinity(0)))}):
        n, reps, dt = sample(threads, seconds / 2)
        kv = int(st.context_lens[:n].sum()) * per_tok * reps
        runs.append((kv / dt / 1e9, threads, n, reps, dt))
    best = max(runs)
    gbs, threads, n, reps, dt = best
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"final step (cache write + decode) of the first {n} of {n_all} sequences "
                      f"({int(st.context_lens[:n].sum())} context tokens) x {reps}, fp64 NumPy, "
                      f"{threads} BLAS thread{'s' if threads > 1 else ''}, {dt:.2f} s",
            "tokens_per_s": round(n * reps / dt, 3),
            "by_threads": {str(r[1]): round(r[0], 4) for r in runs}}


def cpu_baseline_varlen(w, seconds, prefill_only):
    """Time the CPU oracle (as written, untuned) on a bounded row sample of a
    varlen step: every decode row, and every k-th row of each prefill chunk,
    k chosen to fill about `seconds`.  The oracle's cost per row grows with
    the keys it attends, so the full step's oracle time is the sample's time
    scaled by (keys x heads of all rows) / (keys x heads of the sampled
    rows); the line reports the algorithmic KV bytes (or, prefill chunks
    only, the causal flops) of one step over that time."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import attention, run as orun
    st = orun.run_script(w)  # cache fill: setup, not timed
    qsl, lens = st.query_start_loc, st.context_lens
    rows_all, keys = [], []
    for s in range(len(lens)):
        a, b = int(qsl[s]), int(qsl[s + 1])
        for i in range(b - a):
            rows_all.append((a + i, b - a > 1))
            keys.append(int(lens[s]) - (b - a) + i + 1)
    keys = np.asarray(keys, np.float64)

    def sample(k):
        return [r for j, (r, pre) in enumerate(rows_all) if not pre or j % k == 0]

    def timed(rows):
        pairs = [(r, h) for r in rows for h in range(w.num_heads)]
        t0 = time.perf_counter()
        attention.varlen(w.q, qsl, lens, st.k_cache, st.v_cache, st.block_tables, w.scale,
                         w.dtype, w.num_kv_heads, pairs)
        return time.perf_counter() - t0

    threads = 1
    with threadpool_limits(limits=threads):
        k = 64
        t = timed(sample(k))
        while t < seconds / 4 and k > 1:  # denser samples until the budget is used
            k = max(1, k // 4)
            t = timed(sample(k))
    rows = sample(k)
    frac = keys[[r for r in rows]].sum() / keys.sum()
    t_full = t / frac
    per_tok = 2 * w.num_kv_heads * w.head_dim * w.cache_elem_bytes
    kv, _ = unique_kv_bytes(st.block_tables, lens, w.block_size, w.num_kv_heads, w.head_dim,
                            w.cache_elem_bytes)
    line = {"unit": "GB/s", "value": round(float(kv / t_full / 1e9), 4), "cores": threads,
            "kind": "oracle",
            "sample": f"oracle varlen attention of {len(rows)} of {len(rows_all)} query rows "
                      f"(every decode row, every {k}-th prefill row) x {w.num_heads} heads in "
                      f"{t:.2f} s, fp64 NumPy, 1 BLAS thread; the step's time taken as that "
                      f"x {1 / frac:.2f} (its share of keys x heads)",
            "step_seconds_estimate": round(float(t_full), 3)}
    if prefill_only:
        fl = prefill_flops(qsl, lens, w.num_heads, w.head_dim)
        line.update(unit="TFLOP/s", value=round(float(fl / t_full / 1e12), 6))
    return line


def prefill_flops(qsl, lens, H, D):
    """Causal QK^T and PV flops of the chunks with >= 2 rows (masked work not counted)."""
    total = 0
    for s in range(len(lens)):
        ql = int(qsl[s + 1] - qsl[s])
        if ql < 2:
            continue
        prior = int(lens[s]) - ql
        total += 4 * D * H * (ql * prior + ql * (ql + 1) // 2)
    return int(total)


def copy_calibration(steps):
    """pa_copy_blocks over a known byte count, for scaling the HBM byte counters."""
    import torch
    import paged_kv_cache_158_amd as pa
    nb, B, hkv, D = 8192, 16, 8, 128
    kc = torch.zeros((nb, B, hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    half = nb // 2
    pairs = torch.stack([torch.arange(half), torch.arange(half) + half], 1).int().cuda()
    per_launch = 2 * half * B * hkv * D * 2  # bytes read (== bytes written), K and V
    for _ in range(3):
        pa.copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        pa.copy_blocks(kc, vc, pairs)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    print(json.dumps({"mode": "copy", "kernel": "copy_blocks_kernel",
                      "bytes_read_per_launch": per_launch, "bytes_written_per_launch": per_launch,
                      "read_KiB_per_launch": per_launch / 1024, "avg_launch_us": round(us, 3),
                      "GBps_read_plus_write": round(2 * per_launch / (us * 1e-6) / 1e9, 1)}))


def swap_throughput(steps):
    """pa_swap_blocks of 2048 scattered 64 KiB blocks (bf16, 16 tokens x 8 KV
    heads x 128 dims, K and V) from an 8192-block GPU pool to a pinned host
    pool (swap out) and back to other scattered GPU blocks (swap in), each
    timed over `steps` launches between one event pair.  The same bytes moved
    by one contiguous host-link copy (torch copy_, i.e. the runtime's DMA
    engines) in each direction are the practical ceiling."""
    import torch
    import paged_kv_cache_158_amd as pa
    nb, n, B, hkv, D = 8192, 2048, 16, 8, 128
    gen = torch.Generator(device="cuda").manual_seed(11)
    kc = torch.randn((nb, B, hkv, D), device="cuda", generator=gen).to(torch.bfloat16)
    vc = torch.randn((nb, B, hkv, D), device="cuda", generator=gen).to(torch.bfloat16)
    hk = torch.empty((n, B, hkv, D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty((n, B, hkv, D), dtype=torch.bfloat16, pin_memory=True)
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(12))
    out_pairs = torch.stack([perm[:n], torch.arange(n)], 1).int().cuda()
    in_pairs = torch.stack([torch.arange(n), perm[n:2 * n]], 1).int().cuda()
    per_launch = 2 * n * B * hkv * D * 2  # K and V bytes moved per launch
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / steps

    t_out = timed(lambda: pa.swap_blocks(kc, vc, hk, hv, out_pairs))
    t_in = timed(lambda: pa.swap_blocks(hk, hv, kc, vc, in_pairs))
    dk = kc[:n].contiguous()
    t_d2h = timed(lambda: (hk.copy_(dk, non_blocking=True), hv.copy_(dk, non_blocking=True)))
    t_h2d = timed(lambda: (dk.copy_(hk, non_blocking=True), dk.copy_(hv, non_blocking=True)))
    gbps = lambda us: round(per_launch / (us * 1e-6) / 1e9, 2)
    line = {"mode": "swap", "kernel": "swap_blocks_kernel", "blocks_per_launch": n,
            "bytes_per_launch": per_launch,
            "swap_out_us": round(t_out, 1), "swap_out_GBps": gbps(t_out),
            "swap_in_us": round(t_in, 1), "swap_in_GBps": gbps(t_in),
            "contiguous_copy_d2h_GBps": gbps(t_d2h), "contiguous_copy_h2d_GBps": gbps(t_h2d),
            "swap_out_frac_of_copy": round(t_d2h / t_out, 3),
            "swap_in_frac_of_copy": round(t_h2d / t_in, 3),
            "steps": steps}
    log(f"[bench] swap out {line['swap_out_GBps']} GB/s, in {line['swap_in_GBps']} GB/s; "
        f"contiguous copies d2h {line['contiguous_copy_d2h_GBps']}, h2d "
        f"{line['contiguous_copy_h2d_GBps']} GB/s")
    print(json.dumps(line))


def main():
    args = parse()
    if args.print_source_hash:
        print(kernel_source_hash())
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): this build runs the paged-attention path on a single MI355X; "
              "sharding across GPUs is a design note, not a measured configuration.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import paged_kv_cache_158_amd as pa
    from paged_kv_cache_158_amd.engine import ScriptRunner

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "copy":
        copy_calibration(args.steps)
        return
    if args.mode == "swap":
        swap_throughput(min(args.steps, 20))
        return
    t_setup = time.time()
    w = synth.FULL[args.workload]()
    elem = w.cache_elem_bytes
    layout = pa.LAYOUT_ROTATED if args.layout == "rotated" else pa.LAYOUT_PLAIN
    # the engine orders a decode step's rows by first block, so that rows
    # sharing a prompt prefix are neighbours (the kernels then read it once)
    runner = ScriptRunner(w, dev, fill="zero", layout=layout, group_prefixes=True)
    runner.run_history()
    fin = runner.prepare_final(None if args.partition < 0 else args.partition)
    torch.cuda.synchronize()
    B, hkv, D = w.block_size, w.num_kv_heads, w.head_dim
    kv_unique, kv_logical = unique_kv_bytes(fin.host_tables, fin.host_lens, B, hkv, D, elem)
    pool_bytes = 2 * runner.k_cache.numel() * elem
    R = args.rotate or max(1, math.ceil(4 * MALL_BYTES / max(kv_unique, 1)))
    R = max(1, min(R, int((64 << 30) // pool_bytes)))
    pools = [(runner.k_cache, runner.v_cache)]
    for _ in range(R - 1):
        pools.append((runner.k_cache.clone(), runner.v_cache.clone()))
    torch.cuda.synchronize()
    P = runner.partition_size
    P_eff = pa.decode_partition_size(runner.dims, len(w.batch), fin.max_context_len, P)
    log(f"[bench] {w.name}: {len(w.batch)} seqs, max ctx {fin.max_context_len}, "
        f"partition {P_eff if P_eff else 'balanced split'}, {len(fin.host_copies)} CoW copies, KV unique {kv_unique/1e6:.1f} MB "
        f"(logical {kv_logical/1e6:.1f} MB), {R} pool copies, setup {time.time()-t_setup:.1f}s")

    mbps = int(fin.block_tables.shape[1])
    varlen = w.kind == "varlen"

    sc = runner.kv_scales  # FP8 caches: per-KV-head scales (None otherwise)

    # a decode step that appends one token per batch row, in batch order, runs
    # the cache write inside the decode launch (pa_decode_append)
    appends = w.final_appends()
    fused = (not varlen and [s_ for s_, _ in appends] == [int(s_) for s_ in w.batch]
             and all(n_ == 1 for _, n_ in appends))

    # a fused step is one C call whose arguments are marshalled once per
    # pool copy (a serving loop's prepared launch), so host overhead stays
    # far below the kernel time
    prepared = []
    if fused:
        for partials_only in (False, True):
            prepared.append([pa.prepare_decode_append(
                fin.q, fin.k, fin.v, fin.slot_mapping, kc, vc, fin.block_tables,
                fin.context_lens, w.scale, fin.out, fin.max_context_len, P, fin.workspace,
                kv_scales=sc, partials_only=partials_only, layout=layout) for kc, vc in pools])

    def step(i):
        kc, vc = pools[i % R]
        if fin.copy_pairs is not None:
            pa.copy_blocks(kc, vc, fin.copy_pairs)
        if fused:
            prepared[0][i % R]()
            return
        pa.cache_write(fin.k, fin.v, fin.slot_mapping, kc, vc, kv_scales=sc, layout=layout)
        if varlen:
            pa.varlen(fin.q, fin.query_start_loc, fin.context_lens, kc, vc, fin.block_tables,
                      w.scale, fin.out, fin.max_query_len, fin.max_context_len, fin.workspace,
                      kv_scales=sc, layout=layout)
        else:
            pa.decode(fin.q, kc, vc, fin.block_tables, fin.context_lens, w.scale, fin.out,
                      fin.max_context_len, P, fin.workspace, kv_scales=sc, layout=layout)

    def roofline_kernel(i):
        # the priced kernel alone: the decode partition kernel, or for a
        # varlen step the whole pa_varlen call (prefill, decode rows, merge)
        kc, vc = pools[i % R]
        if varlen:
            pa.varlen(fin.q, fin.query_start_loc, fin.context_lens, kc, vc, fin.block_tables,
                      w.scale, fin.out, fin.max_query_len, fin.max_context_len, fin.workspace,
                      kv_scales=sc, layout=layout)
        elif fused:  # the partition kernel as the step launches it (with the write)
            prepared[1][i % R]()
        else:
            pa.decode_partials(fin.q, kc, vc, fin.block_tables, fin.context_lens, w.scale,
                               fin.out, fin.max_context_len, P, fin.workspace, kv_scales=sc,
                               layout=layout)

    def timed(fn, n):
        # back-to-back launches between one pair of events on the current
        # stream (events between every launch would add their own overhead)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return time.perf_counter() - t0, a.elapsed_time(b) / 1e3

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    wall, gpu_s = timed(step, K)          # timed region 1: whole steps
    for i in range(min(args.warmup, 5)):
        roofline_kernel(i)
    _, kern_s = timed(roofline_kernel, K)  # timed region 2: the priced kernel alone
    elapsed = max(wall, gpu_s)
    ms_per_step = elapsed / K * 1e3
    value = kv_unique * K / elapsed / 1e9
    avg_kern = kern_s / K * 1e6
    achieved = kv_unique / (avg_kern * 1e-6) / 1e9
    log(f"[bench] {K} steps: {ms_per_step*1e3:.1f} us/step (wall {wall*1e3/K*1e3:.1f}, events "
        f"{gpu_s*1e3/K*1e3:.1f}); {'pa_varlen' if varlen else 'partition kernel'} avg "
        f"{avg_kern:.2f} us over {K} back-to-back launches -> {achieved:.0f} GB/s "
        f"= {achieved/HBM_PEAK_GBS*100:.1f}% of HBM peak")

    n_tok = int(fin.slot_mapping.numel())

    cfg = {"workload": w.name, "num_seqs": len(w.batch), "num_heads": w.num_heads,
           "num_kv_heads": hkv, "head_dim": D, "block_size": B, "num_blocks": w.num_blocks,
           "max_context_len": fin.max_context_len,
           "context_tokens": int(fin.host_lens.sum()), "new_tokens_per_step": n_tok,
           "cache_layout": args.layout,
           "batch_order": ("rows grouped by first block" if fin.order is not None else "as given"),
           "partition_size": P_eff, "pool_copies_rotated": R, "cow_copies_per_step":
           len(fin.host_copies), "kv_bytes_unique_per_step": int(kv_unique),
           "kv_bytes_logical_per_step": int(kv_logical),
           "step_calls": ("pa_decode_append (cache write + decode in one launch)" if fused
                          else "pa_cache_write + " + ("pa_varlen" if varlen else "pa_decode"))}
    if runner.prefill_skipped:
        cfg["prompt_tokens_served_by_prefix_cache"] = int(runner.prefill_skipped)
    line = {
        "metric": "paged-attention decode KV-read GB/s (whole step: cache write + decode)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype if w.kv_dtype != "fp8" else "bf16 (q, out) / fp8 e4m3 (KV cache)",
        "data": "synthetic",
        "config": cfg,
        "pct_hbm_peak": round(value / HBM_PEAK_GBS * 100, 2),
        "tokens_per_s": round(n_tok / (ms_per_step / 1e3), 1),
        "seqs_per_s": round(len(w.batch) / (ms_per_step / 1e3), 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if varlen else measured_traffic(w.name, decode_kernel_name(w)),
                     "kernel": ("pa_varlen (prefill + decode-row + merge kernels)" if varlen
                                else decode_kernel_name(w)),
                     "bytes_per_launch": int(kv_unique), "avg_launch_us": round(avg_kern, 3),
                     "timing": f"{K} back-to-back launches between one HIP event pair"},
        "cpu_baseline": None,
    }
    if varlen:
        fl = prefill_flops(fin.host_qsl, fin.host_lens, w.num_heads, D)
        line["prefill_flops_per_step"] = fl
        line["prefill_tflops_lower_bound"] = round(fl / (avg_kern * 1e-6) / 1e12, 2)
        line["metric"] = "paged-attention mixed prefill+decode step KV-read GB/s"
        qlens = np.diff(fin.host_qsl)
        if (qlens >= 2).all():
            # prefill chunks only: a contraction, priced against the dense
            # bf16 matrix-core peak
            tflops = fl / (avg_kern * 1e-6) / 1e12
            line["metric"] = "paged-attention chunked-prefill step TFLOP/s (causal QK^T + PV)"
            line["value"] = round(fl * K / elapsed / 1e12, 2)
            line["unit"] = "TFLOP/s"
            line["pct_hbm_peak"] = None
            line["roofline"].update({"bound": "mfma", "achieved": round(tflops, 1),
                                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                                     "kernel": "pa_varlen (prefill units)",
                                     "flops_per_launch": fl})
    if args.cpu_seconds > 0:
        t = time.time()
        if varlen:
            line["cpu_baseline"] = cpu_baseline_varlen(
                w, args.cpu_seconds, line["roofline"]["bound"] == "mfma")
        else:
            line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        log(f"[bench] cpu baseline {line['cpu_baseline']['value']} GB/s "
            f"({time.time()-t:.1f}s incl. oracle cache fill)")
    s = json.dumps(line)
    print(s, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
