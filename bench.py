#!/usr/bin/env python3
"""Benchmark of the paged KV-cache decode step on one MI355X.

A step is one pass of the whole hot path over one batch: the copy-on-write
block copies when the workload has them (pa_copy_blocks), then every
sequence's new token stored in its slot and paged decode attention over the
whole context (pa_decode_attention_append: slot computation, KV write and
attention in one call).  --separate runs the same step as pa_write_kv_at
followed by pa_decode_attention.  Inputs are resident in HBM
before timing starts.  Each step reads a different one of several identical
pool copies (together far larger than the 256 MB last-level cache), so no
step is served from a cache warmed by the previous one.

    python bench.py [--steps K] [--warmup W]

prints ONE JSON line.  Its headline is the Llama-3.1-70B-shaped decode batch
(256 sequences, 64 query / 8 KV heads); `sub_results` holds the
Llama-3-8B-shaped batch, the shared-prefix batch (through the plain call and
through pa_decode_attention_shared, which reads each shared block once per
group of samples), the long-context batch and the chunked-prefill step, each
with its own roofline and CPU baseline.  Per
workload: KV GB/s of the whole step (`value`), seq-steps/s, the decode
call's roofline fraction (HIP events on the stream it runs on: one pair
around the timed back-to-back steps when a step is the decode call alone,
else a pair around each call), the median / p10 / p90 of single calls, the
achievable rates of the bandwidth probes (a contiguous stream and the
decode's own K/V gather with no arithmetic; --no-probes skips them), the
KV write at scale (the workload's history fill) and the CPU oracle's rate
on a bounded sample.

    python bench.py --config N

measures workload N (1-5) alone, with the same fields; with --shared its
decode runs through pa_decode_attention_shared.

    python bench.py --workload prefill

measures the chunked-prefill step alone (the chunk's K/V stored with
pa_write_kv_at, then pa_prefill_attention): useful TFLOP/s of the causal
attention against the bf16 matrix-core peak.

    python bench.py --workload swap

measures pa_swap_blocks: 8192 blocks (512 MiB of K and V) out to pinned
host memory and back, against the PCIe 5.0 x16 peak and a contiguous
torch copy of the same bytes (the DMA engines' rate on this machine).

    python bench.py --workload study

the paging-overhead and block-size study: the 8B- and 70B-shaped batches at
block sizes 8, 16, 32 and 64, blocks scattered or contiguous, with the
decode call's time and rate, the tail waste of the last blocks, the waste a
contiguous per-sequence reservation would leave, the table bytes, and the
pages' own closed-form figures beside them; one JSON line per case, then a
markdown table.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved KV GB/s (% of HBM peak) and seq-steps/sec"
PREFILL_METRIC = "chunked-prefill paged attention: useful TFLOP/s (causal, % of bf16 MFMA peak)"
SWAP_METRIC = "block swap HBM <-> pinned host memory: GB/s per direction"
HBM_PEAK_GBPS = 8000.0       # MI355X HBM3E, AMD published peak
HOST_LINK_PEAK_GBPS = 64.0   # PCIe 5.0 x16, one direction
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores, AMD published peak
LLC_BYTES = 256 << 20        # MI355X Infinity Cache


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=["decode", "prefill", "swap", "study"],
                    default="decode",
                    help="decode step (default), the chunked-prefill step, block swap, or the "
                         "block-size study")
    ap.add_argument("--config", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="one decode workload alone (default: the 70B-shaped batch as the "
                         "headline with workloads 2, 4, 5 and the prefill step as sub-results)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="bound on the oracle's timed CPU sample of the headline workload")
    ap.add_argument("--sub-cpu-seconds", type=float, default=6.0,
                    help="bound on the oracle's timed CPU sample of each sub-result")
    ap.add_argument("--vector-only", action="store_true",
                    help="decode with the vector-ALU kernel (fixed partitions) instead of the "
                         "matrix-core kernel, for the A/B of the two")
    ap.add_argument("--study-reps", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the bandwidth probes (achievable stream / gather rates)")
    ap.add_argument("--partition", type=int, default=None,
                    help="decode partition size (default: the workload's / the library's choice)")
    ap.add_argument("--separate", action="store_true",
                    help="store the new tokens with pa_write_kv_at, then pa_decode_attention")
    ap.add_argument("--shared", action="store_true",
                    help="run the decode through pa_decode_attention_shared (groups of "
                         "sequences that share prefix blocks read them once)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run pa_copy_blocks over a known number of bytes (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def cpu_baseline(wl, budget_s):
    """The oracle, as it stands, on the sequences of the same workload in
    order (starting over after the last) until `budget_s` seconds have passed
    (at least one sequence)."""
    import resource

    import numpy as np

    from oracle import paged_attention as O
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from plan_oracle import run_oracle

    kp, vp, _, _ = run_oracle(wl, wl.setup + [op for op in wl.step if op[0] != "decode"])
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = None
    done = 0
    kv = 0
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        i = done % wl.num_seqs
        O.decode_attention(wl.q, kp, vp, wl.tables["final"], wl.context_lens, wl.scale, wl.dtype,
                           seqs=[i])
        kv += int(wl.context_lens[i]) * wl.num_kv_heads * wl.head_dim * 2 * (2 if wl.dtype == "bf16" else 4)
        done += 1
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    # the step's other operations, each once, as the oracle does them (slot
    # computation + write of the new tokens; the copy-on-write copies)
    others = {}
    for kind, x in wl.step:
        t1 = time.perf_counter()
        if kind == "write":
            sl = O.slot_mapping(wl.tables[x.table], x.seq_ids, x.positions, wl.block_size,
                                wl.num_blocks)
            O.write_kv(kp, vp, x.k, x.v, sl)
            others["write"] = {"ms": round(1e3 * (time.perf_counter() - t1), 3),
                               "tokens": int(x.positions.size)}
        elif kind == "copy":
            O.copy_blocks(kp, vp, x)
            others["copy"] = {"ms": round(1e3 * (time.perf_counter() - t1), 3),
                              "pairs": int(len(x))}
    return {
        "value": kv / wall / 1e9, "unit": "GB/s", "cores": round(cpu / wall, 2), "kind": "oracle",
        "other_ops_once": others,
        "sample": (f"float64 numpy oracle decode, one sequence (all {wl.num_q_heads} query heads) "
                   f"per call, {done} sequence-steps cycling over the {wl.num_seqs} sequences of "
                   f"the same workload ({done / wl.num_seqs:.2f} passes): {wall:.1f} s wall, "
                   f"{done / wall:.2f} seq-steps/s; cores = CPU time / wall time; "
                   f"BLAS pool {blas} threads; host affinity {len(os.sched_getaffinity(0))} cpus"),
        "seq_steps_per_s": done / wall,
    }


def cpu_baseline_prefill(wl, budget_s):
    """The oracle's prefill attention, as it stands, one sequence per call
    (its chunk, context and table) cycling over the workload's sequences
    until `budget_s` seconds have passed (at least one sequence)."""
    import resource

    import numpy as np

    from oracle import paged_attention as O
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from plan_oracle import run_oracle

    kp, vp, _, _ = run_oracle(wl, wl.setup + [op for op in wl.step if op[0] != "prefill"])
    qs = wl.query_start
    done = flops = 0
    r0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    while done == 0 or time.perf_counter() - t0 < budget_s:
        i = done % wl.num_seqs
        n, L = int(wl.context_lens[i]), int(qs[i + 1] - qs[i])
        O.prefill_attention(wl.q[qs[i]:qs[i + 1]], kp, vp, wl.tables["final"][i:i + 1],
                            wl.context_lens[i:i + 1], np.array([0, L], np.int32), wl.scale,
                            wl.dtype)
        flops += 4 * (L * (n - L) + L * (L + 1) // 2) * wl.num_q_heads * wl.head_dim
        done += 1
    wall = time.perf_counter() - t0
    r1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (r1.ru_utime - r0.ru_utime) + (r1.ru_stime - r0.ru_stime)
    return {
        "value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": round(cpu / wall, 2),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle prefill, one sequence's chunk per call, {done} "
                   f"sequences cycling over the {wl.num_seqs} of the same workload: "
                   f"{wall:.1f} s wall; cores = CPU time / wall time; host affinity "
                   f"{len(os.sched_getaffinity(0))} cpus"),
    }


def prefill_result(args, cpu_seconds):
    """The chunked-prefill step (pa_write_kv_at of the chunks' K/V, then
    pa_prefill_attention) timed over rotated pool copies; returns its result
    object (useful causal TFLOP/s against the bf16 matrix-core peak)."""
    import torch

    import workloads as W
    from workloads.device import DeviceWorkload

    wl = W.make_prefill()
    dev = DeviceWorkload(wl)
    dev.run_setup()
    dev.release_setup_inputs()
    pool_bytes = 2 * dev.pools[0][0].numel() * dev.pools[0][0].element_size()
    npools = max(2, min(8, -(-4 * LLC_BYTES // pool_bytes) + 1))
    dev.add_pool_copies(npools - 1)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    att_ops = [op for op in dev.step_ops if op[0] == "prefill"]
    other_ops = [op for op in dev.step_ops if op[0] != "prefill"]
    prepared = [(dev.prepare(other_ops, k, stream=stream), dev.prepare(att_ops, k, stream=stream))
                for k in range(npools)]

    def step(k, ev=None):
        others, att = prepared[k % npools]
        for c in others:
            c()
        if ev is not None:
            ev[0].record(stream)
        for c in att:
            c()
        if ev is not None:
            ev[1].record(stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k, events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    att_ms = [a.elapsed_time(b) for a, b in events]
    att_avg = sum(att_ms) / len(att_ms)
    flops = wl.prefill_flops()
    achieved = flops / (att_avg * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    res = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2), "unit": "TFLOP/s", "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {
            "workload": wl.name, "num_seqs": wl.num_seqs,
            "query_tokens": int(wl.query_start[-1]), "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
            "block_size": wl.block_size, "sum_context_tokens": int(wl.context_lens.sum()),
            "step_calls": ["pa_write_kv_at", "pa_prefill_attention"],
            "seed": list(wl.seed), "pool_copies_rotated": npools,
            "parallelism": "single GPU",
        },
        "flops_per_step": flops,
        "prefill_ms": {"avg": round(att_avg, 5), "min": round(min(att_ms), 5),
                       "max": round(max(att_ms), 5)},
        "roofline": {
            "kernel": "pa_prefill_attention: prefill_flash_kernel (events around the call)",
            "bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4), "traffic": None,
            "algorithmic_flops_per_launch": flops, "avg_launch_us": round(att_avg * 1e3, 2),
        },
    }
    traffic, src = measured_traffic(wl, "pa_prefill.hip")
    if traffic:
        res["roofline"]["traffic"] = traffic
        res["roofline"]["traffic_source"] = src
        res["roofline"]["traffic_note"] = (
            "HBM bytes per call (K/V reads, mostly served from L2 after the first query tile, "
            "and the float32 output); the bound is the matrix cores, not this traffic")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(wl, cpu_seconds)
    del prepared, dev
    torch.cuda.empty_cache()
    return res


def swap_main(args):
    """Swap-out of every block of a 512 MiB pool pair to pinned host pools,
    then swap-in to a permuted placement; per-direction GB/s from HIP events
    on the stream, next to a contiguous torch copy of the same size."""
    import numpy as np
    import torch

    import paged_kv_cache_188_amd as pa
    nb, hkv, bs, d = 8192, 8, 16, 128
    kd = torch.randn((nb, hkv, d // 8, bs, 8), device="cuda").to(torch.bfloat16)
    vd = torch.randn((nb, hkv, bs, d), device="cuda").to(torch.bfloat16)
    hk = torch.empty(kd.shape, dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty(vd.shape, dtype=torch.bfloat16, pin_memory=True)
    rng = np.random.default_rng(188)
    out_pairs = torch.from_numpy(np.stack([np.arange(nb), rng.permutation(nb)], 1)
                                 .astype(np.int32)).cuda()
    in_pairs = torch.from_numpy(np.stack([rng.permutation(nb), np.arange(nb)], 1)
                                .astype(np.int32)).cuda()
    nbytes = 2 * kd.numel() * kd.element_size()
    stream = torch.cuda.current_stream()

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / reps

    reps = max(1, min(args.steps, 10))
    t_out = timed(lambda: pa.swap_blocks(hk, hv, kd, vd, out_pairs), reps)
    t_in = timed(lambda: pa.swap_blocks(kd, vd, hk, hv, in_pairs), reps)
    flat_d = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    flat_h = torch.empty(nbytes // 2, dtype=torch.bfloat16, pin_memory=True)
    t_d2h = timed(lambda: flat_h.copy_(flat_d, non_blocking=True), reps)
    t_h2d = timed(lambda: flat_d.copy_(flat_h, non_blocking=True), reps)
    gbs = lambda ms: nbytes / (ms * 1e-3) / 1e9
    out_rate, in_rate = gbs(t_out), gbs(t_in)
    res = {
        "metric": SWAP_METRIC, "value": round(min(out_rate, in_rate), 2), "unit": "GB/s",
        "n_gpus": 1, "steps": reps, "warmup": 2, "ms_per_step": round(t_out + t_in, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"swap {nb} blocks (Hkv={hkv} bs={bs} D={d} bf16, K and V: "
                               f"{nbytes >> 20} MiB) out to pinned host memory and back",
                   "parallelism": "single GPU"},
        "swap_out_gbs": round(out_rate, 2), "swap_in_gbs": round(in_rate, 2),
        "torch_copy_d2h_gbs": round(gbs(t_d2h), 2), "torch_copy_h2d_gbs": round(gbs(t_h2d), 2),
        "roofline": {
            "kernel": "pa_swap_blocks: copy_blocks_kernel over the host link (events per call)",
            "bound": "host link", "achieved": round(min(out_rate, in_rate), 2),
            "peak": HOST_LINK_PEAK_GBPS, "unit": "GB/s",
            "frac": round(min(out_rate, in_rate) / HOST_LINK_PEAK_GBPS, 4), "traffic": None,
            "algorithmic_bytes_per_launch": nbytes,
            "avg_launch_us": {"out": round(t_out * 1e3, 1), "in": round(t_in * 1e3, 1)},
        },
    }
    print(json.dumps(res), flush=True)


def measured_traffic(wl, kernel_src="pa_decode.hip", call=None):
    """HBM bytes per call from a committed counter summary
    (profiles/*traffic*.txt) taken on this workload with the kernel source as
    it is now: (bytes, provenance), or (None, None) when no summary matches.
    The counters are not read in this run; the provenance says where the
    figure comes from."""
    import glob
    import hashlib
    src = os.path.join(ROOT, "paged_kv_cache_188_amd", "csrc", kernel_src)
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*traffic*.txt"))):
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        if (kv.get("kernel_source_sha256") == sha and kv.get("workload") == wl.name
                and kv.get("call") == call):
            return int(kv["traffic_bytes_per_launch"]), {
                "from_profile": os.path.relpath(path, ROOT), "kernel_source_sha256": sha[:16],
                "measured_in_this_run": False,
                "how": "rocprofv3 TCC_EA0_RDREQ x 128 B and WRITE_SIZE, calibrated on a copy "
                       "kernel of known size"}
    return None, None


def calibrate_copy(steps):
    """Copy 8192 blocks of 32 KiB in each of the K and V pools: 512 MiB read
    and 512 MiB written per launch (536,870,912 B each way), with no reuse
    between launches."""
    import torch

    import paged_kv_cache_188_amd as pa
    nb, hkv, bs, d = 16384, 8, 16, 128
    k = torch.zeros((nb, hkv, d // 8, bs, 8), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device="cuda")
    half = nb // 2
    pairs = torch.stack([torch.arange(half), torch.arange(half) + half], 1).to(torch.int32).cuda()
    for _ in range(steps):
        pa.copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    block_bytes = hkv * bs * d * 2
    print(json.dumps({"calibration": "pa_copy_blocks", "launches": steps,
                      "read_bytes_per_launch": 2 * half * block_bytes,
                      "write_bytes_per_launch": 2 * half * block_bytes}), flush=True)


def _span_ms(torch, stream, fn, reps):
    """Average time of fn(r) for r = 0 .. reps-1 issued back to back: one HIP
    event pair around all of them on `stream`, divided by reps."""
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for r in range(reps):
        fn(r)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def _pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def achievable(torch, pa, dev, wl, npools, stream, reps=20):
    """What the memory system delivers on this machine with no arithmetic at all
    (include/pa_probe.h): a contiguous stream over the pools, and the decode
    call's own K/V chunk gather through the same tables, each at four grid
    sizes; the best of each is the achievable reference."""
    table = dev.tables[[x for kind, x in wl.step if kind == "decode"][0]]
    chunk = wl.block_size * wl.head_dim * (2 if wl.dtype == "bf16" else 4)
    blocks = int(sum(-(-int(c) // wl.block_size) for c in wl.context_lens if c > 0))
    gather_bytes = 2 * blocks * wl.num_kv_heads * chunk
    pool_bytes = sum(t.numel() * t.element_size() for t in dev.pools[0])
    res = {"gather_bytes": gather_bytes, "stream_bytes": pool_bytes, "grids": {}}
    best_g = best_s = 0.0
    for sink_len in (512, 1024, 2048, 4096):
        def g(r):
            k, v = dev.pools[r % npools]
            pa.probe_gather(k, v, table, dev.ctx, sink_len=sink_len, stream=stream)

        def s(r):
            for t in dev.pools[r % npools]:
                pa.probe_read(t, sink_len=sink_len, stream=stream)
        g(0), s(0)
        tg = _span_ms(torch, stream, g, reps)
        ts = _span_ms(torch, stream, s, reps)
        gg, sg = gather_bytes / (tg * 1e-3) / 1e9, pool_bytes / (ts * 1e-3) / 1e9
        res["grids"][sink_len] = {"gather_gbps": round(gg, 1), "stream_gbps": round(sg, 1)}
        best_g, best_s = max(best_g, gg), max(best_s, sg)
    res["gather_gbps"] = round(best_g, 1)
    res["stream_gbps"] = round(best_s, 1)
    return res


def other_ops_timing(torch, dev, wl, npools, stream, reps=20):
    """The step's KV write (pa_write_kv_at of its new tokens, the same rows
    the append call stores) and copy-on-write copies (pa_copy_blocks), each
    timed alone: one event pair around reps back-to-back calls.  Bytes are
    the K/V rows or blocks read plus written."""
    e = 2 if wl.dtype == "bf16" else 4
    res = {}
    for op in dev.step_ops:
        kind, x = op
        if kind not in ("write", "copy"):
            continue
        calls = [dev.prepare([op], k, stream=stream)[0] for k in range(npools)]
        calls[0]()
        ms = _span_ms(torch, stream, lambda r: calls[r % npools](), reps)
        if kind == "write":
            t = int(x["positions"].numel())
            nbytes = 2 * 2 * t * wl.num_kv_heads * wl.head_dim * e + 20 * t
            res["pa_write_kv_at"] = {"us": round(ms * 1e3, 2), "tokens": t,
                                     "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        else:
            n = int(x.shape[0])
            nbytes = 2 * 2 * n * wl.num_kv_heads * wl.block_size * wl.head_dim * e + 8 * n
            res["pa_copy_blocks"] = {"us": round(ms * 1e3, 2), "pairs": n,
                                     "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    return res


def history_write_timing(torch, dev, wl, stream, reps=5):
    """The workload's history fill at scale: each setup write
    (pa_write_kv_at of every cached token) timed alone, one event pair around
    reps back-to-back calls; bytes are the K/V rows read plus written.  Beside
    it, torch's device-to-device copy of a contiguous buffer of the rows' size
    (the same bytes read and written, no scatter) as the box's read + write
    reference."""
    e = 2 if wl.dtype == "bf16" else 4
    out = []
    for op in dev.setup_ops:
        kind, x = op
        if kind != "write":
            continue
        call = dev.prepare([op], 0, stream=stream)[0]
        call()
        ms = _span_ms(torch, stream, lambda r: call(), reps)
        t = int(x["positions"].numel())
        nbytes = 2 * 2 * t * wl.num_kv_heads * wl.head_dim * e + 20 * t
        gbps = nbytes / (ms * 1e-3) / 1e9
        rows = 2 * t * wl.num_kv_heads * wl.head_dim * e
        src = torch.empty(rows, dtype=torch.uint8, device=dev.device)
        dst = torch.empty_like(src)
        dst.copy_(src)
        cms = _span_ms(torch, stream, lambda r: dst.copy_(src), reps)
        cgbps = 2 * rows / (cms * 1e-3) / 1e9
        del src, dst
        out.append({"call": "pa_write_kv_at", "tokens": t, "us": round(ms * 1e3, 1),
                    "gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
                    "torch_copy_same_bytes": {"us": round(cms * 1e3, 1), "gbps": round(cgbps, 1),
                                              "frac_of_hbm_peak":
                                                  round(cgbps / HBM_PEAK_GBPS, 4)}})
    return out


def block_copy_reference(torch, pa, stream, reps=10):
    """What a read + write stream reaches on this machine through libpa's own
    block copy: 8192 blocks of 64 KiB (K and V, 32 KiB each) copied from one
    half of a pool pair into the other, 512 MiB read and 512 MiB written per
    call: with the blocks in order; with source and destination blocks in
    two seeded random orders; and with the sources in order and the
    destinations in a random order, the pattern of a history write (rows
    read in order, stored into scattered blocks).  One event pair around reps
    back-to-back calls each."""
    nb, hkv, bs, d = 16384, 8, 16, 128
    k = torch.zeros((nb, hkv, d // 8, bs, 8), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device="cuda")
    half = nb // 2
    g = torch.Generator().manual_seed(188)
    orders = {"sequential": (torch.arange(half), torch.arange(half) + half),
              "shuffled": (torch.randperm(half, generator=g),
                           torch.randperm(half, generator=g) + half),
              "sequential_to_shuffled": (torch.arange(half),
                                         torch.randperm(half, generator=g) + half)}
    nbytes = 2 * 2 * half * hkv * bs * d * 2  # K and V, read and written
    out = {"blocks": half, "block_bytes": 2 * hkv * bs * d * 2,
           "bytes_read_plus_written": nbytes}
    for name, (src, dst) in orders.items():
        pairs = torch.stack([src, dst], 1).to(torch.int32).cuda()
        pa.copy_blocks(k, v, pairs, stream=stream)
        ms = _span_ms(torch, stream, lambda r: pa.copy_blocks(k, v, pairs, stream=stream), reps)
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"us": round(ms * 1e3, 1), "gbps": round(gbps, 1),
                     "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    del k, v
    torch.cuda.empty_cache()
    return out


def decode_result(cid, args, cpu_seconds, separate=False, shared=False):
    """One decode workload: the step timed over rotated pool copies, the
    decode call's roofline, single-call distribution, probes, the step's
    other calls and the history write timed alone, and the CPU oracle on a
    bounded sample.  shared=True runs the decode through
    pa_decode_attention_shared.  Returns the result object (no driver-level
    keys)."""
    import numpy as np
    import torch

    import paged_kv_cache_188_amd as pa
    import workloads as W
    from workloads.device import DeviceWorkload

    wl = W.make(cid)
    if args.partition is not None:
        wl.partition_size = args.partition
    dev = DeviceWorkload(wl)
    stream = torch.cuda.current_stream()
    dev.run_setup()
    hist = history_write_timing(torch, dev, wl, stream)
    dev.release_setup_inputs()
    pool_bytes = 2 * dev.pools[0][0].numel() * dev.pools[0][0].element_size()
    npools = max(2, min(8, -(-4 * LLC_BYTES // pool_bytes) + 1))
    dev.add_pool_copies(npools - 1)
    torch.cuda.synchronize()

    ops = dev.step_ops if separate else dev.step_ops_append
    appended = any(kind == "decode_append" for kind, _ in ops)
    decode_ops = [op for op in ops if op[0] in ("decode", "decode_append")]
    other_ops = [op for op in ops if op[0] not in ("decode", "decode_append")]
    # every call validated and marshalled once per pool copy: a step's host
    # work is then a few foreign-function calls, far less than its GPU time,
    # so the stream never runs dry between steps
    prepared = [dev.prepare(other_ops + decode_ops, k, stream=stream,
                            vector_only=args.vector_only, shared=shared) for k in range(npools)]
    n_other = len(other_ops)
    # When the step is the decode call(s) alone, one pair of HIP events spans
    # the K back-to-back steps; otherwise events bracket each step's decode
    # calls.  (An event record is a packet of its own in the stream and adds
    # a few microseconds to whatever it brackets.)
    per_call_events = n_other > 0

    def step(k, ev=None):
        calls = prepared[k % npools]
        for c in calls[:n_other]:
            c()
        if ev is not None:
            ev[0].record(stream)
        for c in calls[n_other:]:
            c()
        if ev is not None:
            ev[1].record(stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)] if per_call_events else [None] * args.steps
    span = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    t0 = time.perf_counter()
    span[0].record(stream)
    for k in range(args.steps):
        step(args.warmup + k, events[k])
    span[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # distribution of single calls: every call between its own event pair
    # (the event packets add their own few microseconds to each)
    if per_call_events:
        one_ms = [a.elapsed_time(b) for a, b in events]
    else:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for k in range(args.steps):
            step(args.warmup + args.steps + k, evs[k])
        torch.cuda.synchronize()
        one_ms = [a.elapsed_time(b) for a, b in evs]
    ach = None if args.no_probes else achievable(torch, pa, dev, wl, npools, stream)
    ops_timing = other_ops_timing(torch, dev, wl, npools, stream)

    ms_step = wall * 1e3 / args.steps
    workers = pa.decode_streamk_workers(wl.num_seqs, wl.head_dim, wl.block_size,
                                        wl.partition_size, dev.torch_dtype,
                                        vector_only=args.vector_only)
    call = "pa_decode_attention_append" if appended else "pa_decode_attention"
    if shared:
        call = "pa_decode_attention_shared"
        gs, sl, _ = dev.shared_args("final")
        gs, sl = gs.cpu().numpy(), sl.cpu().numpy()
        decomposition = {"path": "stream-K, shared prefixes", "persistent_waves": workers,
                         "groups": int(len(sl)), "groups_sharing": int((sl > 0).sum()),
                         "members_per_group": sorted(set(np.diff(gs).tolist()))}
        kernel = (f"{call}: decode_mfma_streamk_kernel (prefix pass, own-token pass) + "
                  "decode_streamk_merge_kernel x2 + decode_shared_combine_kernel")
    elif workers > 0:
        decomposition = {"path": "stream-K", "persistent_waves": workers}
        kernel = f"{call}: decode_mfma_streamk_kernel + decode_streamk_merge_kernel"
    else:
        decomposition = {"path": "fixed partitions", "partition_size": pa.decode_partition_size(
            wl.num_seqs, wl.num_kv_heads, wl.block_size, wl.max_context_len, wl.partition_size)}
        main_k = "decode_valu_kernel" if args.vector_only or wl.dtype != "bf16" \
            else "decode_mfma_kernel"
        kernel = (f"{call}: " + ("append_kv_kernel + " if appended else "")
                  + main_k + " + decode_reduce_kernel")
    if per_call_events:
        dec_ms = [a.elapsed_time(b) for a, b in events]
        dec_avg_ms = sum(dec_ms) / len(dec_ms)
        dec_timing = {"avg": round(dec_avg_ms, 5), "min": round(min(dec_ms), 5),
                      "max": round(max(dec_ms), 5),
                      "how": "HIP events around each step's decode call(s)"}
        kernel += " (events around each call)"
    else:
        dec_avg_ms = span[0].elapsed_time(span[1]) / args.steps
        dec_timing = {"avg": round(dec_avg_ms, 5),
                      "how": f"HIP events around {args.steps} back-to-back steps, each the "
                             "decode call alone, divided by the step count"}
        kernel += f" (events around {args.steps} back-to-back calls)"
    kv_bytes = wl.kv_bytes_read()
    dec_bytes = wl.shared_decode_bytes(gs, sl) if shared else wl.decode_bytes()
    if appended:  # the call also stores every non-empty sequence's new K/V row
        dec_bytes += int((wl.context_lens > 0).sum()) * wl.num_kv_heads * wl.head_dim * 2 \
            * (2 if wl.dtype == "bf16" else 4)
    achieved = dec_bytes / (dec_avg_ms * 1e-3) / 1e9
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    traffic, traffic_src = (None, None) if args.vector_only or args.partition is not None \
        else measured_traffic(wl, call=call if shared else None)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "num_seqs": wl.num_seqs, "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
            "block_size": wl.block_size, "num_blocks": wl.num_blocks,
            "sum_context_tokens": int(wl.context_lens.sum()),
            "max_context_len": wl.max_context_len,
            "decomposition": decomposition,
            "step_calls": [{"copy": "pa_copy_blocks", "write": "pa_write_kv_at",
                            "decode": call, "decode_append": call}[kind]
                           for kind, _ in ops],
            "seed": list(wl.seed), "pool_copies_rotated": npools,
            "parallelism": "single GPU",
        },
        "seq_steps_per_s": round(wl.num_seqs / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_ms": dec_timing,
        "decode_call_us": {"median": round(1e3 * _pct(one_ms, 0.5), 2),
                           "p10": round(1e3 * _pct(one_ms, 0.1), 2),
                           "p90": round(1e3 * _pct(one_ms, 0.9), 2),
                           "how": "HIP events around each single call"},
        "roofline": {
            "kernel": kernel,
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
            "algorithmic_bytes_per_launch": dec_bytes,
            "avg_launch_us": round(dec_avg_ms * 1e3, 2),
        },
    }
    res["other_ops"] = ops_timing
    res["history_write"] = hist
    uniq = wl.unique_kv_bytes()
    if shared:
        res["roofline"]["note"] = (
            "algorithmic bytes: each group's shared prefix read once, every sequence's own "
            "tokens once, queries and outputs; value (logical bytes, every sequence's full "
            "context, per step time) counts shared blocks once per sequence")
        res["roofline"]["unique_kv_bytes"] = uniq
    elif uniq < kv_bytes:
        # blocks shared between sequences: the call reads each sequence's
        # whole context through its table, and the repeated reads of shared
        # blocks can hit in the caches, so the logical-byte rate above is not
        # a fraction of HBM traffic; the distinct blocks' bytes are the least
        # the HBM must deliver
        res["roofline"]["note"] = ("logical bytes (each sequence's full context); shared "
                                   "blocks may be served from cache")
        res["roofline"]["unique_kv_bytes"] = uniq
        res["roofline"]["unique_kv_gbps"] = round(uniq / (dec_avg_ms * 1e-3) / 1e9, 1)
    if ach is not None:
        ach["decode_frac_of_gather"] = round(achieved / ach["gather_gbps"], 4)
        ach["decode_frac_of_stream"] = round(achieved / ach["stream_gbps"], 4)
        res["achievable"] = ach
    if traffic:
        res["roofline"]["traffic_gbps"] = round(traffic / (dec_avg_ms * 1e-3) / 1e9, 1)
    del prepared, dev
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, cpu_seconds)
    return res


def _driver_keys(res, args):
    """The keys of the one-line contract, in front of a result object."""
    out = {"metric": res["metric"], "value": res["value"], "unit": res["unit"], "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": res["dtype"], "data": res["data"]}
    out.update({k: v for k, v in res.items() if k not in out})
    return out


def study(args):
    """Paging overhead and block size, measured with the decode kernels.

    [nalar] "Sisa alokasi dibatasi oleh granularitas blok" trades tail
    waste (the unused slots of each sequence's last block) against metadata
    (table entries) as the block size changes, and [nalar] "Kernel attention
    harus mengikuti block table" notes that walking the table costs
    something.  For the Llama-3-8B-shaped batch (64 sequences, 32 / 8 heads,
    contexts uniform in [128, 4096]) and the Llama-3.1-70B-shaped batch (256
    sequences, 64 / 8 heads, lognormal contexts up to 8192), at block sizes 8,
    16, 32 and 64, blocks scattered (seeded shuffle) or contiguous: the
    pa_decode_attention_append call's median time over rotated pool copies,
    its KV and algorithmic rates, the unused share of the allocated slots,
    the share a contiguous per-sequence reservation of the maximum length
    would leave unused ([gininih] "Masalah fragmentasi memori KV Cache
    konvensional": 60-80 % of the memory wasted that way; [bicarait]
    "Blueprint Arsitektur 1: Akar Masalah Fragmentasi KV Cache"), and the
    table bytes the kernel reads.  The pages' own closed-form figures are
    computed beside them: the 93 % of a 4096-slot reservation left unused by
    a 300-token request ([gyaansetu] "The memory problem"), and the (N-1)/N
    prompt-memory saving of N samples sharing one prompt ([bicarait]
    "Berbagi Memori Fisik")."""
    import math

    import numpy as np
    import torch

    import paged_kv_cache_188_amd as pa
    import workloads as W
    from workloads.device import DeviceWorkload

    closed = {
        "reservation_4096_used_300_unused_frac": round((4096 - 300) / 4096, 4),
        "paged_bs16_used_300_unused_frac": round((math.ceil(300 / 16) * 16 - 300)
                                                 / (math.ceil(300 / 16) * 16), 4),
        "shared_prompt_saving_N4": 3 / 4,
        "shared_prompt_saving_N8": 7 / 8,
    }
    print(json.dumps({"closed_forms": closed}), flush=True)
    stream = torch.cuda.current_stream()
    shapes = [
        ("llama3-8b", 2, 64, 32, lambda r: r.integers(128, 4096, size=64, endpoint=True), 4096),
        ("llama3.1-70b", 3, 256, 64,
         lambda r: np.clip(np.rint(r.lognormal(math.log(1024), 0.8, size=256)), 16, 8192), 8192),
    ]
    rows = []
    for label, cid, S, hq, draw, max_len in shapes:
        ctx = draw(np.random.default_rng(np.random.SeedSequence([188, cid]))).astype(np.int32)
        for bs in (8, 16, 32, 64):
            for shuffle in (True, False):
                rng = np.random.default_rng(np.random.SeedSequence([188, cid, bs, int(shuffle)]))
                wl = W.decode_workload(
                    f"{label}-decode bs={bs} {'shuffled' if shuffle else 'contiguous'}", W.BF16,
                    ctx, hq, 8, 128, bs, rng=rng, seed=(188, cid),
                    max_blocks_per_seq=math.ceil(max_len / bs), shuffle=shuffle)
                dev = DeviceWorkload(wl)
                dev.run_setup()
                dev.release_setup_inputs()
                pool_bytes = 2 * dev.pools[0][0].numel() * dev.pools[0][0].element_size()
                npools = max(2, min(8, -(-4 * LLC_BYTES // pool_bytes) + 1))
                dev.add_pool_copies(npools - 1)
                calls = [dev.prepare(dev.step_ops_append, k, stream=stream)
                         for k in range(npools)]
                for k in range(5):
                    for c in calls[k % npools]:
                        c()
                torch.cuda.synchronize()
                ev = [(torch.cuda.Event(enable_timing=True),
                       torch.cuda.Event(enable_timing=True)) for _ in range(args.study_reps)]
                for k, (a, b) in enumerate(ev):
                    a.record(stream)
                    for c in calls[k % npools]:
                        c()
                    b.record(stream)
                torch.cuda.synchronize()
                med = _pct([a.elapsed_time(b) for a, b in ev], 0.5)
                blocks = np.ceil(ctx / bs).astype(np.int64)
                allocated = int((blocks * bs).sum())
                workers = pa.decode_streamk_workers(wl.num_seqs, wl.head_dim, bs, 0,
                                                    dev.torch_dtype)
                row = {
                    "batch": label, "block_size": bs,
                    "placement": "shuffled" if shuffle else "contiguous",
                    "decode_call_us": round(med * 1e3, 2),
                    "kv_GBps": round(wl.kv_bytes_read() / med / 1e6, 1),
                    "algorithmic_GBps": round(wl.decode_bytes() / med / 1e6, 1),
                    "frac_of_8TBps": round(wl.decode_bytes() / med / 1e6 / HBM_PEAK_GBPS, 4),
                    "path": "stream-K" if workers > 0 else "fixed partitions",
                    "tail_waste_frac": round(1 - int(ctx.sum()) / allocated, 5),
                    "reservation_waste_frac": round(1 - int(ctx.sum()) / (S * max_len), 4),
                    "table_bytes_read": int(4 * blocks.sum()),
                }
                rows.append(row)
                print(json.dumps(row), flush=True)
                del calls, dev
                torch.cuda.empty_cache()
    print("| batch | block size | placement | decode call (us) | KV GB/s | frac of 8 TB/s | "
          "path | unused slots (paged) | unused slots (reserved max) | table bytes |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['batch']} | {r['block_size']} | {r['placement']} | {r['decode_call_us']} | "
              f"{r['kv_GBps']} | {r['frac_of_8TBps']} | {r['path']} | "
              f"{100 * r['tail_waste_frac']:.2f} % | {100 * r['reservation_waste_frac']:.1f} % | "
              f"{r['table_bytes_read']} |")


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.steps)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(each sequence's blocks live on one GPU; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.workload == "prefill":
        print(json.dumps(_driver_keys(prefill_result(args, args.cpu_seconds), args)), flush=True)
        return
    if args.workload == "swap":
        swap_main(args)
        return
    if args.workload == "study":
        study(args)
        return
    if args.config is not None:
        res = decode_result(args.config, args, args.cpu_seconds, separate=args.separate,
                            shared=args.shared)
        print(json.dumps(_driver_keys(res, args)), flush=True)
        return
    # default: the 70B-shaped batch is the headline; the 8B-shaped,
    # shared-prefix and long-context batches and the chunked-prefill step are
    # sub-results of the same line, each with its own roofline and baseline
    head = decode_result(3, args, args.cpu_seconds, separate=args.separate)
    print(f"[bench] {head['config']['workload']}: {head['roofline']['frac']}", file=sys.stderr,
          flush=True)
    subs = {}
    for cid, shared in ((2, False), (4, False), (4, True), (5, False)):
        r = decode_result(cid, args, args.sub_cpu_seconds, separate=args.separate, shared=shared)
        name = r["config"]["workload"] + (" | pa_decode_attention_shared" if shared else "")
        subs[name] = r
        print(f"[bench] {name}: {r['roofline']['frac']} {r['decode_call_us']['median']} us",
              file=sys.stderr, flush=True)
    r = prefill_result(args, args.sub_cpu_seconds)
    subs[r["config"]["workload"]] = r
    print(f"[bench] {r['config']['workload']}: {r['roofline']['frac']}", file=sys.stderr,
          flush=True)
    out = _driver_keys(head, args)
    out["sub_results"] = subs
    import paged_kv_cache_188_amd as pa
    out["read_write_reference"] = block_copy_reference(torch, pa, torch.cuda.current_stream())
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
