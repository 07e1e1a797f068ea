"""Throughput of one decode step of the paged-KV hot path on one MI355X.

A step = this step's copy-on-write block copies (none in this workload) +
pa_write_decode (every sequence's new token stored into its slot, then decode
attention over the paged cache, in one launch), on seeded synthetic inputs
already resident in HBM. `--two-calls` times pa_write_kv + pa_decode instead.
Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload llama3_8b]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, vendor figure
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
_CSRC = os.path.join(ROOT, "paged_kv_cache_131_amd", "csrc")
# sources whose change invalidates a recorded traffic figure, per workload kind
KERNEL_SOURCES = {
    "decode": [os.path.join(_CSRC, f) for f in ("pa_kernels.hip", "pa_api.cpp", "pa_internal.h", "pa_device.h")],
    "prefill": [os.path.join(_CSRC, f) for f in ("pa_prefill.hip", "pa_api.cpp", "pa_internal.h", "pa_device.h")],
}

WORKLOAD_TEXT = {
    "llama3_8b": "Llama-3-8B-shaped GQA decode: 256 seqs, 32 q / 8 kv heads, head_dim 128, block 16, bf16, "
                 "lengths lognormal(median 800, sigma 1) clipped to [16, 8192], shuffled pool",
    "opt13b": "OPT-13B-shaped decode: 64 seqs, 40 heads (MHA), head_dim 128, block 16, fp16, lengths U[128, 2048]",
    "long_context": "long-context split decode: 16 seqs, 64 q / 8 kv heads, head_dim 128, block 32, bf16, "
                    "lengths U[32768, 131072], 512-token partitions",
    "parallel_sampling": "parallel sampling, last of 256 decode steps: 32 prompts of 1016 tokens x 8 samples "
                         "sharing the prompt blocks (copy-on-write at divergence), 32 q / 8 kv heads, head_dim 128, "
                         "block 16, bf16",
    "beam_search": "beam search, last of 64 decode steps: 32 prompts of 1000 tokens x 4 beams, beams re-selected "
                   "every step (fork / release, copy-on-write of shared last blocks), 32 q / 8 kv heads, head_dim "
                   "128, block 16, bf16",
    "shared_prefix": "shared prefix: 256 requests mapping one {prefix}-token prompt prefix plus own suffixes of "
                     "U[16, 512] tokens, 32 q / 8 kv heads, head_dim 128, block 16, bf16",
    "prefill": "prompt phase: 32 whole prompts, lengths lognormal(median 800, sigma 1) clipped to [16, 8192], causal "
               "attention over their K/V in the paged pool, 32 q / 8 kv heads, head_dim 128, block 16, bf16, "
               "shuffled pool",
}
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # MI355X dense matrix peak


def kernel_hash(workload: str) -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES["prefill" if workload == "prefill" else "decode"]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_bytes(c, context_lens) -> dict:
    """Algorithmic bytes of one pa_decode call: K and V of every context token,
    q, the fp32 output, the block ids read and the lengths."""
    es = {"f32": 4, "f16": 2, "bf16": 2}[c.etype]
    L = context_lens.astype(np.int64)
    kv = int(L.sum()) * c.num_kv_heads * c.head_dim * 2 * es
    q = c.num_seqs * c.num_heads * c.head_dim * es
    out = c.num_seqs * c.num_heads * c.head_dim * 4
    ids = 4 * int((-(-L // c.block_size)).sum())
    lens = 4 * c.num_seqs
    return {"kv": kv, "q": q, "out": out, "ids": ids, "lens": lens, "total": kv + q + out + ids + lens}


def write_bytes(c, T: int, fused: bool) -> int:
    """New K and V of every sequence read once and stored once (+ the slot
    mapping when the write is its own call; the fused call finds the slot in
    the block table entries already counted for the decode)."""
    es = {"f32": 4, "f16": 2, "bf16": 2}[c.etype]
    return 2 * T * c.num_kv_heads * c.head_dim * es * 2 + (0 if fused else 4 * T)


# The oracle job the forked workers of oracle_timed() run: (fn(unit), work(unit)).
_ORACLE_JOB = None


def host_cores() -> int:
    """Cores this process may run on, capped at 16 (one GPU's share of an
    eight-GPU host's cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_worker(job):
    units, budget_s = job
    from threadpoolctl import threadpool_limits

    fn, work = _ORACLE_JOB
    done, amount = 0, 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for u in units:
            fn(u)
            done += 1
            amount += work(u)
            if time.perf_counter() - t0 >= budget_s:
                break
    return done, amount


def oracle_timed(fn, work, units, budget_s: float, procs: int) -> dict:
    """Runs fn(u) over `units` in order until the budget is spent (at least
    one unit per process), BLAS pinned to one thread per process. procs > 1:
    forked worker processes take units round-robin, each until the budget is
    spent; the figure is the summed work over the wall time of the whole
    pool. Called before anything touches the GPU."""
    global _ORACLE_JOB
    _ORACLE_JOB = (fn, work)
    units = list(units)
    t0 = time.perf_counter()
    if procs <= 1:
        done, amount = _oracle_worker((units, budget_s))
    else:
        import multiprocessing as mp

        with mp.get_context("fork").Pool(procs) as pool:
            parts = pool.map(_oracle_worker, [(units[k::procs], budget_s) for k in range(procs)])
        done, amount = sum(p[0] for p in parts), sum(p[1] for p in parts)
    dt = time.perf_counter() - t0
    _ORACLE_JOB = None
    return {"units": done, "amount": amount, "seconds": dt, "procs": procs}


def cpu_baseline(w, budget_s: float) -> dict:
    """The oracle, as it stands, on the same workload: one sequence (all
    heads) per unit in batch order, on every host core (forked processes),
    plus the single-process figure."""
    import oracle

    c = w.cfg
    kr, vr = oracle.write_kv(w.k_cache, w.v_cache, w.k_new, w.v_new, w.slot_mapping, c.block_size)
    es = {"f32": 4, "f16": 2, "bf16": 2}[c.etype]

    def fn(s):
        oracle.decode(w.q, kr, vr, w.block_tables, w.context_lens, c.scale, c.block_size, c.etype, seqs=[s])

    def work(s):
        return int(w.context_lens[s]) * c.num_kv_heads * c.head_dim * 2 * es

    procs = host_cores()
    one = oracle_timed(fn, work, range(c.num_seqs), budget_s / 3, 1)
    many = oracle_timed(fn, work, range(c.num_seqs), budget_s * 2 / 3, procs)

    def fig(r):
        return r["amount"] / r["seconds"] / 1e9

    return {"value": fig(many), "unit": "GB/s", "cores": procs, "kind": "oracle",
            "sample": f"{many['units']} of {c.num_seqs} sequences (all heads; worker k takes sequences k, k+{procs}, "
                      f"...) in {many['seconds']:.1f} s on {procs} forked processes, "
                      f"{many['units'] / many['seconds']:.2f} seq/s, float64 NumPy oracle",
            "single_thread": {"value": fig(one), "unit": "GB/s", "cores": 1,
                              "sample": f"first {one['units']} sequences in {one['seconds']:.1f} s, "
                                        f"{one['units'] / one['seconds']:.2f} seq/s"}}


def traffic_for(kernel: str, workload: str):
    """HBM bytes per step of the timed launches ("a+b+...": the sum over
    those kernels) from the committed counter summary, if it was taken on the
    current kernel sources and holds every one of them."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload, {})
    if entry.get("kernel_hash") != kernel_hash(workload):
        return None
    per = entry.get("kernels", {})
    names = kernel.split("+")
    if not all(k in per for k in names):
        return None
    return sum(per[k]["traffic_bytes"] for k in names)


# Kernels of the decode step's launches, in launch order: the planning
# launches of the shared split, the decode kernel, the closing merge launch.
DECODE_KERNELS = ("write_kv_kernel", "link_kernel", "plan_kernel", "decode_kernel", "merge_kernel")


def step_kernels(launches: int, fused: bool) -> str:
    """The timed step's kernels from the number of launches the decode call
    makes (pa_decode_launches): 1 decode only, 2 with the closing merge, 4
    with the shared split's two planning launches before them."""
    names = {1: ["decode_kernel"], 2: ["decode_kernel", "merge_kernel"],
             3: ["link_kernel", "plan_kernel", "decode_kernel"],
             4: ["link_kernel", "plan_kernel", "decode_kernel", "merge_kernel"]}[launches]
    return "+".join(names if fused else ["write_kv_kernel"] + names)


def summarize_counters(fetch_csv: str, write_csv: str, workload: str, calibration_mib: int) -> dict:
    """Per-launch HBM bytes of the step's kernels from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the
    counter read for the run's plain device copy of calibration_mib MiB, and
    recorded in the traffic file with the hash of the kernel sources."""
    import csv
    from collections import defaultdict

    def per_kernel(path):
        vals, calib = defaultdict(list), 0.0
        with open(path) as f:
            for r in csv.DictReader(f):
                name, v = r["Kernel_Name"], float(r["Counter_Value"])
                if name.startswith("__amd_rocclr_copyBuffer"):
                    calib = max(calib, v)
                    continue
                for k in DECODE_KERNELS + ("prefill_kernel",):
                    if f"::{k}<" in name or f"::{k}(" in name:
                        vals[k].append(v)
        return {k: float(np.mean(v)) for k, v in vals.items()}, calib

    fetch, fcal = per_kernel(fetch_csv)
    write, wcal = per_kernel(write_csv)
    want = calibration_mib * 1024.0
    fs, ws = want / fcal, want / wcal
    kernels = {k: {"fetch_kib_per_launch": round(fetch[k], 1), "write_kib_per_launch": round(write[k], 1),
                   "traffic_bytes": int(round((fetch[k] * fs + write[k] * ws) * 1024))}
               for k in fetch if k in write}
    entry = {"kernel_hash": kernel_hash(workload), "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
             "calibration": f"one {calibration_mib} MiB device-to-device torch copy (__amd_rocclr_copyBuffer) in "
                            f"the same run: FETCH_SIZE {fcal:.1f} KiB, WRITE_SIZE {wcal:.1f} KiB",
             "kernels": kernels}
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[workload] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    return entry


class Case:
    """Device inputs of the timed step and what the report needs about them."""


def unique_kv_bytes(c, tables, lens) -> int:
    """K and V bytes of the distinct blocks the step reads (a block several
    sequences map counts once, with the most tokens any of them reads)."""
    es = {"f32": 4, "f16": 2, "bf16": 2}[c.etype]
    B = c.block_size
    reads = {}
    for s, L in enumerate(lens.tolist()):
        for b in range(-(-L // B)):
            blk = int(tables[s, b])
            reads[blk] = max(reads.get(blk, 0), min(B, L - b * B))
    return sum(reads.values()) * c.num_kv_heads * c.head_dim * 2 * es


def decode_case(w, pb, dev, gen_s: float, torch=None, reps: int = 10) -> Case:
    """Device copies of a generated decode workload. A workload with
    copy-on-write pairs (a shared prefix ending inside a block) gets its
    copies -- timed here on their own -- and the writes into the copies
    before the timed decode steps, as the steps that made them would have."""
    c = Case()
    cfg = w.cfg
    c.gen_s = gen_s
    et = cfg.etype
    c.w, c.cfg = w, cfg
    c.extra = {}
    c.kc, c.vc = pb.to_device(w.k_cache, et, dev), pb.to_device(w.v_cache, et, dev)
    if w.copy_pairs is not None:
        pairs = pb.int32_to_device(w.copy_pairs, dev)
        for _ in range(3):   # idempotent until the writes below
            pb.pa_copy_blocks(c.kc, c.vc, pairs)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            pb.pa_copy_blocks(c.kc, c.vc, pairs)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        P = w.copy_pairs.shape[0]
        nbytes = 2 * P * cfg.num_kv_heads * cfg.block_size * cfg.head_dim * 2 * 2 + 8 * P
        c.extra["copy_blocks"] = {"pairs": P, "avg_ms": round(ms, 5), "bytes": nbytes,
                                  "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        pb.pa_write_kv(pb.to_device(w.pre_k, et, dev), pb.to_device(w.pre_v, et, dev), c.kc, c.vc,
                       pb.int32_to_device(w.pre_slots, dev))
        torch.cuda.synchronize()
    c.q = pb.to_device(w.q, et, dev)
    c.k_new, c.v_new = pb.to_device(w.k_new, et, dev), pb.to_device(w.v_new, et, dev)
    c.slots = pb.int32_to_device(w.slot_mapping, dev)
    c.bt, c.cl = pb.int32_to_device(w.block_tables, dev), pb.int32_to_device(w.context_lens, dev)
    c.copy_pairs = np.zeros((0, 2), np.int32)  # the timed step has no copies
    c.context_lens, c.max_len = w.context_lens, w.max_context_len
    c.unique_kv = unique_kv_bytes(cfg, w.block_tables, w.context_lens)
    return c


def loop_case(ps, nsteps: int, pb, dev, torch, reps: int) -> Case:
    """Runs steps 1..nsteps-1 of a multi-step workload (parallel sampling,
    beam search) on the device -- copies, then writes, as a serving loop
    would -- and returns step nsteps; the copy-on-write call of step 1 is
    timed on the way."""
    c = Case()
    t0 = time.perf_counter()
    cfg, et = ps.cfg, ps.cfg.etype
    c.cfg, c.w = cfg, None
    c.kc, c.vc = pb.to_device(ps.k_cache, et, dev), pb.to_device(ps.v_cache, et, dev)
    c.extra = {}
    for step in range(1, nsteps + 1):
        st = ps.step()
        pairs = pb.int32_to_device(st.block_mapping, dev) if st.block_mapping.shape[0] else None
        if step == 1 and pairs is not None:
            # repeated copies of one step are idempotent until the step writes
            for _ in range(3):
                pb.pa_copy_blocks(c.kc, c.vc, pairs)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                pb.pa_copy_blocks(c.kc, c.vc, pairs)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            P = st.block_mapping.shape[0]
            nbytes = 2 * P * cfg.num_kv_heads * cfg.block_size * cfg.head_dim * 2 * 2 + 8 * P
            c.extra["copy_blocks"] = {"pairs": P, "avg_ms": round(ms, 5), "bytes": nbytes,
                                      "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        if step == nsteps:
            break
        if pairs is not None:
            pb.pa_copy_blocks(c.kc, c.vc, pairs)
        pb.pa_write_kv(pb.to_device(st.k_new, et, dev), pb.to_device(st.v_new, et, dev), c.kc, c.vc,
                       pb.int32_to_device(st.slot_mapping, dev))
    torch.cuda.synchronize()
    c.q = pb.to_device(st.q, et, dev)
    c.k_new, c.v_new = pb.to_device(st.k_new, et, dev), pb.to_device(st.v_new, et, dev)
    c.slots = pb.int32_to_device(st.slot_mapping, dev)
    c.bt, c.cl = pb.int32_to_device(st.block_tables, dev), pb.int32_to_device(st.context_lens, dev)
    c.copy_pairs = st.block_mapping
    c.context_lens, c.max_len = st.context_lens, int(st.context_lens.max())
    c.unique_kv = unique_kv_bytes(cfg, st.block_tables, st.context_lens)
    c.extra["copy_pairs_timed_step"] = int(st.block_mapping.shape[0])
    c.gen_s = time.perf_counter() - t0
    return c


def swap_sweep(torch, pb, total_mib: int, reps: int) -> dict:
    """pa_swap_out / pa_swap_in of a shuffled set of blocks totalling
    total_mib MiB (K + V) per block size, Llama-3-8B head shape (8 KV heads,
    head_dim 128, bf16), against one contiguous device <-> pinned-host copy of
    the same size (the link's rate)."""
    dev = torch.device("cuda:0")
    res = {}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    nbytes = total_mib << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d2h = timed(lambda: host.copy_(src, non_blocking=True))
    h2d = timed(lambda: src.copy_(host, non_blocking=True))
    res["contiguous_copy"] = {"bytes": nbytes, "d2h_GBps": round(nbytes / d2h / 1e6, 1),
                              "h2d_GBps": round(nbytes / h2d / 1e6, 1)}
    del src, host
    rng = np.random.default_rng(0)
    for B in (8, 16, 32, 64, 128):
        block_bytes = 2 * 8 * B * 128 * 2
        n = nbytes // block_bytes
        kc = torch.empty((n, 8, B, 128), dtype=torch.bfloat16, device=dev)
        vc = torch.empty((n, 8, 128, B), dtype=torch.bfloat16, device=dev)
        space = pb.swap_space(n, kc)
        pairs = np.stack([rng.permutation(n), np.arange(n)], axis=1).astype(np.int32)
        m = pb.int32_to_device(pairs, dev)
        t_out = timed(lambda: pb.pa_swap_out(space, kc, vc, m))
        t_in = timed(lambda: pb.pa_swap_in(kc, vc, space, m))
        res[f"B{B}"] = {"blocks": int(n), "block_bytes": block_bytes,
                        "out_ms": round(t_out, 4), "out_GBps": round(n * block_bytes / t_out / 1e6, 1),
                        "in_ms": round(t_in, 4), "in_GBps": round(n * block_bytes / t_in / 1e6, 1)}
        del kc, vc, space
    return res


def shape_sweep(torch, pb, wl, reps: int) -> list:
    """pa_write_decode over a grid of batch sizes and equal context lengths
    (Llama-3-8B head shape: 32 query / 8 KV heads, head_dim 128, block 16,
    bf16, shuffled pool, balanced split), up to 4.2 M context tokens per step.
    K/V values are seeded normal draws on the device (timing only). Each
    shape is timed twice: calls issued one by one from Python (where small
    steps wait on the host's issue rate), and the same calls replayed from
    a HIP graph (the GPU's time)."""
    import dataclasses

    dev = torch.device("cuda:0")
    base = wl.CONFIGS["llama3_8b"]
    rows = []
    for S in (1, 4, 16, 64, 256, 1024):
        for L in (256, 1024, 4096, 16384, 65536):
            if not 2048 <= S * L <= 4_200_000:
                continue
            cfg = dataclasses.replace(base, num_seqs=S, lengths=("fixed", (L,) * S), max_len=L)
            w = wl.make_decode_workload(cfg, values=False)
            NB, Hkv, B, d = w.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim
            g = torch.Generator(device=dev)
            g.manual_seed(0)
            kc = torch.randn((NB, Hkv, B, d), device=dev, dtype=torch.bfloat16, generator=g)
            vc = torch.randn((NB, Hkv, d, B), device=dev, dtype=torch.bfloat16, generator=g)
            q = torch.randn((S, cfg.num_heads, d), device=dev, dtype=torch.bfloat16, generator=g)
            kn = torch.randn((S, Hkv, d), device=dev, dtype=torch.bfloat16, generator=g)
            vn = torch.randn((S, Hkv, d), device=dev, dtype=torch.bfloat16, generator=g)
            bt, cl = pb.int32_to_device(w.block_tables, dev), pb.int32_to_device(w.context_lens, dev)
            out = torch.empty(q.shape, dtype=torch.float32, device=dev)
            need = pb.pa_decode_workspace_bytes(S, cfg.num_heads, cfg.num_kv_heads, d, w.max_context_len, -1)
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)

            def step():
                pb.pa_write_decode(out, q, kn, vn, kc, vc, bt, cl, cfg.scale, w.max_context_len, workspace=ws)

            for _ in range(10):
                step()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                step()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / reps * 1000
            # the same steps replayed from a HIP graph: the GPU's own time per
            # step, without the host's cost of issuing each call
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for _ in range(reps):
                    step()
            graph.replay()
            torch.cuda.synchronize()
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            gus = e0.elapsed_time(e1) / reps * 1000
            del graph
            nbytes = decode_bytes(cfg, w.context_lens)["total"] + write_bytes(cfg, S, True)
            rows.append({"num_seqs": S, "context_len": L, "step_us": round(us, 1), "graph_step_us": round(gus, 1),
                         "bytes": nbytes, "GBps": round(nbytes / us / 1e3),
                         "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 3),
                         "graph_frac": round(nbytes / gus / 1e3 / HBM_PEAK_GBS, 3),
                         "launches": pb.pa_decode_launches(S, cfg.num_heads, cfg.num_kv_heads, d, w.max_context_len,
                                                           -1, q.dtype, "auto", True)})
            print(json.dumps(rows[-1]), flush=True)
            del kc, vc
            torch.cuda.empty_cache()
    return rows


def cold_calls(step, n: int, torch, dev) -> dict:
    """n single steps, each after an untimed 1 GiB write of scratch memory
    (evicts the L2s and the Infinity Cache), each timed by its own event pair
    on the launch stream: the per-call time with nothing of the inputs
    cached."""
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    times = []
    for _ in range(n):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    return {"calls": n, "median_ms": round(float(np.median(times)), 5), "min_ms": round(float(min(times)), 5),
            "timed": "one event pair per call, each after an untimed 1 GiB scratch write"}


def calibration_copy(args, torch, dev) -> None:
    """One plain device copy of known size, run before the timed launches, for
    the traffic counters' calibration."""
    if args.calibration_copy_mib:
        n = args.calibration_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def copy_reference(torch, dev, mib: int = 2048, reps: int = 5) -> dict:
    """A plain device-to-device copy of `mib` MiB timed on this GPU (HIP
    events around `reps` back-to-back copies after one untimed copy): the
    on-box bandwidth of the simplest streaming kernel, reads plus writes."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"kernel": f"torch copy_ of {mib} MiB, device to device", "bytes": 2 * n,
            "ms": round(ms, 4), "GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}


def prefill_cpu_baseline(w, budget_s: float) -> dict:
    """The oracle on whole prompts, shortest first, on every host core
    (forked processes), plus the single-process figure."""
    import oracle

    c = w.cfg
    order = np.argsort(w.context_lens, kind="stable").tolist()
    n = w.queries.astype(np.int64)
    L = w.context_lens.astype(np.int64)

    def fn(s):
        oracle.prefill(w.q, w.q_start, w.k_cache, w.v_cache, w.block_tables, w.context_lens, c.scale,
                       c.block_size, c.etype, seqs=[s])

    def work(s):
        pairs = int(n[s] * (L[s] - n[s]) + n[s] * (n[s] + 1) // 2)
        return pairs * c.num_heads * c.head_dim * 4

    procs = host_cores()
    one = oracle_timed(fn, work, order, budget_s / 3, 1)
    many = oracle_timed(fn, work, order, budget_s * 2 / 3, procs)
    return {"value": many["amount"] / many["seconds"] / 1e12, "unit": "TFLOP/s", "cores": procs, "kind": "oracle",
            "sample": f"{many['units']} of the shortest of {c.num_seqs} prompts (all heads) in {many['seconds']:.1f} s "
                      f"on {procs} forked processes, float64 NumPy oracle",
            "single_thread": {"value": one["amount"] / one["seconds"] / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "sample": f"the {one['units']} shortest prompts in {one['seconds']:.1f} s"}}


def prefill_main(args, torch, pb, wl, dev) -> int:
    """One step = pa_prefill over the whole batch (K/V already in the pool)."""
    import dataclasses
    cfg = wl.PREFILL if not args.block_size else dataclasses.replace(wl.PREFILL, block_size=args.block_size)
    t0 = time.perf_counter()
    w = wl.make_prefill_workload(cfg, contiguous=args.contiguous)
    gen_s = time.perf_counter() - t0
    # the oracle runs before the library is loaded or the GPU touched
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(w, args.cpu_budget)
    pb.load_library()
    et = cfg.etype
    q = pb.to_device(w.q, et, dev)
    out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    qs, kc, vc = pb.int32_to_device(w.q_start, dev), pb.to_device(w.k_cache, et, dev), pb.to_device(w.v_cache, et, dev)
    bt, cl = pb.int32_to_device(w.block_tables, dev), pb.int32_to_device(w.context_lens, dev)
    calibration_copy(args, torch, dev)

    def step():
        pb.pa_prefill(out, q, qs, kc, vc, bt, cl, cfg.scale)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = elapsed * 1e3 / args.steps
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (call_ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[et]
    result = {
        "metric": "prompt-phase attention over the paged cache: achieved TFLOP/s at 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": et,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT["prefill"], "num_seqs": cfg.num_seqs, "total_queries": w.total_q,
                   "max_context_len": int(w.context_lens.max()), "block_size": cfg.block_size,
                   "pool": "contiguous" if args.contiguous else "shuffled"},
        "flops": flops,
        "flops_rule": "4 * head_dim per (query head, query, visible cached token): QK and PV products",
        "tokens_per_s": round(w.total_q / (ms_per_step * 1e-3), 1),
        "prefill": {"call": "pa_prefill", "avg_ms": round(call_ms, 5), "kv_bytes": w.kv_bytes(),
                    "timed": "HIP events on the launch stream around the timed steps, divided by the steps"},
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel", "achieved": round(achieved, 1), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic_for("prefill_kernel", "prefill")},
        "input_generation_s": round(gen_s, 2),
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    return 0


def pool_name(args) -> str:
    """How the decode workload's blocks are placed in the pool."""
    return "reserved" if args.reserved else "contiguous" if args.contiguous else "shuffled"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="llama3_8b", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--algo", default="auto", choices=["auto", "vector", "mfma"])
    ap.add_argument("--partition", type=int, default=None, help="partition size (-1 balanced, 0 none)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--block-size", type=int, default=None, help="tokens per block (default: the workload's)")
    ap.add_argument("--contiguous", action="store_true",
                    help="hand out the pool's blocks in order instead of the seeded shuffled order")
    ap.add_argument("--reserved", action="store_true",
                    help="decode: give every sequence a max_len region of its own (logical block i of sequence "
                         "s at block s * max_blocks + i), the reservation that paging replaces")
    ap.add_argument("--two-calls", action="store_true", help="time pa_write_kv + pa_decode instead of the fused call")
    ap.add_argument("--prefix-len", type=int, default=1024,
                    help="shared_prefix: tokens of the shared prefix (not a multiple of 16: copy-on-write of its "
                         "last block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", type=int, default=20, metavar="N",
                    help="also time N single steps, each after evicting the caches (0: skip)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run one plain device copy of this size first (traffic counter calibration)")
    ap.add_argument("--swap-sweep", type=int, default=0, metavar="MIB",
                    help="measure pa_swap_out/pa_swap_in of MIB MiB of blocks per block size and exit")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="time pa_write_decode over a grid of batch sizes and context lengths and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic file from two rocprofv3 counter_collection.csv files and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        entry = summarize_counters(*args.summarize_counters, args.workload, args.calibration_copy_mib or 1024)
        print(json.dumps(entry, indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode path here has no "
              "multi-GPU mode: per-GPU work is the single-GPU kernel on that GPU's share", file=sys.stderr)
        return 2

    import torch

    from paged_kv_cache_131_amd import binding as pb
    from paged_kv_cache_131_amd import workloads as wl

    dev = torch.device("cuda:0")
    if args.contiguous and args.reserved:
        raise SystemExit("--contiguous and --reserved are two different pool layouts")
    if args.reserved and args.workload == "prefill":
        raise SystemExit("--reserved applies to the decode workloads")
    if args.workload == "prefill" and not (args.swap_sweep or args.shape_sweep):
        return prefill_main(args, torch, pb, wl, dev)
    # a drawn workload is generated first and the oracle's baseline timed on
    # it before the library is loaded or the GPU touched
    w0, cpu = None, None
    if args.workload in ("shared_prefix",) + tuple(wl.CONFIGS) and not (args.swap_sweep or args.shape_sweep):
        import dataclasses
        t0 = time.perf_counter()
        if args.workload == "shared_prefix":
            w0 = wl.make_shared_prefix_workload(prefix_len=args.prefix_len)
        else:
            cfg0 = wl.CONFIGS[args.workload]
            if args.block_size:
                cfg0 = dataclasses.replace(cfg0, block_size=args.block_size)
            w0 = wl.make_decode_workload(cfg0, contiguous=args.contiguous, reserved=args.reserved)
        gen_s = time.perf_counter() - t0
        if not args.no_cpu_baseline:
            cpu = cpu_baseline(w0, args.cpu_budget)
    pb.load_library()
    if args.swap_sweep:
        print(json.dumps({"swap_sweep": swap_sweep(torch, pb, args.swap_sweep, 5)}), flush=True)
        return 0
    if args.shape_sweep:
        print(json.dumps({"shape_sweep": shape_sweep(torch, pb, wl, 50)}), flush=True)
        return 0
    if args.workload in ("parallel_sampling", "beam_search", "shared_prefix") and (
            args.block_size or args.contiguous or args.reserved):
        raise SystemExit("--block-size/--contiguous/--reserved apply to the drawn-length workloads")
    if args.workload == "parallel_sampling":
        c = loop_case(wl.ParallelSamplingWorkload(prompt_len=1016), 256, pb, dev, torch, max(args.steps, 10))
    elif args.workload == "beam_search":
        c = loop_case(wl.BeamSearchWorkload(), 64, pb, dev, torch, max(args.steps, 10))
    else:
        c = decode_case(w0, pb, dev, gen_s, torch, max(args.steps, 10))
    cfg, et = c.cfg, c.cfg.etype
    part = cfg.partition_size if args.partition is None else args.partition
    kc, vc, q, k_new, v_new, slots, bt, cl = c.kc, c.vc, c.q, c.k_new, c.v_new, c.slots, c.bt, c.cl
    copies = pb.int32_to_device(c.copy_pairs, dev) if c.copy_pairs.shape[0] else torch.empty(
        (0, 2), dtype=torch.int32, device=dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    max_len = c.max_len

    calibration_copy(args, torch, dev)

    fused = not args.two_calls
    if fused and args.algo != "auto":
        raise SystemExit("--algo needs --two-calls (the fused call picks the kernel family itself)")

    def step():
        pb.pa_copy_blocks(kc, vc, copies)   # this step's copy-on-write pairs (none here: no launch)
        if fused:
            pb.pa_write_decode(out, q, k_new, v_new, kc, vc, bt, cl, cfg.scale, max_len, partition_size=part)
        else:
            pb.pa_write_kv(k_new, v_new, kc, vc, slots)
            pb.pa_decode(out, q, kc, vc, bt, cl, cfg.scale, max_len, partition_size=part, algo=args.algo)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # one event pair on the launch stream brackets the timed steps (events
    # between the launches would add their own gaps to what they measure)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    call_ms = ev0.elapsed_time(ev1) / args.steps

    cold = cold_calls(step, args.cold, torch, dev) if args.cold else None

    db = decode_bytes(cfg, c.context_lens)
    wb = write_bytes(cfg, len(c.context_lens), fused)
    if c.unique_kv != db["kv"]:
        # shared blocks count once: the bytes HBM must deliver at least
        db["kv_logical"] = db["kv"]
        db["total"] += c.unique_kv - db["kv"]
        db["kv"] = c.unique_kv
    step_bytes = db["total"] + wb
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # per step on the GPU: the call's launches (the decode kernel; the
    # shared split's planning launches before it; the closing launch that
    # merges split sequences and stores the new tokens, unless the decode
    # kernel does both itself)
    launch_bytes = step_bytes if fused else db["total"] + wb
    achieved = launch_bytes / (call_ms * 1e-3) / 1e9
    launches = pb.pa_decode_launches(len(c.context_lens), cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, max_len,
                                     part, q.dtype, args.algo, fused)
    kernel = step_kernels(launches, fused)
    traffic = traffic_for(kernel, args.workload)
    result = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) + sequences/s at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": et,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_TEXT[args.workload].format(prefix=args.prefix_len),
            "num_seqs": len(c.context_lens),
            "context_tokens": int(c.context_lens.astype(np.int64).sum()),
            "max_context_len": max_len,
            "partition_size": part,
            "block_size": cfg.block_size,
            "pool": pool_name(args),
            "algo": args.algo,
            "step": ("copy blocks (0 pairs) + fused write 1 token/seq and decode" if fused
                     else "copy blocks (0 pairs) + write 1 token/seq + decode"),
        },
        "sequences_per_s": round(len(c.context_lens) / (ms_per_step * 1e-3), 1),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "step_bytes": step_bytes,
        "decode": {"call": "pa_write_decode" if fused else "pa_write_kv + pa_decode", "bytes": db,
                   "write_bytes": wb, "launch_bytes": launch_bytes, "avg_ms": round(call_ms, 5),
                   "GBps": round(achieved, 1), "seq_per_s": round(len(c.context_lens) / (call_ms * 1e-3), 1),
                   "timed": "HIP events on the launch stream around the timed steps, divided by the steps"},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "input_generation_s": round(c.gen_s, 2),
        **c.extra,
    }
    if cold:
        med, mn = cold["median_ms"], cold["min_ms"]
        cold["GBps_median"] = round(launch_bytes / (med * 1e-3) / 1e9, 1)
        cold["GBps_min_time"] = round(launch_bytes / (mn * 1e-3) / 1e9, 1)
        result["cold_cache"] = cold
    if not args.calibration_copy_mib:  # a counter run's only copy is the calibration copy
        ref = copy_reference(torch, dev)
        ref["decode_frac_of_copy"] = round(achieved / ref["GBps"], 4)
        result["copy_reference"] = ref
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
