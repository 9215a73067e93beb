#!/usr/bin/env python3
"""Throughput of top-k sparse MLA decode on one MI355X.

A step is one sparse_mla_decode_run call over the whole workload (index translation,
gather + dequant, QK, online softmax with sinks, PV, and the split merge when the plan
splits).  Inputs are seeded synthetic data resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints one JSON line.  The default workload is b128_mtp4_h128_fp8: 128 requests x 4
MTP rows, 128 heads, top-k 2048 over contexts of 8K..128K tokens, FP8+UE8M0 cache.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PMC_FILE = os.path.join(ROOT, "profiles", "decode_b128_mtp4_h128_fp8_pmc.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_mla_decode_03_amd", "csrc", f)
                  for f in ("smla_decode.hip", "smla_device.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def pmc_traffic(launch_units: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    if not os.path.exists(PMC_FILE):
        return None
    kv = {}
    with open(PMC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        fetch = float(kv["fetch_kib_per_dispatch"]) * 1024 / float(kv["fetch_copy_factor"])
        write = float(kv["write_kib_per_dispatch"]) * 1024 / float(kv["write_copy_factor"])
    except (KeyError, ValueError):
        return None
    return fetch + write


def cache_store_measure(B, torch, dev, n_tokens: int, reps: int):
    """Time sparse_mla_cache_store (FP8 + UE8M0, page size 64) writing n_tokens new tokens
    to distinct random slots of a pool twice their size.  Algorithmic bytes per token:
    1024 (bf16 latent) + 128 (bf16 rope) + 4 (slot) read, 512 + 128 + 8 written."""
    ps = 64
    npages = max(2, 2 * n_tokens // ps)
    g = torch.Generator(device=dev).manual_seed(17)
    cache = torch.zeros((npages, 648 * ps), dtype=torch.uint8, device=dev)
    lat = torch.randn((n_tokens, 512), generator=g, device=dev).to(torch.bfloat16)
    rope = torch.randn((n_tokens, 64), generator=g, device=dev).to(torch.bfloat16)
    slots = torch.randperm(npages * ps, generator=g, device=dev)[:n_tokens].to(torch.int32)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        B.cache_store(cache, "fp8", ps, lat, rope, slots, stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        e0.record(stream)
        B.cache_store(cache, "fp8", ps, lat, rope, slots, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    mean_s = sum(ms) / len(ms) / 1e3
    nbytes = n_tokens * (1024 + 128 + 4 + 512 + 128 + 8)
    return {"tokens": n_tokens, "page_size": ps, "pages": npages,
            "launch_ms_mean": mean_s * 1e3, "launch_ms_p50": ms[len(ms) // 2],
            "tokens_per_s": n_tokens / mean_s,
            "roofline": {"bound": "hbm", "achieved": nbytes / mean_s / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": nbytes / mean_s / 1e9 / PEAK_HBM_GBS,
                         "bytes_per_launch": nbytes}}


def kv_code(B, name: str) -> int:
    return {"bf16": B.KV_BF16, "fp8": B.KV_FP8_UE8M0, "fp8t": B.KV_FP8_TENSOR}[name]


def decode_measure(B, W, torch, dev, name: str, reps: int, seed: int):
    """Time one decode launch of a workload other than the headline one: the batch that
    mixes prefill chunks and decode rows, or the headline shape over another cache format."""
    spec = W.WORKLOADS[name]
    inp = W.make_inputs(spec, seed, device=dev, cache_device=dev)
    R, H = inp.num_rows, inp.num_heads
    prob = B.make_problem(R, spec.num_requests, H, spec.topk, spec.page_size, inp.num_pages,
                          inp.page_table.shape[1], kv_code(B, spec.kv_format), B.IDX_LOGICAL, 0, 0,
                          spec.softmax_scale, spec.kv_scale)
    info = B.plan(prob)
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    ws = (torch.empty(info.workspace_bytes, dtype=torch.uint8, device=dev)
          if info.workspace_bytes else None)
    stream = torch.cuda.current_stream()

    def step():
        B.run(info, inp.q, inp.kv_cache, inp.indices, inp.row_req, inp.page_table, inp.sinks,
              out, lse, None, None, ws, stream)

    for _ in range(3):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    mean_s = sum(ms) / len(ms) / 1e3
    n = inp.num_valid()
    flops = W.algorithmic_flops(inp)
    counts = torch.bincount(inp.row_req.long().cpu()).tolist()
    del inp
    return {"workload": name, "kv_format": spec.kv_format, "rows": R, "requests": spec.num_requests,
            "rows_per_request": {str(k): counts.count(k) for k in sorted(set(counts))},
            "attended_entries": n, "num_splits": info.num_splits,
            "launch_ms_mean": mean_s * 1e3, "launch_ms_p50": ms[len(ms) // 2],
            "entries_per_s": n / mean_s,
            "roofline": {"bound": "mfma", "achieved": flops / mean_s / 1e12, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / mean_s / 1e12 / PEAK_BF16_TFLOPS,
                         "flops_per_launch": flops}}


def workload_measure(B, W, torch, dev, name: str, seed: int, reps: int):
    """One decode call (split decode and merge included) on another of the five workloads:
    warm launches back to back, and cold launches each after a 1 GiB write that evicts the
    caches; throughput and roofline fractions are taken on the cold median."""
    spec = W.WORKLOADS[name]
    inp = W.make_inputs(spec, seed, device=dev, cache_device=dev)
    R, H = inp.num_rows, inp.num_heads
    prob = B.make_problem(R, spec.num_requests, H, spec.topk, spec.page_size, inp.num_pages,
                          inp.page_table.shape[1], kv_code(B, spec.kv_format), B.IDX_LOGICAL,
                          spec.num_splits, spec.flags, spec.softmax_scale, spec.kv_scale)
    info = B.plan(prob)
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    ws = (torch.empty(info.workspace_bytes, dtype=torch.uint8, device=dev)
          if info.workspace_bytes else None)
    stream = torch.cuda.current_stream()
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def step():
        B.run(info, inp.q, inp.kv_cache, inp.indices, inp.row_req, inp.page_table, inp.sinks,
              out, lse, None, None, ws, stream)

    for _ in range(3):
        step()
    times = {}
    for mode in ("warm", "cold"):
        ms = []
        for i in range(reps):
            if mode == "cold":
                scratch.fill_(i & 255)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        ms.sort()
        times[mode] = ms[len(ms) // 2]
    t = times["cold"] / 1e3
    n = inp.num_valid()
    flops = W.algorithmic_flops(inp)
    cbytes = W.compulsory_bytes(inp)
    hbm_frac = cbytes / t / 1e9 / PEAK_HBM_GBS
    mfma_frac = flops / t / 1e12 / PEAK_BF16_TFLOPS
    del inp, scratch
    return {"kv_format": spec.kv_format, "rows": R, "heads": H, "num_splits": info.num_splits,
            "balanced_rows": bool(spec.flags & B.F_BALANCE_ROWS),
            "attended_entries": n, "launch_ms_p50": times["warm"], "cold_cache_launch_ms_p50": times["cold"],
            "entries_per_s": n / t, "tokens_per_s": R / t,
            "hbm_tb_s": cbytes / t / 1e12, "hbm_frac": hbm_frac,
            "mfma_tflop_s": flops / t / 1e12, "mfma_frac": mfma_frac,
            "bound": "hbm" if hbm_frac >= mfma_frac else "mfma",
            "compulsory_bytes": cbytes, "flops": flops}


def indexer_measure(B, W, torch, dev, name: str, reps: int):
    """Time the indexer on one workload: the logits kernel and the top-k kernel, each
    launched `reps` times after warm-up, HIP events on the launch stream."""
    spec = W.INDEXER_WORKLOADS[name]
    inp = W.make_indexer_inputs(spec, 5, device=dev, cache_device=dev)
    stream = torch.cuda.current_stream()
    logits = torch.empty((inp.num_rows, inp.width), dtype=torch.float32, device=dev)
    out = torch.empty((inp.num_rows, spec.topk), dtype=torch.int32, device=dev)

    def logits_call():
        B.indexer_logits(inp.q_codes, inp.weights, inp.key_cache, inp.row_len, inp.page_table,
                         spec.next_n, inp.width, logits=logits, stream=stream)

    def topk_call():
        B.indexer_topk(logits, inp.row_len, spec.topk, out=out, stream=stream)

    def timed(fn):
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        return sum(ms) / len(ms), ms[len(ms) // 2]

    lg_mean, lg_p50 = timed(logits_call)
    tk_mean, tk_p50 = timed(topk_call)
    nbytes = W.indexer_algorithmic_bytes(inp)
    flops = W.indexer_algorithmic_flops(inp)
    positions = int(inp.row_len.sum().item())
    tk_bytes = positions * 4 + inp.num_rows * spec.topk * 4 + inp.num_rows * 4
    gbs = nbytes / (lg_mean / 1e3) / 1e9
    return {"workload": name, "rows": inp.num_rows, "next_n": spec.next_n, "heads": spec.num_heads,
            "topk": spec.topk, "visible_positions": positions,
            "logits_ms_mean": lg_mean, "logits_ms_p50": lg_p50,
            "topk_ms_mean": tk_mean, "topk_ms_p50": tk_p50,
            "logits_roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": gbs / PEAK_HBM_GBS, "bytes_per_launch": nbytes,
                                "fp8_tflop_s": flops / (lg_mean / 1e3) / 1e12,
                                "fp8_frac": flops / (lg_mean / 1e3) / 1e12 / PEAK_FP8_TFLOPS},
            "topk_roofline": {"bound": "hbm", "achieved": tk_bytes / (tk_mean / 1e3) / 1e9,
                              "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": tk_bytes / (tk_mean / 1e3) / 1e9 / PEAK_HBM_GBS,
                              "bytes_per_launch": tk_bytes}}


def _oracle_rows_worker(task):
    """One chunk of rows through the float64 oracle in a single-threaded worker process:
    returns the attended entries, the seconds spent, and the output differences against
    the GPU's bf16 result for the same rows (the non-gating tight diagnostic)."""
    import numpy as np

    from oracle import sparse_mla_oracle as orc

    d, lo, hi, deadline, meta = task
    if time.time() > deadline:
        return 0, 0, 0.0, 0.0, 0.0, 0, 0.0
    ld = lambda n: np.load(os.path.join(d, n + ".npy"), mmap_mode="r")  # noqa: E731
    cache = np.memmap(os.path.join(d, "cache.u8"), dtype=np.uint8, mode="r",
                      shape=tuple(meta["cache_shape"]))
    q, idx, rr, pt = ld("q"), ld("indices"), ld("row_req"), ld("page_table")
    gout, glse = ld("gpu_out"), ld("gpu_lse")
    sinks = ld("sinks") if meta["has_sinks"] else None
    t0 = time.perf_counter()
    o, lse = orc.sparse_mla_decode(q, cache, meta["kv_format"], meta["page_size"], idx, rr, pt,
                                   sinks, meta["softmax_scale"], rows=range(lo, hi),
                                   kv_scale=meta["kv_scale"])
    secs = time.perf_counter() - t0
    g = orc.bf16_bits_to_f64(np.asarray(gout[lo:hi]))
    dd = np.abs(g - o)
    lr = np.abs(np.asarray(glse[lo:hi], dtype=np.float64) - lse) / np.maximum(1.0, np.abs(lse))
    lr = lr[np.isfinite(lse)]
    entries = int((np.asarray(idx[lo:hi]) != -1).sum())
    return hi - lo, entries, secs, float(dd.sum()), float(dd.max()), dd.size, \
        float(lr.max()) if lr.size else 0.0


def cpu_baseline(inp, out, lse, budget_s: float):
    """The float64 oracle on the same workload, timed on this host's cores: one
    single-threaded worker process per core the process may run on (BLAS pinned to one
    thread), each taking contiguous row ranges, over as many rows as about budget_s of wall
    time allows.  The oracle reads the same cache bytes (a copy in shared memory) and the
    same indices; its outputs are compared with the GPU's (mean and max |d|, LSE relative),
    a diagnostic beside the gating tolerance."""
    import multiprocessing as mp
    import shutil
    import tempfile

    import numpy as np
    import torch

    from oracle import sparse_mla_oracle as orc

    cores = len(os.sched_getaffinity(0))
    d = tempfile.mkdtemp(prefix="smla_cpu_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        t_prep = time.perf_counter()
        cache = inp.kv_cache.cpu().numpy()
        cache.tofile(os.path.join(d, "cache.u8"))
        shape = cache.shape
        del cache
        sv = lambda n, a: np.save(os.path.join(d, n + ".npy"), a)  # noqa: E731
        sv("q", inp.q.cpu().view(torch.int16).numpy().view(np.uint16))
        sv("indices", inp.indices.cpu().numpy())
        sv("row_req", inp.row_req.cpu().numpy())
        sv("page_table", inp.page_table.cpu().numpy())
        sv("gpu_out", out.cpu().view(torch.int16).numpy().view(np.uint16))
        sv("gpu_lse", lse.cpu().numpy())
        if inp.sinks is not None:
            sv("sinks", inp.sinks.cpu().numpy())
        t_prep = time.perf_counter() - t_prep
        meta = {"cache_shape": list(shape), "has_sinks": inp.sinks is not None,
                "kv_format": {"bf16": orc.KV_BF16, "fp8": orc.KV_FP8_UE8M0,
                              "fp8t": orc.KV_FP8_TENSOR}[inp.spec.kv_format],
                "page_size": inp.spec.page_size, "softmax_scale": inp.spec.softmax_scale,
                "kv_scale": inp.spec.kv_scale}
        env_keep = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                  "MKL_NUM_THREADS")}
        for k in env_keep:
            os.environ[k] = "1"
        ctx = mp.get_context("spawn")
        R = inp.num_rows
        chunk = 2
        try:
            with ctx.Pool(cores) as pool:
                # warm: every worker imports numpy and the oracle before the clock starts
                pool.map(_oracle_rows_worker, [(d, 0, 0, 0.0, meta)] * cores)
                t0 = time.perf_counter()
                deadline = time.time() + budget_s
                tasks = [(d, lo, min(R, lo + chunk), deadline, meta) for lo in range(0, R, chunk)]
                res = pool.map(_oracle_rows_worker, tasks, chunksize=1)
                wall = time.perf_counter() - t0
        finally:
            for k, v in env_keep.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
    finally:
        shutil.rmtree(d, ignore_errors=True)
    rows = sum(r[0] for r in res)
    entries = sum(r[1] for r in res)
    n_el = sum(r[5] for r in res)
    mean_abs = sum(r[3] for r in res) / max(1, n_el)
    return {"value": entries / wall, "unit": "entries/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {R} rows ({entries} attended entries) of the same workload, "
                      f"float64 numpy oracle, {cores} single-threaded worker processes, "
                      f"{wall:.1f} s wall (cache copy to shared memory {t_prep:.1f} s, not timed)",
            "tokens_per_s": rows / wall,
            "tight_diagnostic": {"rows": rows, "mean_abs": mean_abs,
                                 "max_abs": max([r[4] for r in res] or [0.0]),
                                 "lse_rel_max": max([r[6] for r in res] or [0.0]),
                                 "mean_abs_bound": 2.5e-4, "gating": False,
                                 "within": mean_abs <= 2.5e-4}}


def cpu_single_process(B, W, torch, dev, name: str, seed: int):
    """The oracle in this process with BLAS on one thread, over every row of a workload."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import sparse_mla_oracle as orc

    spec = W.WORKLOADS[name]
    inp = W.make_inputs(spec, seed, device=dev, cache_device=dev)
    qb = inp.q.cpu().view(torch.int16).numpy().view(np.uint16)
    cache = inp.kv_cache.cpu().numpy()
    kvf = {"bf16": orc.KV_BF16, "fp8": orc.KV_FP8_UE8M0, "fp8t": orc.KV_FP8_TENSOR}[spec.kv_format]
    sinks = None if inp.sinks is None else inp.sinks.cpu().numpy()
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        orc.sparse_mla_decode(qb, cache, kvf, spec.page_size, inp.indices.cpu().numpy(),
                              inp.row_req.cpu().numpy(), inp.page_table.cpu().numpy(), sinks,
                              spec.softmax_scale, kv_scale=spec.kv_scale)
        secs = time.perf_counter() - t0
    n = inp.num_valid()
    return {"workload": name, "rows": inp.num_rows, "attended_entries": n, "seconds": secs,
            "value": n / secs, "unit": "entries/s", "cores": 1, "kind": "oracle"}


def spike_measure(B, torch, inp, info, out, lse, ws, stream, excess_log2: float, every: int = 64,
                  rounds: int = 4, per_round: int = 5):
    """The headline launch with one spiked row in every `every`: for head 0 of each such
    row, the cache entry at list position 1287 (tile 40 of 64) gets a rope part that is a
    multiple of the row's rope query, so its score lies about excess_log2 log2 units above
    the row's typical largest score (N(0,1) scores: about 2).  Spiked and plain launches
    alternate in blocks; the entries' original bytes are restored afterwards."""
    import math

    ps = inp.spec.page_size
    scale = inp.spec.softmax_scale
    R = inp.num_rows
    pos = min(40 * 32 + 7, inp.indices.shape[1] - 1)
    rows = torch.arange(0, R, every, device=inp.indices.device)
    t = inp.indices[rows, pos].long()
    page = inp.page_table[inp.row_req[rows].long(), t // ps].long()
    rr = t % ps
    col = (512 * ps + rr * 128)[:, None] + torch.arange(128, device=t.device)[None, :]
    orig = inp.kv_cache[page[:, None], col].clone()
    qr = inp.q[rows, 0, 512:].float()
    target = excess_log2 * math.log(2.0) + 2.0
    alpha = target / (scale * (qr * qr).sum(dim=1, keepdim=True))
    spiked = (alpha * qr).to(torch.bfloat16).contiguous().view(torch.uint8).reshape(-1, 128)

    def step():
        B.run(info, inp.q, inp.kv_cache, inp.indices, inp.row_req, inp.page_table, inp.sinks,
              out, lse, None, None, ws, stream)

    times = {"spiked": [], "plain": []}
    try:
        for rnd in range(rounds):
            for mode in (("spiked", "plain") if rnd % 2 == 0 else ("plain", "spiked")):
                inp.kv_cache[page[:, None], col] = spiked if mode == "spiked" else orig
                step()
                evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(per_round)]
                for e0, e1 in evs:
                    e0.record(stream)
                    step()
                    e1.record(stream)
                torch.cuda.synchronize()
                times[mode] += [e0.elapsed_time(e1) for e0, e1 in evs]
    finally:
        inp.kv_cache[page[:, None], col] = orig
        torch.cuda.synchronize()
    ms = {k: sum(v) / len(v) for k, v in times.items()}
    return {"every": every, "spiked_rows": int(rows.numel()), "target_excess_log2": excess_log2,
            "list_position": pos, "spiked_launch_ms_mean": ms["spiked"],
            "plain_launch_ms_mean": ms["plain"], "ratio": ms["spiked"] / ms["plain"]}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="b128_mtp4_h128_fp8")
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--num-splits", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="wall seconds of the multi-process oracle baseline (rows started "
                         "before it ends are finished)")
    ap.add_argument("--cpu-single", default="b32_h64_fp8:2",
                    help="workload:seed timed with the oracle in one process on one core "
                         "('' to skip)")
    ap.add_argument("--spike-every", type=int, default=64,
                    help="also time the headline launch with one spiked row in every N (0: skip)")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra launches, each after a 1 GiB scratch write that evicts the "
                         "caches (L2 and the 256 MB MALL); reported beside the warm figure")
    ap.add_argument("--store-tokens", type=int, default=65536,
                    help="tokens per timed cache-store launch (0: skip that measurement)")
    ap.add_argument("--mixed", default="mixed_b24_h128_fp8",
                    help="prefill+decode batch measured beside the decode ('' to skip)")
    ap.add_argument("--fp8-tensor", default="b128_mtp4_h128_fp8t",
                    help="also time this workload over the contiguous per-tensor FP8 cache "
                         "(empty: skip)")
    ap.add_argument("--indexer", default="idx_b128_mtp4_h64",
                    help="indexer workload measured beside the decode ('' to skip)")
    ap.add_argument("--other-workloads",
                    default="tiny_bf16:1,b32_h64_fp8:2,b2_h128_bf16_split16:4,ragged_b256_h64_fp8:5",
                    help="the other decode workloads (name:seed, comma separated; '' to skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run only a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by rows, with no exchange between GPUs)", file=sys.stderr)
        return 2

    import torch

    from sparse_mla_decode_03_amd import binding as B
    from sparse_mla_decode_03_amd import workloads as W

    dev = torch.device("cuda")
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "dispatches": 5}))
        return 0

    spec = W.WORKLOADS[args.workload]
    if args.num_splits is not None:
        spec = spec.scaled(num_splits=args.num_splits)
    t_gen = time.perf_counter()
    inp = W.make_inputs(spec, args.seed, device=dev, cache_device=dev)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen
    R, H, K = inp.num_rows, inp.num_heads, spec.topk
    kvf = kv_code(B, spec.kv_format)
    prob = B.make_problem(R, spec.num_requests, H, K, spec.page_size, inp.num_pages,
                          inp.page_table.shape[1], kvf, B.IDX_LOGICAL, spec.num_splits, spec.flags,
                          spec.softmax_scale, spec.kv_scale)
    info = B.plan(prob)
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    ws = (torch.empty(info.workspace_bytes, dtype=torch.uint8, device=dev)
          if info.workspace_bytes else None)
    stream = torch.cuda.current_stream()

    def step():
        B.run(info, inp.q, inp.kv_cache, inp.indices, inp.row_req, inp.page_table, inp.sinks,
              out, lse, None, None, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in evs]

    # Cold-cache launches: the scratch write sits outside each event pair.
    cold_ms = []
    if args.cold_steps > 0:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.cold_steps)]
        for e0, e1 in cevs:
            scratch.fill_(1)
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        cold_ms = sorted(e0.elapsed_time(e1) for e0, e1 in cevs)
        del scratch
    mean_launch_s = sum(launch_ms) / len(launch_ms) / 1e3

    n_valid = inp.num_valid()
    flops = W.algorithmic_flops(inp)
    cbytes = W.compulsory_bytes(inp)
    K_steps = args.steps
    value = n_valid * K_steps / wall
    mfma_tflops = flops / mean_launch_s / 1e12
    hbm_gbs = cbytes / mean_launch_s / 1e9
    traffic = pmc_traffic(1)
    res = {
        "metric": "sparse-MLA decode attended KV entries/s",
        "value": value,
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": wall / K_steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": spec.name, "requests": spec.num_requests, "rows": R, "heads": H,
            "topk": K, "kv_format": {"fp8": "fp8_e4m3+ue8m0", "fp8t": "fp8_e4m3_per_tensor",
                                          "bf16": "bf16"}[spec.kv_format],
            "page_size": spec.page_size, "pages": inp.num_pages, "num_splits": info.num_splits,
            "attended_entries_per_step": n_valid,
            "tokens_per_s": R * K_steps / wall,
            "compulsory_bytes_per_step": cbytes,
            "hbm_tb_s": hbm_gbs / 1e3,
            "hbm_frac": hbm_gbs / PEAK_HBM_GBS,
            "mfma_tflop_s": mfma_tflops,
            "launch_ms_mean": mean_launch_s * 1e3,
            "launch_ms_min": min(launch_ms),
            "launch_ms_p50": sorted(launch_ms)[len(launch_ms) // 2],
            "launch_ms_p90": sorted(launch_ms)[min(len(launch_ms) - 1, (9 * len(launch_ms)) // 10)],
            "launch_ms_p10": sorted(launch_ms)[len(launch_ms) // 10],
            "cold_cache_launch_ms_p50": cold_ms[len(cold_ms) // 2] if cold_ms else None,
            "cold_cache_launch_ms_p10": cold_ms[len(cold_ms) // 10] if cold_ms else None,
            "cold_cache_launch_ms_p90": cold_ms[min(len(cold_ms) - 1, (9 * len(cold_ms)) // 10)] if cold_ms else None,
            "input_generation_s": round(t_gen, 2),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": mfma_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": mfma_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "kernel": "decode_kernel (+merge when split)",
            "flops_per_launch": flops,
        },
    }
    # once-per-step index build: translate once, then decode in GLOBAL mode (per layer)
    slots = B.translate_indices(inp.indices, inp.row_req, inp.page_table, spec.page_size, inp.num_pages,
                                stream=stream)
    gprob = B.make_problem(R, spec.num_requests, H, K, spec.page_size, inp.num_pages,
                           inp.page_table.shape[1], kvf, B.IDX_GLOBAL, spec.num_splits, spec.flags,
                           spec.softmax_scale, spec.kv_scale)
    ginfo = B.plan(gprob)

    def timed_ms(fn, reps=20):
        for _ in range(3):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps

    tr_ms = timed_ms(lambda: B.translate_indices(inp.indices, inp.row_req, inp.page_table, spec.page_size,
                                                 inp.num_pages, out=slots, stream=stream))

    def gstep():
        B.run(ginfo, inp.q, inp.kv_cache, slots, inp.row_req, inp.page_table, inp.sinks,
              out, lse, None, None, ws, stream)

    # GLOBAL and LOGICAL launches alternate, so the clock drift of a long run hits both alike
    pairs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(2)] for _ in range(20)]
    for (g0, g1), (l0, l1) in pairs:
        g0.record(stream)
        gstep()
        g1.record(stream)
        l0.record(stream)
        step()
        l1.record(stream)
    torch.cuda.synchronize()
    g_ms = sum(p[0][0].elapsed_time(p[0][1]) for p in pairs) / len(pairs)
    l_ms = sum(p[1][0].elapsed_time(p[1][1]) for p in pairs) / len(pairs)
    res["index_build"] = {"translate_ms": tr_ms, "decode_global_ms": g_ms, "decode_logical_ms": l_ms,
                          "note": "GLOBAL-mode decode over slots built once per step, alternated "
                                  "with LOGICAL-mode launches over the positions"}
    if args.store_tokens > 0:
        res["cache_store"] = cache_store_measure(B, torch, dev, args.store_tokens, 20)
    if args.mixed:
        res["mixed_prefill_decode"] = decode_measure(B, W, torch, dev, args.mixed, 10, 41)
    if args.fp8_tensor:
        res["per_tensor_fp8"] = decode_measure(B, W, torch, dev, args.fp8_tensor, 20, 43)
    if args.indexer:
        res["indexer"] = indexer_measure(B, W, torch, dev, args.indexer, 20)
    if args.other_workloads:
        res["workloads"] = {}
        for item in args.other_workloads.split(","):
            name, seed = item.split(":")
            res["workloads"][name] = workload_measure(B, W, torch, dev, name, int(seed), 20)
    if args.spike_every > 0 and spec.kv_format == "fp8":
        res["spikes"] = {
            "within_2^64": spike_measure(B, torch, inp, info, out, lse, ws, stream, 48.0, args.spike_every),
            "beyond_2^64": spike_measure(B, torch, inp, info, out, lse, ws, stream, 100.0, args.spike_every),
            "note": "one row in every 64 with one late entry whose head-0 score lies the given "
                    "number of log2 units above the row's typical largest score; spiked and "
                    "plain launches alternated"}
    if not args.no_cpu_baseline:
        step()                                  # out/lse of the plain inputs for the diagnostic
        torch.cuda.synchronize()
        cb = cpu_baseline(inp, out, lse, args.cpu_budget)
        if args.cpu_single:
            name, seed = args.cpu_single.split(":")
            del inp
            torch.cuda.empty_cache()
            cb["single_process"] = cpu_single_process(B, W, torch, dev, name, int(seed))
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
