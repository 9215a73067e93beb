"""Helpers shared by the GPU tests: run the HIP path on workload inputs, run the oracle
on the same bytes, and compare at the stated tolerances."""

from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import sparse_mla_oracle as orc
from sparse_mla_decode_03_amd import binding as B
from sparse_mla_decode_03_amd import workloads as W

# Tolerances of the decode output against the float64 oracle (bf16 output, fp32 LSE).
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LSE_REL = 1e-3

KV = {"bf16": orc.KV_BF16, "fp8": orc.KV_FP8_UE8M0, "fp8t": orc.KV_FP8_TENSOR}


def announce(msg: str) -> None:
    sys.__stdout__.write(f"\n[gpu] {msg}\n")
    sys.__stdout__.flush()


def q_bits(q: torch.Tensor) -> np.ndarray:
    return q.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_decode(inp: W.Inputs, num_splits=None, flags=None, index_mode=B.IDX_LOGICAL, indices=None,
               sinks="same", page_table=None, kv_cache=None, return_info=False):
    dev = torch.device("cuda")
    g = lambda t: None if t is None else t.to(dev).contiguous()  # noqa: E731
    s = inp.sinks if isinstance(sinks, str) else sinks
    return B.sparse_mla_decode(
        g(inp.q), g(inp.kv_cache if kv_cache is None else kv_cache),
        g(inp.indices if indices is None else indices), g(inp.row_req),
        g(inp.page_table if page_table is None else page_table), g(s), inp.spec.kv_format,
        inp.spec.page_size, inp.spec.softmax_scale, index_mode=index_mode,
        num_splits=inp.spec.num_splits if num_splits is None else num_splits,
        flags=inp.spec.flags if flags is None else flags,
        return_info=return_info, kv_scale=inp.spec.kv_scale)


def oracle_decode(inp: W.Inputs, rows=None, indices=None, sinks="same", index_mode=orc.IDX_LOGICAL,
                  page_table=None, kv_cache=None):
    s = inp.sinks if isinstance(sinks, str) else sinks
    cache = inp.kv_cache if kv_cache is None else kv_cache
    return orc.sparse_mla_decode(
        q_bits(inp.q), cache.cpu().numpy(), KV[inp.spec.kv_format], inp.spec.page_size,
        (inp.indices if indices is None else indices).cpu().numpy(), inp.row_req.cpu().numpy(),
        (inp.page_table if page_table is None else page_table).cpu().numpy(),
        None if s is None else s.cpu().numpy(), inp.spec.softmax_scale, index_mode=index_mode,
        rows=rows, kv_scale=inp.spec.kv_scale)


def compare(out: torch.Tensor, lse: torch.Tensor, o_ref: np.ndarray, l_ref: np.ndarray,
            max_abs=MAX_ABS, mean_abs=MEAN_ABS, lse_rel=LSE_REL, what="") -> dict:
    o = out.float().cpu().double().numpy()
    d = np.abs(o - o_ref)
    stats = {"max_abs": float(d.max()) if d.size else 0.0,
             "mean_abs": float(d.mean()) if d.size else 0.0}
    l = lse.cpu().double().numpy()
    inf_g, inf_r = np.isneginf(l), np.isneginf(l_ref)
    assert np.array_equal(inf_g, inf_r), f"{what}: -inf LSE pattern differs"
    fin = ~inf_r
    rel = np.abs(l[fin] - l_ref[fin]) / np.maximum(1.0, np.abs(l_ref[fin]))
    stats["lse_rel"] = float(rel.max()) if rel.size else 0.0
    announce(f"{what} {stats}")
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    assert stats["max_abs"] <= max_abs, f"{what}: max|d| {stats['max_abs']} > {max_abs}"
    assert stats["mean_abs"] <= mean_abs, f"{what}: mean|d| {stats['mean_abs']} > {mean_abs}"
    assert stats["lse_rel"] <= lse_rel, f"{what}: lse rel {stats['lse_rel']} > {lse_rel}"
    return stats


def page_subset(inp: W.Inputs, rows):
    """Cache pages reachable from `rows`, copied to the host, with a remapped page table:
    lets the oracle read a few rows of a multi-GB cache."""
    rr = inp.row_req.cpu()
    reqs = torch.unique(rr[torch.as_tensor(list(rows))])
    pt = inp.page_table.cpu()
    used = pt[reqs]
    used = torch.unique(used[used >= 0])
    remap = torch.full((inp.num_pages,), -1, dtype=torch.int32)
    remap[used.long()] = torch.arange(used.numel(), dtype=torch.int32)
    sub_cache = inp.kv_cache.index_select(0, used.to(inp.kv_cache.device).long()).cpu()
    new_pt = torch.where(pt >= 0, remap[pt.clamp(min=0).long()], torch.full_like(pt, -1))
    return sub_cache, new_pt
