"""The allocation-free entry point (sparse_mla_decode_run_noalloc) against sparse_mla_decode_run
on the GPU: split plans (partials in the library's per-GPU scratch), an unsplit one and
balanced rows, two calls in a row with the second smaller, the first call again after the
second, and every result also against the float64 oracle at the usual tolerance."""

from __future__ import annotations

import pytest
import torch

from sparse_mla_decode_03_amd import binding as B
from sparse_mla_decode_03_amd import workloads as W
from tests.gpu_util import announce, compare, oracle_decode

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda")


def _case(fmt, heads, topk, nreq, rows, splits, seed, flags=0):
    spec = W.WorkloadSpec("noalloc", nreq, rows, heads, topk, topk + 100, 3 * topk, fmt,
                          num_splits=splits, valid="uniform")
    inp = W.make_inputs(spec, seed)
    g = inp.to(DEV)
    kvf = {"fp8": B.KV_FP8_UE8M0, "bf16": B.KV_BF16}[fmt]
    prob = B.make_problem(inp.num_rows, nreq, heads, topk, spec.page_size, inp.num_pages,
                          inp.page_table.shape[1], kvf, B.IDX_LOGICAL, splits, flags, spec.softmax_scale)
    info = B.plan(prob)
    return inp, g, info


def _both(inp, g, info):
    R, H = inp.num_rows, inp.num_heads
    out_ws = torch.empty((R, H, 512), dtype=torch.bfloat16, device=DEV)
    lse_ws = torch.empty((R, H), dtype=torch.float32, device=DEV)
    ws = (torch.empty(info.workspace_bytes, dtype=torch.uint8, device=DEV)
          if info.workspace_bytes else None)
    B.run(info, g.q, g.kv_cache, g.indices, g.row_req, g.page_table, g.sinks, out_ws, lse_ws, None,
          None, ws)
    out_na = torch.full((R, H, 512), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse_na = torch.full((R, H), float("nan"), dtype=torch.float32, device=DEV)
    B.run_noalloc(info, g.q, g.kv_cache, g.indices, g.row_req, g.page_table, g.sinks, out_na, lse_na)
    torch.cuda.synchronize()
    return out_ws, lse_ws, out_na, lse_na


def test_noalloc_matches_run_on_two_calls_then_again():
    # first: 12 rows x 4 splits x 128 heads (12.6 MB of partials); second, smaller: 3 rows x 3
    # splits x 32 heads; then the first again (the scratch holds the second call's partials)
    big = _case("fp8", 128, 512, 6, (2,), 4, 701)
    small = _case("bf16", 32, 256, 3, (1,), 3, 702)
    assert big[2].num_splits == 4 and small[2].num_splits == 3
    assert 0 < small[2].workspace_bytes < big[2].workspace_bytes <= B.NOALLOC_SCRATCH_BYTES
    for name, (inp, g, info) in (("first", big), ("second (smaller)", small), ("first again", big)):
        announce(f"noalloc {name} R={inp.num_rows} H={inp.num_heads} S={info.num_splits}")
        out_ws, lse_ws, out_na, lse_na = _both(inp, g, info)
        # the same kernels on the same bytes: identical results
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), name
        assert torch.equal(lse_na, lse_ws), name
        o, l = oracle_decode(inp)
        compare(out_na, lse_na, o, l, what=f"noalloc {name}")


def test_noalloc_unsplit_plan_needs_no_scratch():
    inp, g, info = _case("fp8", 64, 256, 64, (4,), 1, 703)
    assert info.num_splits == 1 and info.workspace_bytes == 0
    announce("noalloc unsplit")
    out_ws, lse_ws, out_na, lse_na = _both(inp, g, info)
    assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16))
    assert torch.equal(lse_na, lse_ws)


def test_noalloc_balanced_rows_two_calls():
    # balanced rows keep their row counts and order in the scratch too (beside the partials of
    # a split plan); the second call is smaller and unsplit
    big = _case("fp8", 64, 512, 20, (1, 2, 4), 2, 704, flags=B.F_BALANCE_ROWS)
    small = _case("bf16", 32, 256, 5, (1,), 1, 705, flags=B.F_BALANCE_ROWS)
    assert big[2].num_splits == 2 and small[2].num_splits == 1
    assert 0 < small[2].workspace_bytes < big[2].workspace_bytes <= B.NOALLOC_SCRATCH_BYTES
    for name, (inp, g, info) in (("balanced first", big), ("balanced second (smaller)", small)):
        announce(f"noalloc {name} R={inp.num_rows} H={inp.num_heads} S={info.num_splits}")
        out_ws, lse_ws, out_na, lse_na = _both(inp, g, info)
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), name
        assert torch.equal(lse_na, lse_ws), name
        o, l = oracle_decode(inp)
        compare(out_na, lse_na, o, l, what=f"noalloc {name}")
