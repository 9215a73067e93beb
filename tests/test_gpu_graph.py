"""The decode captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI): every replay, with
the program's own eager work and synchronizations between replays, gives the bits of the
eager call.  Cases: unsplit, a positional split with its merge, balanced rows (the two
scheduling launches, per-row split counts and the merge) and index checking (its flag word
is reset by a fill kernel, never by a memset node)."""

from __future__ import annotations

import pytest
import torch

from sparse_mla_decode_03_amd import binding as B
from sparse_mla_decode_03_amd import workloads as W
from tests.gpu_util import announce

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda")

CASES = {
    "unsplit": dict(fmt="fp8", heads=128, topk=512, nreq=8, rows=(4,), splits=1, flags=0, valid="all"),
    "split": dict(fmt="bf16", heads=64, topk=1024, nreq=3, rows=(1,), splits=4, flags=0, valid="all"),
    "balanced": dict(fmt="fp8", heads=64, topk=512, nreq=100, rows=(1, 2, 4), splits=2,
                     flags=B.F_BALANCE_ROWS, valid="uniform"),
    "checked": dict(fmt="fp8", heads=32, topk=256, nreq=4, rows=(2,), splits=2,
                    flags=B.F_CHECK_INDICES, valid="all"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager(name):
    c = CASES[name]
    spec = W.WorkloadSpec("graph", c["nreq"], c["rows"], c["heads"], c["topk"], c["topk"] + 100,
                          3 * c["topk"], c["fmt"], num_splits=c["splits"], valid=c["valid"])
    g = W.make_inputs(spec, 801).to(DEV)
    R, H = g.num_rows, g.num_heads
    kvf = {"fp8": B.KV_FP8_UE8M0, "bf16": B.KV_BF16}[c["fmt"]]
    info = B.plan(B.make_problem(R, c["nreq"], H, c["topk"], spec.page_size, g.num_pages,
                                 g.page_table.shape[1], kvf, B.IDX_LOGICAL, c["splits"], c["flags"],
                                 spec.softmax_scale))
    assert info.num_splits == c["splits"]
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((R, H), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(info.workspace_bytes, 16), dtype=torch.uint8, device=DEV)

    def call():
        B.run(info, g.q, g.kv_cache, g.indices, g.row_req, g.page_table, g.sinks, out, lse, None, None, ws)

    announce(f"graph {name} R={R} H={H} S={info.num_splits}")
    call()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()                                        # a warm-up call off the default stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for i in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xA5)                                # the workspace needs no initial contents
        x = torch.randn(256, 256, device=DEV) @ torch.randn(256, 256, device=DEV)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(x).all()
        assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"{name}: replay {i}"
        assert torch.equal(lse, ref_l), f"{name}: replay {i}"


def test_graph_of_a_whole_step():
    """One decode step as one graph: indexer logits -> top-k -> the once-per-step slot build ->
    decode in GLOBAL mode over those slots.  Every intermediate buffer is scrambled before
    each replay; the lists and the outputs come back bit-identical to the eager step."""
    ispec = W.INDEXER_WORKLOADS["idx_small"].scaled(next_n=2, num_requests=3, ctx_lo=300, ctx_hi=900)
    iinp = W.make_indexer_inputs(ispec, 41)
    dspec = W.WorkloadSpec("step", 3, (2,), 64, 256, 300, 900, W.KV_FP8)
    d = W.make_inputs(dspec, 41).to(DEV)
    assert torch.equal(d.context_lens.cpu(), iinp.context_lens)
    R, H, K = d.num_rows, d.num_heads, 256
    q_codes, weights = iinp.q_codes.to(DEV).contiguous(), iinp.weights.to(DEV).contiguous()
    key_cache, row_len = iinp.key_cache.to(DEV), iinp.row_len.to(DEV).contiguous()
    ipt = iinp.page_table.to(DEV).contiguous()
    logits = torch.empty((R, iinp.width), dtype=torch.float32, device=DEV)
    idx = torch.empty((R, K), dtype=torch.int32, device=DEV)
    slots = torch.empty((R, K), dtype=torch.int32, device=DEV)
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((R, H), dtype=torch.float32, device=DEV)
    info = B.plan(B.make_problem(R, dspec.num_requests, H, K, dspec.page_size, d.num_pages,
                                 d.page_table.shape[1], B.KV_FP8_UE8M0, B.IDX_GLOBAL, 0, 0,
                                 dspec.softmax_scale))
    ws = torch.empty(max(info.workspace_bytes, 16), dtype=torch.uint8, device=DEV)

    def step():
        B.indexer_logits(q_codes, weights, key_cache, row_len, ipt, ispec.next_n, iinp.width, logits=logits)
        B.indexer_topk(logits, row_len, K, out=idx)
        B.translate_indices(idx, d.row_req, d.page_table, dspec.page_size, d.num_pages, out=slots)
        B.run(info, d.q, d.kv_cache, slots, None, None, d.sinks, out, lse, None, None, ws)

    announce(f"graph of a step R={R} S={info.num_splits}")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, slots, out, lse)]
    assert (ref[0] >= 0).any()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        logits.fill_(float("nan"))
        idx.fill_(-5)
        slots.fill_(-5)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want, what in zip((idx, slots, out, lse), ref, ("top-k", "slots", "out", "lse")):
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want), \
                f"{what}: replay {i}"
