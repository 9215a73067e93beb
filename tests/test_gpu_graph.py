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
