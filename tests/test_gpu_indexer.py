"""GPU parity of the indexer (sparse_mla_indexer_logits / sparse_mla_indexer_topk through
the C ABI) against the indexer oracle.

Logits: every visible position within an error bound derived from the arithmetic (exact
FP8 products, fp32 sums of 128 products per head and 64 weighted heads):
|d| <= 2^-14 * sum_h |w_h| * scale_t * sum_d |q_hd k_td|.
Top-k: integer output, so both sides select from the same fp32 logits (the kernel's) and
must agree exactly, order included (ascending positions)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import indexer_oracle as io
from oracle import sparse_mla_oracle as orc
from sparse_mla_decode_03_amd import binding as B
from sparse_mla_decode_03_amd import workloads as W
from tests.gpu_util import announce, compare, gpu_decode, oracle_decode

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda")


def _magnitude(inp: W.IndexerInputs, rows, cache=None) -> np.ndarray:
    """sum_h |w_h| * scale_t * sum_d |q_hd| |k_td| per (row, visible position)."""
    cache = inp.key_cache.cpu().numpy() if cache is None else cache
    q = inp.q_codes.cpu().numpy()
    w = np.abs(inp.weights.cpu().numpy().astype(np.float64))
    out = []
    for r in rows:
        n = int(inp.row_len[r])
        codes, scale = io.decode_keys(cache, 64, io.row_slots(int(inp.row_req[r]), n,
                                                           inp.page_table.cpu().numpy(), 64))
        m = np.abs(orc.e4m3fn_to_f64(q[r])) @ np.abs(codes).T        # [H, n]
        out.append(scale * (w[r] @ m))
    return out


def _check_logits(inp: W.IndexerInputs, logits: torch.Tensor, rows, what, cache=None):
    got = logits.cpu().numpy()
    cache_np = inp.key_cache.cpu().numpy() if cache is None else cache
    want = io.indexer_logits(inp.q_codes.cpu().numpy(), inp.weights.cpu().numpy(), cache_np, 64,
                             inp.row_req.cpu().numpy(), inp.row_len.cpu().numpy(),
                             inp.page_table.cpu().numpy(), inp.width, rows=rows)
    mags = _magnitude(inp, rows, cache_np)
    worst = 0.0
    for i, r in enumerate(rows):
        n = int(inp.row_len[r])
        d = np.abs(got[r, :n].astype(np.float64) - want[i, :n])
        bound = 2.0 ** -14 * mags[i] + 1e-30
        worst = max(worst, float((d / bound).max()))
        assert np.all(d <= bound), f"{what} row {r}: {int((d > bound).sum())} positions off"
    announce(f"{what}: worst |d| / bound = {worst:.3g}")


def _run(inp: W.IndexerInputs):
    g = lambda t: t.to(DEV).contiguous()  # noqa: E731
    return B.indexer_logits(g(inp.q_codes), g(inp.weights), inp.key_cache.to(DEV), g(inp.row_len),
                            g(inp.page_table), inp.spec.next_n, inp.width)


@pytest.mark.parametrize("next_n", [1, 2, 3, 4])
def test_logits_small(next_n):
    spec = W.INDEXER_WORKLOADS["idx_small"].scaled(next_n=next_n, num_requests=3, ctx_lo=130,
                                                   ctx_hi=2600)
    inp = W.make_indexer_inputs(spec, 10 + next_n)
    announce(f"indexer logits next_n={next_n} lens={inp.row_len.tolist()}")
    logits = _run(inp)
    torch.cuda.synchronize()
    _check_logits(inp, logits, list(range(inp.num_rows)), f"logits next_n={next_n}")


def test_logits_chunk_edges_invalid_pages_and_width_clamp():
    """Contexts across the 32-page chunk boundary and one page short of it; a page id
    outside the pool gives -inf; a row longer than the width is cut at the width."""
    spec = W.INDEXER_WORKLOADS["idx_small"].scaled(next_n=2, num_requests=3, ctx_lo=2047, ctx_hi=2049)
    inp = W.make_indexer_inputs(spec, 21)
    inp.row_len = torch.tensor([2047, 2048, 4100, 4101, 64 * 31 + 1, 64 * 32], dtype=torch.int32)
    pt = torch.full((3, 70), 0, dtype=torch.int32)
    rng = np.random.default_rng(3)
    npages = inp.key_cache.shape[0]
    pt[:] = torch.from_numpy(rng.integers(0, npages, (3, 70)).astype(np.int32))
    pt[1, 40] = -1                                   # positions 2560 .. 2623 of request 1
    pt[1, 41] = npages + 5                           # and 2624 .. 2687
    inp.page_table = pt
    inp.width = 4096                                 # request 1's rows are cut at 4096
    logits = _run(inp)
    torch.cuda.synchronize()
    got = logits.cpu().numpy()
    assert np.all(got[2:4, 2560:2688] == -np.inf)
    # the oracle sees the same invalid pages as -inf positions: compare the rest
    ok_pt = pt.clone()
    ok_pt[1, 40] = 0
    ok_pt[1, 41] = 0
    inp2 = W.IndexerInputs(inp.spec, inp.q_codes, inp.weights, inp.key_cache, inp.row_req,
                           torch.clamp(inp.row_len, max=4096), ok_pt, inp.context_lens, 4096)
    want = io.indexer_logits(inp.q_codes.numpy(), inp.weights.numpy(), inp.key_cache.numpy(), 64,
                             inp.row_req.numpy(), inp2.row_len.numpy(), ok_pt.numpy(), 4096)
    want[2:4, 2560:2688] = -np.inf
    mags = _magnitude(inp2, range(6))
    for r in range(6):
        n = int(inp2.row_len[r])
        fin = np.isfinite(want[r, :n])
        d = np.abs(got[r, :n][fin] - want[r, :n][fin])
        assert np.all(d <= 2.0 ** -14 * mags[r][fin] + 1e-30)


def test_logits_many_requests_empty_rows_and_untouched_tail():
    """More requests than one pass of the workgroup's schedule scan (300 > 256), rows of
    length 0, a request whose rows are all empty between non-empty ones, rows ending inside
    a page, and rows of one request with different lengths.  Every position below a row's
    length matches the oracle; every position at or past it keeps what the buffer held."""
    spec = W.INDEXER_WORKLOADS["idx_small"].scaled(next_n=3, num_requests=300, ctx_lo=1, ctx_hi=400)
    inp = W.make_indexer_inputs(spec, 31)
    rl = inp.row_len.clone()
    rl[0:3] = torch.tensor([0, 5, 0], dtype=torch.int32)           # request 0: mixed
    rl[3 * 150: 3 * 151] = 0                                        # request 150: all empty
    rl[3 * 151: 3 * 152] = torch.tensor([64, 63, 65], dtype=torch.int32)
    rl[-3:] = torch.tensor([1, 0, 129], dtype=torch.int32)          # the last request
    inp.row_len = rl
    g = lambda t: t.to(DEV).contiguous()  # noqa: E731
    sentinel = 12345.5
    buf = torch.full((inp.num_rows, inp.width), sentinel, dtype=torch.float32, device=DEV)
    announce(f"indexer logits: 300 requests x 3 rows, width {inp.width}")
    B.indexer_logits(g(inp.q_codes), g(inp.weights), inp.key_cache.to(DEV), g(inp.row_len),
                     g(inp.page_table), 3, inp.width, logits=buf)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    lens = inp.row_len.numpy()
    for r in range(inp.num_rows):
        assert np.all(got[r, lens[r]:] == sentinel), f"row {r} written past its length {lens[r]}"
    rows = [r for r in range(inp.num_rows) if lens[r] > 0]
    _check_logits(inp, buf, rows, "logits, 300 requests")


def test_logits_full_size_sampled():
    """The index lists of the headline decode workload: 128 requests x 4 rows over 8K..128K
    contexts, in the benchmark's launch configuration; sampled rows checked."""
    spec = W.INDEXER_WORKLOADS["idx_b128_mtp4_h64"]
    inp = W.make_indexer_inputs(spec, 5, device="cpu", cache_device=DEV)
    announce(f"indexer full size R={inp.num_rows} width={inp.width} pages={inp.key_cache.shape[0]}")
    logits = _run(inp)
    torch.cuda.synchronize()
    lens = inp.row_len.numpy()
    longest = int(np.argmax(lens))
    rows = sorted({0, 3, inp.num_rows - 1, longest, int(np.argmin(lens))})
    # the oracle reads only the pages of the sampled rows
    cache = inp.key_cache
    reqs = sorted({int(inp.row_req[r]) for r in rows})
    used = np.unique(np.concatenate([inp.page_table[b].numpy() for b in reqs]))
    used = used[used >= 0]
    remap = np.full(cache.shape[0], -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    sub = cache.index_select(0, torch.from_numpy(used).to(DEV)).cpu().numpy()
    pt = inp.page_table.numpy()
    sub_pt = np.where(pt >= 0, remap[np.maximum(pt, 0)], -1).astype(np.int32)
    inp_sub = W.IndexerInputs(inp.spec, inp.q_codes, inp.weights, torch.from_numpy(sub), inp.row_req,
                              inp.row_len, torch.from_numpy(sub_pt), inp.context_lens, inp.width)
    _check_logits(inp_sub, logits, rows, "logits full size", cache=sub)
    assert torch.isfinite(logits[longest, : int(lens[longest])]).all()


def _topk_case(logits: torch.Tensor, lens: torch.Tensor, topk: int, what: str):
    out = B.indexer_topk(logits.to(DEV), lens.to(DEV), topk)
    torch.cuda.synchronize()
    # the kernel reads min(row_len, width) positions of each row
    n = np.minimum(lens.cpu().numpy(), logits.shape[1])
    want = io.indexer_topk(logits.cpu().numpy().astype(np.float64), n, topk)
    got = out.cpu().numpy()
    assert np.array_equal(got, want), f"{what}: {int((got != want).sum())} entries differ"


def test_topk_edges():
    rng = np.random.default_rng(8)
    width = 5000
    lg = torch.from_numpy(rng.standard_normal((8, width)).astype(np.float32))
    lens = torch.tensor([5000, 4999, 2049, 2048, 2047, 1, 0, 7000], dtype=torch.int32)
    announce("topk edges")
    _topk_case(lg, lens, 2048, "random, lengths around K, empty, past the width")
    # heavy ties: few distinct values, the boundary falls inside a run of equal values
    tied = torch.from_numpy(rng.integers(0, 5, (8, width)).astype(np.float32))
    _topk_case(tied, lens, 2048, "five distinct values")
    allsame = torch.full((2, width), 3.25)
    _topk_case(allsame, torch.tensor([width, 3000], dtype=torch.int32), 2048, "all equal")
    # negative values, -inf entries and mixed signs of zero
    neg = torch.from_numpy(-np.abs(rng.standard_normal((3, width))).astype(np.float32))
    neg[0, ::7] = -float("inf")
    neg[1, ::3] = 0.0
    neg[1, 1::3] = -0.0
    _topk_case(neg, torch.tensor([width, width, 100], dtype=torch.int32), 2048, "negative, -inf, +-0")
    # a first-bin crowd larger than the kernel keeps in LDS (the three-pass route), and one
    # that fits
    big = torch.full((3, 20000), 1.5)
    big[1, ::5] = 2.0
    big[2] = torch.from_numpy(rng.standard_normal(20000).astype(np.float32))
    _topk_case(big, torch.tensor([20000, 20000, 19999], dtype=torch.int32), 2048, "crowded first bin")
    _topk_case(lg, lens, 1, "K = 1")
    _topk_case(lg, lens, 3000, "K = 3000")
    _topk_case(lg, lens, 700, "K = 700")
    _topk_case(tied, lens, 1000, "five distinct values, K = 1000")
    # about 5000 ties in the boundary bin (held in LDS; their ranks are taken over several
    # rounds of the workgroup), with and without distinct larger values above them
    four = torch.from_numpy(rng.integers(0, 4, (2, 20000)).astype(np.float32))
    four[1, ::50] = torch.from_numpy(10.0 + rng.standard_normal(400).astype(np.float32))
    _topk_case(four, torch.tensor([20000, 19999], dtype=torch.int32), 2048, "four values, ties in LDS")
    # K at the kernel's staging capacity (6080 positions staged in LDS) and one past it
    wide = torch.from_numpy(rng.standard_normal((2, 20000)).astype(np.float32))
    wl = torch.tensor([20000, 13000], dtype=torch.int32)
    _topk_case(wide, wl, 6080, "K = 6080")
    _topk_case(wide, wl, 6081, "K = 6081")


def test_topk_sample_misses_and_overflow():
    """The kernel estimates a capture threshold from the first 8192 positions of a row and
    keeps every key above it while it builds the histogram; rows where that estimate fails
    (a sample of larger values than the rest: the K-th largest key lies below the capture
    bin; a sample of smaller values: more keys above it than the list holds) take the route
    that reads the row again, with the same result."""
    rng = np.random.default_rng(21)
    width = 60000
    base = rng.standard_normal((4, width)).astype(np.float32)
    lg = torch.from_numpy(base.copy())
    lg[0, :8192] += 6.0                      # sample far above the rest
    lg[1, 8192:] += 4.0                      # sample far below the rest
    lg[2, 8192:] = torch.from_numpy(np.repeat(rng.standard_normal(13000).astype(np.float32), 4)[: width - 8192])
    lens = torch.tensor([width, width, width, 30000], dtype=torch.int32)
    announce("topk sample misses")
    _topk_case(lg, lens, 2048, "biased samples")
    _topk_case(lg, lens, 9000, "biased samples, K = 9000")


@pytest.mark.parametrize("rows", [300, 700, 1100])
def test_topk_row_order(rows):
    """More rows than compute units: the workgroups order the rows by length and pair long
    with short ones on a CU (up to 1024 rows; beyond, rows keep their order).  Every row's
    output must match, so the order is a bijection: ragged and equal lengths, rows at or
    under K, empty rows."""
    rng = np.random.default_rng(100 + rows)
    width = 16384
    lg = torch.from_numpy(rng.standard_normal((rows, width)).astype(np.float32))
    lens = rng.integers(0, width + 1, rows)
    lens[::7] = 12000                        # runs of equal lengths
    lens[3::11] = 2048
    lens[5::13] = 0
    announce(f"topk row order R={rows}")
    _topk_case(lg, torch.from_numpy(lens.astype(np.int32)), 2048, f"{rows} rows")


def test_topk_full_size():
    """Top-k over the logits of the headline decode workload (128 requests x 4 rows over
    8K..128K contexts, K = 2048) in the benchmark's launch configuration: every row
    against the oracle, on the kernel's own logits."""
    spec = W.INDEXER_WORKLOADS["idx_b128_mtp4_h64"]
    inp = W.make_indexer_inputs(spec, 5, device=DEV, cache_device=DEV)
    announce(f"topk full size R={inp.num_rows} width={inp.width}")
    logits = B.indexer_logits(inp.q_codes, inp.weights, inp.key_cache, inp.row_len, inp.page_table,
                              spec.next_n, inp.width)
    _topk_case(logits, inp.row_len, spec.topk, "full size")


def test_topk_rows_longer_than_the_bitmap():
    """Rows past the kernel's in-LDS position bitmap (131072 positions) take the route that
    keeps the boundary bin's entries in position order and writes the output in a last pass
    over the row; one row just inside the bitmap for comparison, ties included."""
    rng = np.random.default_rng(12)
    width = 140032
    lg = torch.from_numpy(rng.standard_normal((3, width)).astype(np.float32))
    lg[2] = torch.from_numpy(rng.integers(0, 6, width).astype(np.float32))
    lens = torch.tensor([140032, 131072, 139999], dtype=torch.int32)
    announce("topk rows past the bitmap")
    _topk_case(lg, lens, 2048, "rows of 131072 and 140000 positions")


def test_indexer_then_decode():
    """The indexer's lists drive the decode path: logits -> top-k -> decode, compared with
    the decode oracle on the same lists."""
    ispec = W.INDEXER_WORKLOADS["idx_small"].scaled(next_n=2, num_requests=3, ctx_lo=300, ctx_hi=900)
    iinp = W.make_indexer_inputs(ispec, 31)
    logits = _run(iinp)
    idx = B.indexer_topk(logits, iinp.row_len.to(DEV), 256)
    torch.cuda.synchronize()
    want_idx = io.indexer_topk(logits.cpu().numpy().astype(np.float64), iinp.row_len.numpy(), 256)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    # a decode workload over the same requests, pages and rows, reading these lists
    dspec = W.WorkloadSpec("after_indexer", 3, (2,), 64, 256, 300, 900, W.KV_FP8)
    dinp = W.make_inputs(dspec, 31)
    assert np.array_equal(dinp.context_lens.numpy(), iinp.context_lens.numpy())
    dinp.indices = idx.cpu()
    announce("indexer -> decode")
    out, lse = gpu_decode(dinp)
    o, l = oracle_decode(dinp)
    compare(out, lse, o, l, what="indexer -> decode")


@pytest.mark.parametrize("name,full", [("b128_mtp4_h128_fp8", False), ("ragged_b256_h64_fp8", False),
                                       ("b128_mtp4_h128_fp8", True)])
def test_global_index_build_then_global_decode(name, full):
    """sparse_mla_translate_indices against the oracle's block-table translation (exact),
    masked entries as -1; then the decode in GLOBAL mode over the built slots gives the
    same bits as the decode in LOGICAL mode over the positions."""
    spec = W.WORKLOADS[name]
    if not full:
        spec = spec.scaled(num_requests=8 if name.startswith("ragged") else 3, ctx_hi=20000)
    inp = W.make_inputs(spec, 51, device="cpu", cache_device=DEV if full else None)
    idx = inp.indices.clone()
    # plant entries the decode path masks: below -1, past the table, a request's page id
    # outside the pool (a copy of the table is used for that)
    idx[0, 5] = -7
    idx[1, 9] = inp.page_table.shape[1] * spec.page_size + 3
    pt = inp.page_table.clone()
    b1 = int(inp.row_req[min(2, inp.num_rows - 1)])
    pt[b1, 0] = inp.num_pages + 11
    announce(f"index build {name} full={full} R={inp.num_rows}")
    slots = B.translate_indices(idx.to(DEV), inp.row_req.to(DEV), pt.to(DEV), spec.page_size, inp.num_pages)
    torch.cuda.synchronize()
    got = slots.cpu().numpy()
    ptn, rr = pt.numpy(), inp.row_req.numpy()
    for r in range(inp.num_rows):
        row = idx[r].numpy()
        bad = (row < 0) | (row // spec.page_size >= ptn.shape[1])
        page = np.where(bad, 0, ptn[rr[r], np.where(bad, 0, row // spec.page_size)])
        bad |= (page < 0) | (page >= inp.num_pages)
        keep = np.where(~bad)[0]
        # the raw row, bad entries included: the oracle masks them itself
        pos, want = orc.translate(row, orc.IDX_LOGICAL, int(rr[r]), ptn, spec.page_size, inp.num_pages)
        assert np.array_equal(pos, keep)
        assert np.array_equal(got[r, keep], want) and np.all(got[r, bad] == -1)
    # the same decode, LOGICAL over positions vs GLOBAL over the built slots
    out_l, lse_l = gpu_decode(inp, indices=idx, page_table=pt)
    out_g, lse_g = gpu_decode(inp, indices=slots.cpu(), index_mode=B.IDX_GLOBAL, page_table=pt)
    torch.cuda.synchronize()
    assert torch.equal(out_l.view(torch.int16), out_g.view(torch.int16))
    assert torch.equal(lse_l, lse_g)
