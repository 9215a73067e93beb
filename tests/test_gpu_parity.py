"""GPU parity: the HIP path through the C ABI against the float64 oracle on the same
seeded inputs.  Tolerances: max|d| <= 2e-2, mean|d| <= 2e-3 on the bf16 output, LSE
within 1e-3 relative; integer/byte work (the gather) bit-exact."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import sparse_mla_oracle as orc
from sparse_mla_decode_03_amd import binding as B
from sparse_mla_decode_03_amd import workloads as W
from tests.golden_io import fp8_page_fixture
from tests.gpu_util import (KV, announce, compare, gpu_decode, oracle_decode, page_subset, q_bits)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda")

# Reduced versions of the five workloads: same heads, top-k, format and structure, fewer
# requests so the oracle checks every output element.
REDUCED = {
    "tiny_bf16": W.WORKLOADS["tiny_bf16"],
    "b32_h64_fp8": W.WORKLOADS["b32_h64_fp8"].scaled(num_requests=4, ctx_hi=8192),
    "b128_mtp4_h128_fp8": W.WORKLOADS["b128_mtp4_h128_fp8"].scaled(num_requests=2, ctx_hi=16384),
    "b2_h128_bf16_split16": W.WORKLOADS["b2_h128_bf16_split16"],
    "ragged_b256_h64_fp8": W.WORKLOADS["ragged_b256_h64_fp8"].scaled(num_requests=16),
}


def _small(fmt="fp8", heads=64, topk=256, nreq=3, rows=(1, 2), ctx=(300, 900), ps=64,
           sinks="normal", valid="all", seed=101, kv_scale=1.0):
    spec = W.WorkloadSpec("small", nreq, rows, heads, topk, ctx[0], ctx[1], fmt, page_size=ps,
                          valid=valid, sinks=sinks, kv_scale=kv_scale)
    return W.make_inputs(spec, seed)


# ------------------------------------------------------------------ gather (bit-exact)

def _bf16_bits_exact(vals: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(vals).to(torch.bfloat16)
    assert np.array_equal(t.double().numpy(), vals), "value not representable in bf16"
    return t.view(torch.int16).numpy()


def test_gather_fixture_page_bit_exact():
    page, ps, expects = fp8_page_fixture()
    cache = torch.frombuffer(bytearray(page), dtype=torch.uint8).reshape(1, -1).to(DEV)
    announce("gather_debug fixture page")
    got = B.gather_debug(cache, "fp8", ps, torch.tensor([0, 1], dtype=torch.int32, device=DEV))
    got = got.cpu().double().numpy()
    for slot, lo, hi, val in expects:
        assert np.all(got[slot, lo:hi] == val), (slot, lo, hi)


def test_gather_all_codes_and_scales_bit_exact():
    """Every finite e4m3fn code under scale bytes 10..246 dequantizes exactly."""
    ps, npg = 4, 32
    rng = np.random.default_rng(7)
    pages = np.zeros((npg, 648 * ps), dtype=np.uint8)
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    for p in range(npg):
        lat = np.stack([np.roll(np.tile(codes, 2), 37 * (p * ps + r)) for r in range(ps)])
        pages[p, : 512 * ps] = lat.reshape(-1)
        pages[p, 512 * ps: 640 * ps] = rng.integers(0, 256, size=128 * ps).astype(np.uint8)
        rope = pages[p, 512 * ps: 640 * ps].view(np.uint16)
        rope[(rope & 0x7F80) == 0x7F80] = 0x3F80      # no inf/NaN rope values
        pages[p, 640 * ps:] = rng.integers(10, 247, size=8 * ps).astype(np.uint8)
    slots = np.arange(npg * ps, dtype=np.int32)
    ref = orc.decode_entries(pages, orc.KV_FP8_UE8M0, ps, slots)
    want = _bf16_bits_exact(ref)
    announce("gather_debug all codes")
    got = B.gather_debug(torch.from_numpy(pages).to(DEV), "fp8", ps,
                         torch.from_numpy(slots).to(DEV)).cpu().view(torch.int16).numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} mismatches, first at {bad[0][0]},{bad[1][0]}"


def test_gather_per_tensor_fp8_all_codes_bit_exact():
    """Per-tensor FP8: every finite e4m3fn code at every one of the 576 dims comes back as
    its own value (the tensor scale is applied by the decode as two scalar factors)."""
    ps, npg = 8, 16
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    ent = np.stack([np.roll(np.tile(codes, 3)[:576], 41 * s) for s in range(npg * ps)])
    pages = ent.reshape(npg, 576 * ps)
    slots = np.arange(npg * ps, dtype=np.int32)
    want = _bf16_bits_exact(orc.decode_entries(pages, orc.KV_FP8_TENSOR, ps, slots))
    announce("gather_debug per-tensor fp8 all codes")
    got = B.gather_debug(torch.from_numpy(pages).to(DEV), "fp8t", ps,
                         torch.from_numpy(slots).to(DEV)).cpu().view(torch.int16).numpy()
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"{bad[0].size} mismatches, first at {bad[0][0]},{bad[1][0]}"


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp8t"])
def test_gather_random_slots_bit_exact(fmt):
    inp = _small(fmt=fmt, ctx=(500, 700), ps=16)
    n = inp.num_pages * 16
    slots = np.random.default_rng(3).integers(-3, n + 3, size=999).astype(np.int32)
    ref = orc.decode_entries(inp.kv_cache.numpy(), KV[fmt], 16, np.clip(slots, 0, n - 1))
    ref[(slots < 0) | (slots >= n)] = 0.0
    want = _bf16_bits_exact(ref)
    announce(f"gather_debug random slots {fmt}")
    got = B.gather_debug(inp.kv_cache.to(DEV), fmt, 16, torch.from_numpy(slots).to(DEV))
    assert np.array_equal(got.cpu().view(torch.int16).numpy(), want)


# ------------------------------------------------------------------ parity per workload

@pytest.mark.parametrize("name", W.WORKLOAD_ORDER)
def test_parity_reduced_workloads(name):
    seed = W.WORKLOAD_ORDER.index(name) + 1
    inp = W.make_inputs(REDUCED[name], seed)
    announce(f"parity {name} R={inp.num_rows} H={inp.num_heads} K={inp.spec.topk} seed={seed}")
    out, lse = gpu_decode(inp)
    o, l = oracle_decode(inp)
    compare(out, lse, o, l, what=name)


@pytest.mark.parametrize("name,nrows", [("b32_h64_fp8", None), ("b128_mtp4_h128_fp8", 6),
                                        ("b2_h128_bf16_split16", None),
                                        ("ragged_b256_h64_fp8", 24)])
def test_parity_full_size_sampled(name, nrows):
    """Full-size workload in the benchmark's launch configuration; the oracle checks all
    rows (few-row workloads) or a sample, and every output is checked for finiteness."""
    seed = W.WORKLOAD_ORDER.index(name) + 1
    inp = W.make_inputs(W.WORKLOADS[name], seed, device="cpu", cache_device=DEV)
    announce(f"full {name} R={inp.num_rows} pages={inp.num_pages}")
    out, lse = gpu_decode(inp)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    R = inp.num_rows
    if nrows is None:
        rows = list(range(R))
    else:
        rng = np.random.default_rng(seed)
        rows = sorted({0, R - 1, *rng.choice(R, size=nrows - 2, replace=False).tolist()})
    sub_cache, sub_pt = page_subset(inp, rows)
    o, l = oracle_decode(inp, rows=rows, kv_cache=sub_cache, page_table=sub_pt)
    compare(out[rows], lse[rows], o, l, what=f"{name} rows={len(rows)}")
    if inp.sinks is not None and torch.isneginf(inp.sinks).any():
        # heads without a sink and rows with valid entries have finite LSE
        assert torch.isfinite(lse).all()


# ------------------------------------------------------------------ invariants

def test_invariants_order_mask_sink_relocation_global():
    inp = _small(heads=32, topk=192, nreq=3, rows=(2,), seed=5)
    announce("invariants base")
    out0, lse0 = gpu_decode(inp)
    o, l = oracle_decode(inp)
    compare(out0, lse0, o, l, what="base")
    R, K = inp.indices.shape
    rng = np.random.default_rng(1)
    # permuted order + -1 inserted anywhere (list twice as long)
    wide = torch.full((R, 2 * K), -1, dtype=torch.int32)
    for r in range(R):
        pos = np.sort(rng.choice(2 * K, size=K, replace=False))
        wide[r, pos] = inp.indices[r, rng.permutation(K)]
    out1, lse1 = gpu_decode(inp, indices=wide)
    compare(out1, lse1, o, l, what="permuted+masked")
    d = (out1.float() - out0.float()).abs()
    assert d.max().item() <= 8e-3
    # sink = -inf is the same computation as no sink
    neg = torch.full_like(inp.sinks, -float("inf"))
    out2, lse2 = gpu_decode(inp, sinks=neg)
    out3, lse3 = gpu_decode(inp, sinks=None)
    assert torch.equal(out2, out3) and torch.equal(lse2, lse3)
    # relocated pages: identical bits
    perm = torch.from_numpy(rng.permutation(inp.num_pages)).long()
    cache2 = torch.empty_like(inp.kv_cache)
    cache2[perm] = inp.kv_cache
    pt = inp.page_table
    pt2 = torch.where(pt >= 0, perm[pt.clamp(min=0).long()].int(), pt)
    out4, lse4 = gpu_decode(inp, kv_cache=cache2, page_table=pt2)
    assert torch.equal(out4, out0) and torch.equal(lse4, lse0)
    # GLOBAL mode with pre-translated slots: identical bits
    ps = inp.spec.page_size
    idx = inp.indices
    valid = idx >= 0
    req = inp.row_req.long()[:, None].expand_as(idx)
    slots = pt[req, (idx.clamp(min=0) // ps).long()] * ps + idx.clamp(min=0) % ps
    gidx = torch.where(valid, slots, torch.full_like(idx, -1)).int()
    out5, lse5 = gpu_decode(inp, indices=gidx, index_mode=B.IDX_GLOBAL)
    assert torch.equal(out5, out0) and torch.equal(lse5, lse0)


@pytest.mark.parametrize("splits", [1, 2, 3, 16, 64])
def test_forced_splits_match_unsplit(splits):
    inp = _small(heads=64, topk=256, nreq=2, rows=(1,), valid="uniform", seed=17)
    idx = inp.indices.clone()
    idx[0, :70] = -1                      # empty leading chunks for large S
    o, l = oracle_decode(inp, indices=idx)
    announce(f"forced splits {splits}")
    out, lse = gpu_decode(inp, indices=idx, num_splits=splits)
    compare(out, lse, o, l, what=f"S={splits}")


@pytest.mark.parametrize("heads,splits", [(48, 24), (16, 9), (128, 17)])
def test_forced_splits_over_few_rows(heads, splits):
    # few rows and more than eight splits: the merge of half blocks (padded head groups, a
    # partial second batch of sixteen splits, empty leading chunks)
    inp = _small(heads=heads, topk=1024, nreq=2, rows=(1,), ctx=(1100, 3000), seed=19 + heads)
    idx = inp.indices.clone()
    idx[1, :200] = -1
    o, l = oracle_decode(inp, indices=idx)
    announce(f"few rows H={heads} S={splits}")
    out, lse = gpu_decode(inp, indices=idx, num_splits=splits)
    compare(out, lse, o, l, what=f"few rows H={heads} S={splits}")


@pytest.mark.parametrize("splits", [None, 3])
def test_topk_above_one_workgroup_capacity(splits):
    """K = 5000 exceeds the 2048 positions one workgroup takes: the planner must split (at
    least three chunks, the last one ragged), and the merged result matches the oracle."""
    inp = _small(heads=64, topk=5000, nreq=2, rows=(1,), ctx=(6000, 9000), seed=29)
    idx = inp.indices.clone()
    idx[1, :300] = -1                     # a partly empty first chunk
    o, l = oracle_decode(inp, indices=idx)
    announce(f"K=5000 splits={splits}")
    out, lse, info, _ = gpu_decode(inp, indices=idx, num_splits=0 if splits is None else splits,
                                   return_info=True)
    assert info.num_splits >= 3
    compare(out, lse, o, l, what=f"K=5000 S={info.num_splits}")


@pytest.mark.parametrize("splits", [2, 5, 16])
def test_partials_only_match_oracle_partials(splits):
    inp = _small(heads=32, topk=128, nreq=2, rows=(2,), seed=23)
    announce(f"partials only S={splits}")
    po, pl = gpu_decode(inp, num_splits=splits, flags=B.F_PARTIALS_ONLY)
    oc, lc = orc.sparse_mla_decode_partials(
        q_bits(inp.q), inp.kv_cache.numpy(), KV["fp8"], 64, inp.indices.numpy(),
        inp.row_req.numpy(), inp.page_table.numpy(), inp.spec.softmax_scale, splits)
    d = np.abs(po.cpu().double().numpy() - oc)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    pg = pl.cpu().double().numpy()
    assert np.array_equal(np.isneginf(pg), np.isneginf(lc))
    f = ~np.isneginf(lc)
    assert np.all(np.abs(pg[f] - lc[f]) <= 1e-3 * np.maximum(1, np.abs(lc[f])))


# S = 7 and 8: a partial and a whole batch of eight chunks loaded together; 65, 129 and 256
# (the plan's maximum): more chunk LSEs than lanes, held two, three and four per lane
@pytest.mark.parametrize("R,S,H", [(5, 7, 40), (3, 8, 32), (3, 65, 16), (2, 129, 16), (2, 256, 16)])
def test_merge_kernel_matches_oracle_merge(R, S, H):
    rng = np.random.default_rng(2 + S)
    oc = rng.standard_normal((R, S, H, 512))
    lc = rng.standard_normal((R, S, H)) * 3
    lc[rng.random((R, S, H)) < 0.3] = -np.inf
    lc[0, :, 0] = -np.inf                                 # an all-empty (row, head)
    sinks = rng.standard_normal(H).astype(np.float32)
    sinks[:H // 4] = -np.inf
    o, l = orc.merge_partials(oc.astype(np.float32).astype(np.float64),
                              lc.astype(np.float32).astype(np.float64), sinks)
    announce(f"merge kernel R={R} S={S} H={H}")
    out, lse = B.merge_partials(torch.from_numpy(oc).float().to(DEV),
                                torch.from_numpy(lc).float().to(DEV),
                                torch.from_numpy(sinks).to(DEV))
    # N(0,1) partial rows merge to outputs of a few units, so the output's bf16 rounding (half
    # an ulp: 2^-8 of the value at most) dominates; fp32 accumulation adds far less than 1e-5
    compare(out, lse, o, l, max_abs=0.05, mean_abs=1e-3, lse_rel=1e-5, what="merge")
    d = np.abs(out.float().cpu().double().numpy() - o)
    assert np.all(d <= np.abs(o) * 2.0 ** -8 + 1e-5), "merge: beyond one bf16 rounding of the oracle"


# At least 128 (row, group of 32 heads) pairs: the merge of the decode's own split format
# stages its bf16 results through LDS (four-wave workgroups); 16 and 48 heads pad the last
# group.  Valid prefixes of 1..K entries leave the later chunks of short rows empty (their
# runs are neither written nor read), and one row is empty altogether.
@pytest.mark.parametrize("heads,splits", [(16, 2), (48, 3), (64, 5), (64, 2)])
def test_merge_of_many_rows_with_empty_chunks(heads, splits):
    inp = _small(heads=heads, topk=128, nreq=140, rows=(1,), ctx=(200, 600), valid="uniform",
                 seed=41 + heads + splits)
    assert inp.num_rows * ((heads + 31) // 32) >= 128
    idx = inp.indices.clone()
    idx[3] = -1
    o, l = oracle_decode(inp, indices=idx)
    announce(f"merge of many rows H={heads} S={splits}")
    out, lse = gpu_decode(inp, indices=idx, num_splits=splits)
    compare(out, lse, o, l, what=f"many rows H={heads} S={splits}")
    assert torch.all(out[3] == 0) and torch.equal(lse[3].cpu(), inp.sinks)


# Balanced rows: the rows are counted and ordered on the device, and a split row's chunks
# take equal numbers of its entries.  Ragged valid prefixes, an empty row, a row whose first
# half is -1, and out-of-range indices (not counted: the count applies the translation's own
# test, so the shares partition exactly the entries the decode keeps).
@pytest.mark.parametrize("heads,splits", [(64, 1), (64, 2), (128, 3), (16, 5)])
def test_balanced_rows_match_oracle(heads, splits):
    inp = _small(heads=heads, topk=256, nreq=140, rows=(1,), ctx=(200, 600), valid="uniform",
                 seed=61 + heads + splits)
    idx = inp.indices.clone()
    idx[5] = -1
    idx[6, :128] = -1
    ctx = inp.context_lens.long()
    rng = np.random.default_rng(3)
    for r in rng.choice(inp.num_rows, size=20, replace=False):
        n = int((idx[r] >= 0).sum())
        if n > 2:
            pos = rng.choice(n, size=min(3, n), replace=False)
            idx[r, pos] = int(inp.page_table.shape[1]) * inp.spec.page_size + 7 + int(ctx[r])
    o, l = oracle_decode(inp, indices=idx)
    announce(f"balanced rows H={heads} S={splits}")
    out, lse, info, _ = gpu_decode(inp, indices=idx, num_splits=splits, flags=B.F_BALANCE_ROWS,
                                   return_info=True)
    assert info.num_splits == splits
    compare(out, lse, o, l, what=f"balanced H={heads} S={splits}")
    assert torch.all(out[5] == 0) and torch.equal(lse[5].cpu(), inp.sinks)
    # the same attention as the positional split
    out2, lse2 = gpu_decode(inp, indices=idx, num_splits=splits)
    assert (out.float() - out2.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("fmt,heads,splits", [("bf16", 64, 2), ("fp8t", 64, 2), ("fp8t", 128, 3),
                                               ("bf16", 32, 1)])
def test_balanced_rows_other_formats(fmt, heads, splits):
    # the balanced kernels of the BF16 and per-tensor FP8 caches, one- and two-split rows
    inp = _small(fmt=fmt, heads=heads, topk=256, nreq=150, rows=(1,), ctx=(200, 600), valid="uniform",
                 seed=81 + heads + splits, kv_scale=1.0 / 32 if fmt == "fp8t" else 1.0)
    o, l = oracle_decode(inp)
    announce(f"balanced rows {fmt} H={heads} S={splits}")
    out, lse = gpu_decode(inp, num_splits=splits, flags=B.F_BALANCE_ROWS)
    compare(out, lse, o, l, what=f"balanced {fmt} H={heads} S={splits}")


def test_balanced_schedule_lists():
    """The scheduling launch's own lists, read back from the workspace: each row's count is
    the number of entries the oracle's translation keeps; each row's split count follows the
    rule (tiles over a target of three quarters of an even share of the slots' work, at
    least 4 tiles; at most S; at least what keeps a chunk within 2048 entries); the jobs are
    exactly the (row, split) pairs, longest first by tiles (1024 classes)."""
    inp = _small(heads=64, topk=512, nreq=300, rows=(1,), ctx=(300, 1500), valid="uniform", seed=71)
    idx = inp.indices.clone()
    idx[4] = -1
    idx[7, :20] = int(inp.page_table.shape[1]) * inp.spec.page_size + 1   # past the table
    announce("balanced schedule lists")
    S = 2
    out, lse, info, ws = gpu_decode(inp, indices=idx, num_splits=S, flags=B.F_BALANCE_ROWS,
                                    return_info=True)
    torch.cuda.synchronize()
    R, H, K = inp.num_rows, inp.num_heads, inp.spec.topk
    rup = lambda x: (x + 255) // 256 * 256  # noqa: E731
    parts = rup(R * S * ((H + 31) // 32) * 32 * 512 * 4) + rup(R * S * H * 8)
    w = ws.cpu().numpy()[parts:].view(np.int32)
    counts, splits, jobs, njobs = w[:R], w[R:2 * R], w[2 * R:2 * R + R * S], int(w[2 * R + R * S])
    pt, rr = inp.page_table.numpy(), inp.row_req.numpy()
    want = np.array([len(orc.translate(idx[r].numpy(), orc.IDX_LOGICAL, int(rr[r]), pt,
                                       inp.spec.page_size, inp.num_pages)[0]) for r in range(R)])
    assert np.array_equal(counts, want)
    tiles = (want + 31) // 32
    slots = 2 * torch.cuda.get_device_properties(0).multi_processor_count   # two-wave workgroups
    target = max(-(-3 * int(tiles.sum()) // (4 * slots)), 4)
    rule = np.minimum(S, np.maximum(-(-want // 2048), np.maximum(1, -(-tiles // target))))
    assert np.array_equal(splits, rule) and 1 < rule.max()
    assert njobs == int(rule.sum())
    got = [(int(j) & 0xFFFFFF, int(np.uint32(j)) >> 24) for j in jobs[:njobs]]
    assert sorted(got) == sorted((r, s) for r in range(R) for s in range(int(rule[r])))
    share = lambda n, sr, s: (s + 1) * n // sr - s * n // sr  # noqa: E731
    cls = [min((share(int(want[r]), int(rule[r]), s) + 31) // 32, 1023) for r, s in got]
    assert all(a >= b for a, b in zip(cls, cls[1:])), "jobs not longest first"
    o, l = oracle_decode(inp, indices=idx)
    compare(out, lse, o, l, what="balanced schedule")


def test_balanced_rows_above_one_workgroup_and_global_slots():
    # K = 5000 needs at least three splits; GLOBAL mode takes the slots as they are
    inp = _small(heads=64, topk=5000, nreq=3, rows=(1, 2), ctx=(6000, 9000), valid="uniform", seed=67)
    idx = inp.indices.clone()
    idx[0, :2600] = -1
    o, l = oracle_decode(inp, indices=idx)
    announce("balanced rows K=5000")
    out, lse, info, _ = gpu_decode(inp, indices=idx, num_splits=0, flags=B.F_BALANCE_ROWS,
                                   return_info=True)
    assert info.num_splits >= 3
    compare(out, lse, o, l, what="balanced K=5000")
    ps = inp.spec.page_size
    pt = inp.page_table.long()
    valid = idx >= 0
    req = inp.row_req.long()[:, None].expand_as(idx)
    slots = pt[req, (idx.clamp(min=0) // ps).long()] * ps + idx.clamp(min=0) % ps
    gidx = torch.where(valid, slots, torch.full_like(idx, -1)).int()
    out_g, lse_g = gpu_decode(inp, indices=gidx, index_mode=B.IDX_GLOBAL, num_splits=0,
                              flags=B.F_BALANCE_ROWS)
    assert torch.equal(out_g, out) and torch.equal(lse_g, lse)


# ------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("splits", [0, 1, 2, 3])
def test_empty_rows_and_zero_rows(splits):
    # an empty row gives out = 0 and LSE = the sink exactly, unsplit and through the merge
    inp = _small(heads=16, topk=64, nreq=3, rows=(1,), seed=31)
    idx = inp.indices.clone()
    idx[1] = -1
    announce(f"empty row, splits {splits}")
    out, lse = gpu_decode(inp, indices=idx, num_splits=splits)
    o, l = oracle_decode(inp, indices=idx)
    compare(out, lse, o, l, what="empty row")
    assert torch.all(out[1] == 0)
    assert torch.equal(lse[1].cpu(), inp.sinks)
    out, lse = gpu_decode(inp, indices=idx, sinks=None, num_splits=splits)
    assert torch.all(out[1] == 0) and torch.isneginf(lse[1]).all()
    # zero rows: nothing launched, empty results
    z = W.Inputs(inp.spec, inp.q[:0], inp.kv_cache, inp.indices[:0], inp.row_req[:0],
                 inp.page_table, inp.sinks, inp.context_lens)
    out, lse = gpu_decode(z)
    assert out.shape == (0, 16, 512) and lse.shape == (0, 16)


@pytest.mark.parametrize("heads", [16, 32, 48, 80, 96, 112, 128])
def test_head_counts(heads):
    inp = _small(heads=heads, topk=96, nreq=2, rows=(1,), seed=40 + heads)
    announce(f"heads {heads}")
    out, lse = gpu_decode(inp)
    o, l = oracle_decode(inp)
    compare(out, lse, o, l, what=f"H={heads}")


@pytest.mark.parametrize("fmt,ps", [("bf16", 1), ("fp8", 2), ("fp8", 16), ("bf16", 256)])
def test_page_sizes(fmt, ps):
    inp = _small(fmt=fmt, heads=16, topk=100, nreq=2, rows=(1,), ctx=(600, 1000), ps=ps,
                 seed=50 + ps)
    announce(f"page size {ps}")
    out, lse = gpu_decode(inp)
    o, l = oracle_decode(inp)
    compare(out, lse, o, l, what=f"ps={ps}")


def test_index_check_records_first_bad_and_masks_it():
    inp = _small(heads=16, topk=64, nreq=4, rows=(1,), seed=61)
    idx = inp.indices.clone()
    idx[2, 5] = 10 ** 6          # beyond the page table
    idx[3, 1] = -7               # negative, not -1
    idx[2, 9] = 10 ** 6 + 1
    announce("index check")
    out, lse, info, ws = gpu_decode(inp, indices=idx, flags=B.F_CHECK_INDICES, return_info=True)
    assert B.read_index_error(info, ws) == (2, 5)
    # the oracle masks the same entries (raw indices on both sides)
    o, l = oracle_decode(inp, indices=idx)
    compare(out, lse, o, l, what="masked bad indices")
    out2, lse2, info2, ws2 = gpu_decode(inp, flags=B.F_CHECK_INDICES, return_info=True)
    assert B.read_index_error(info2, ws2) == (-1, -1)


# ------------------------------------------------------------------ sensitivity

@pytest.mark.parametrize("topk,sink", [(4, 5.0), (16, 2.0), (64, 0.0), (128, -1.0)])
def test_small_topk_with_strong_sinks(topk, sink):
    """At small K a dropped entry or an ignored sink moves the output by far more than the
    tolerance; here the bound is tighter still."""
    inp = _small(heads=32, topk=topk, nreq=3, rows=(1, 2), ctx=(200, 400), seed=70 + topk)
    sinks = torch.full((32,), sink, dtype=torch.float32)
    sinks[::3] = -float("inf")
    announce(f"sensitivity K={topk} sink={sink}")
    out, lse = gpu_decode(inp, sinks=sinks)
    o, l = oracle_decode(inp, sinks=sinks)
    compare(out, lse, o, l, max_abs=1e-2, mean_abs=1e-3, what=f"K={topk}")
    if topk <= 16:
        # dropping one entry is visible at this bound
        idx = inp.indices.clone()
        idx[0, 0] = -1
        od, _ = oracle_decode(inp, sinks=sinks, indices=idx)
        assert np.abs(od[0] - o[0]).max() > 2e-2


# 128 heads: four waves, whose last O block is accumulated in VGPRs and zeroed again for the
# repeated pass
@pytest.mark.parametrize("fmt,alpha,heads", [("fp8", 20.0, 32), ("fp8", 40.0, 32), ("bf16", 40.0, 32),
                                             ("fp8", 40.0, 128), ("bf16", 40.0, 128)])
def test_score_far_above_the_first_tiles(fmt, alpha, heads):
    """One entry in a later tile whose rope part is alpha times head j's rope query: its
    score lies far above everything the kernel saw in the first tile, so the reference
    max must be raised and the pass repeated.  alpha = 40 puts the excess past the fp32
    range of exp2 (the probability computed against the old reference is +inf)."""
    from oracle import cache_store_oracle as cso
    inp = _small(fmt=fmt, heads=heads, topk=256, nreq=2, rows=(1, 1), ctx=(700, 900), seed=91)
    ps, j, t = inp.spec.page_size, 5, 5 * 32 + 3
    pos = int(inp.indices[0, t])
    page = int(inp.page_table[int(inp.row_req[0]), pos // ps])
    slot = page * ps + pos % ps
    qb = inp.q[0, j].float()
    rope = (alpha * qb[512:]).to(torch.bfloat16)
    lat = torch.randn((1, 512), generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    bits = lambda x: x.contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    cache = cso.cache_store(inp.kv_cache.cpu().numpy(), KV[fmt], ps, bits(lat), bits(rope[None]),
                            np.array([slot]))
    inp.kv_cache = torch.from_numpy(cache)
    # precondition: in log2 units the spike exceeds every score of row 0's first tile
    c = inp.spec.softmax_scale / np.log(2.0)
    rows = orc.decode_entries(cache, KV[fmt], ps, np.array([
        int(inp.page_table[int(inp.row_req[0]), int(p) // ps]) * ps + int(p) % ps
        for p in inp.indices[0, :32].tolist()] + [slot]))
    qd = inp.q[0, j].double().numpy()
    first = (rows[:32] @ qd).max() * c
    spike = float(rows[32] @ qd) * c
    assert spike - first > (120.0 if alpha >= 40 else 40.0), (spike, first)
    announce(f"restart {fmt} alpha={alpha} heads={heads} excess={spike - first:.1f}")
    out, lse = gpu_decode(inp)
    o, l = oracle_decode(inp)
    compare(out, lse, o, l, what=f"restart {fmt} alpha={alpha}")


@pytest.mark.parametrize("fmt", ["fp8", "bf16"])
def test_non_finite_inputs_complete_and_stay_local(fmt):
    """A NaN query element and a cache entry with +inf rope values: the call completes
    (neither can make the row's pass repeat forever) and every (row, head) whose result
    the oracle finds finite matches it."""
    from oracle import cache_store_oracle as cso
    inp = _small(fmt=fmt, heads=32, topk=256, nreq=3, rows=(1, 2), ctx=(700, 900), seed=93)
    ps = inp.spec.page_size
    q = inp.q.clone()
    q[0, 3, 100] = float("nan")
    inp.q = q
    r = inp.num_rows - 1                         # a row of another request than row 0's
    assert int(inp.row_req[r]) != int(inp.row_req[0])
    pos = int(inp.indices[r, 6 * 32 + 1])
    page = int(inp.page_table[int(inp.row_req[r]), pos // ps])
    lat = torch.randn((1, 512), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    rope = torch.full((1, 64), float("inf")).to(torch.bfloat16)
    bits = lambda x: x.contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    inp.kv_cache = torch.from_numpy(cso.cache_store(inp.kv_cache.cpu().numpy(), KV[fmt], ps, bits(lat),
                                                    bits(rope), np.array([page * ps + pos % ps])))
    announce(f"non-finite inputs {fmt}")
    out, lse = gpu_decode(inp)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        o, l = oracle_decode(inp)
    ok = np.isfinite(o).all(axis=-1) & np.isfinite(l)
    # row 0 loses only head 3; the rows that select the +inf entry lose every head
    assert not ok[0, 3] and ok[0].sum() == 31 and ok.sum() >= 31 + 32
    got = out.float().cpu().double().numpy()
    d = np.abs(got[ok] - o[ok])
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    lg = lse.cpu().double().numpy()
    assert np.all(np.abs(lg[ok] - l[ok]) <= 1e-3 * np.maximum(1.0, np.abs(l[ok])))


@pytest.mark.parametrize("full", [False, True])
def test_mixed_prefill_and_decode_rows_in_one_launch(full):
    """Requests with 1, 4 or 256 query rows in one launch, each row with its own causal
    top-k list: the grid covers exactly the rows, with no padding to the longest request.
    Sampled rows (the prefill chunks' first, middle and last rows among them)."""
    spec = W.WORKLOADS["mixed_b24_h128_fp8"]
    if not full:
        spec = spec.scaled(num_requests=4, ctx_hi=9000)
    inp = W.make_inputs(spec, 41, device="cpu", cache_device=DEV if full else None)
    counts = torch.bincount(inp.row_req.long()).tolist()
    announce(f"mixed rows={inp.num_rows} per request={counts} full={full}")
    out, lse = gpu_decode(inp)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    first = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rng = np.random.default_rng(41)
    rows = {0, inp.num_rows - 1}
    for b, n in enumerate(counts):
        rows |= {int(first[b]), int(first[b] + n // 2), int(first[b] + n - 1)}
    rows |= set(rng.choice(inp.num_rows, size=8, replace=False).tolist())
    rows = sorted(rows)
    if full:
        sub_cache, sub_pt = page_subset(inp, rows)
        o, l = oracle_decode(inp, rows=rows, kv_cache=sub_cache, page_table=sub_pt)
    else:
        o, l = oracle_decode(inp, rows=rows)
    compare(out[rows], lse[rows], o, l, what=f"mixed rows={len(rows)}")


# ------------------------------------------------------------------ per-tensor FP8 cache

FP8T = W.WORKLOADS["b128_mtp4_h128_fp8t"]


def test_parity_per_tensor_fp8_reduced():
    inp = W.make_inputs(FP8T.scaled(num_requests=2, ctx_hi=16384), 61)
    announce(f"parity fp8t R={inp.num_rows} H={inp.num_heads} K={inp.spec.topk}")
    out, lse = gpu_decode(inp)
    o, l = oracle_decode(inp)
    compare(out, lse, o, l, what="fp8t reduced")


@pytest.mark.parametrize("splits", [1, 3, 16])
def test_per_tensor_fp8_forced_splits(splits):
    inp = _small(fmt="fp8t", heads=64, topk=256, nreq=2, rows=(1, 2), valid="uniform",
                 seed=62, kv_scale=1.0 / 32)
    idx = inp.indices.clone()
    idx[0, :50] = -1
    o, l = oracle_decode(inp, indices=idx)
    announce(f"fp8t forced splits {splits}")
    out, lse = gpu_decode(inp, indices=idx, num_splits=splits)
    compare(out, lse, o, l, what=f"fp8t S={splits}")


def test_per_tensor_fp8_partials_only():
    splits = 5
    inp = _small(fmt="fp8t", heads=32, topk=128, nreq=2, rows=(2,), seed=63, kv_scale=0.05)
    announce(f"fp8t partials only S={splits}")
    po, pl = gpu_decode(inp, num_splits=splits, flags=B.F_PARTIALS_ONLY)
    oc, lc = orc.sparse_mla_decode_partials(
        q_bits(inp.q), inp.kv_cache.numpy(), KV["fp8t"], 64, inp.indices.numpy(),
        inp.row_req.numpy(), inp.page_table.numpy(), inp.spec.softmax_scale, splits,
        kv_scale=inp.spec.kv_scale)
    d = np.abs(po.cpu().double().numpy() - oc)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3
    pg = pl.cpu().double().numpy()
    assert np.array_equal(np.isneginf(pg), np.isneginf(lc))
    f = ~np.isneginf(lc)
    assert np.all(np.abs(pg[f] - lc[f]) <= 1e-3 * np.maximum(1, np.abs(lc[f])))


@pytest.mark.parametrize("heads,ps", [(16, 1), (48, 16), (128, 256)])
def test_per_tensor_fp8_heads_and_page_sizes(heads, ps):
    inp = _small(fmt="fp8t", heads=heads, topk=100, nreq=2, rows=(1, 2), ctx=(600, 1000),
                 ps=ps, seed=64 + ps, kv_scale=1.0 / 64)
    announce(f"fp8t heads {heads} page size {ps}")
    out, lse = gpu_decode(inp)
    o, l = oracle_decode(inp)
    compare(out, lse, o, l, what=f"fp8t H={heads} ps={ps}")


def test_per_tensor_fp8_kv_scale_is_a_pure_rescale():
    """Halving kv_scale while the cache codes stay put equals decoding with the keys and
    values halved: scores scale through softmax_scale, the output by the same factor."""
    inp = _small(fmt="fp8t", heads=32, topk=96, nreq=2, rows=(1,), seed=65, kv_scale=0.5)
    announce("fp8t kv_scale rescale")
    out1, lse1 = gpu_decode(inp)
    spec2 = inp.spec.scaled(kv_scale=0.25, softmax_scale=inp.spec.softmax_scale * 2.0)
    inp2 = W.Inputs(spec2, inp.q, inp.kv_cache, inp.indices, inp.row_req, inp.page_table,
                    inp.sinks, inp.context_lens)
    out2, lse2 = gpu_decode(inp2)
    torch.cuda.synchronize()
    # same scores, output halved exactly (a power-of-two factor)
    assert torch.equal(lse1, lse2)
    assert torch.equal(out1.float() * 0.5, out2.float())


def test_per_tensor_fp8_full_size_sampled():
    inp = W.make_inputs(FP8T, 66, device="cpu", cache_device=DEV)
    announce(f"full fp8t R={inp.num_rows} pages={inp.num_pages}")
    out, lse = gpu_decode(inp)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    R = inp.num_rows
    rng = np.random.default_rng(66)
    rows = sorted({0, R - 1, *rng.choice(R, size=4, replace=False).tolist()})
    sub_cache, sub_pt = page_subset(inp, rows)
    o, l = oracle_decode(inp, rows=rows, kv_cache=sub_cache, page_table=sub_pt)
    compare(out[rows], lse[rows], o, l, what=f"fp8t full rows={len(rows)}")


def _plant_spikes(inp, fmt, j, spikes, seed=5):
    """Write cache entries of row 0 whose scores for head j lie `excess` log2 units above
    the largest score of the row's first tile: spikes = [(list position, excess)].  The
    entry's rope is a multiple of head j's rope query (a bf16 rounding of the solved
    multiple); the latent part is redrawn.  Returns the realised excesses, measured with
    the oracle's decoder."""
    from oracle import cache_store_oracle as cso
    ps = inp.spec.page_size
    c = inp.spec.softmax_scale / np.log(2.0)                 # log2 units per score unit
    qd = inp.q[0, j].double().numpy()
    qr = inp.q[0, j].float()[512:]
    bits = lambda x: x.contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    cache = inp.kv_cache.cpu().numpy()
    slot_of = lambda p: int(inp.page_table[int(inp.row_req[0]), int(inp.indices[0, p]) // ps]) * ps \
        + int(inp.indices[0, p]) % ps  # noqa: E731
    first = orc.decode_entries(cache, KV[fmt], ps, np.array([slot_of(p) for p in range(32)]))
    ref = float((first @ qd).max()) * c
    realised = []
    for n, (pos, excess) in enumerate(spikes):
        lat = torch.randn((1, 512), generator=torch.Generator().manual_seed(seed + n)).to(torch.bfloat16)
        lat_dot = float(lat.double()[0] @ torch.from_numpy(qd[:512]))
        alpha = ((ref + excess) / c - lat_dot) / float(qr.double() @ qr.double())
        rope = (alpha * qr).to(torch.bfloat16)
        cache = cso.cache_store(cache, KV[fmt], ps, bits(lat), bits(rope[None]), np.array([slot_of(pos)]))
        x = float(orc.decode_entries(cache, KV[fmt], ps, np.array([slot_of(pos)]))[0] @ qd) * c
        realised.append(x - ref)
    inp.kv_cache = torch.from_numpy(cache)
    return realised


# Excesses (log2 units over the first tile's largest score) of a spike in tile 3 and one in
# tile 7: both within 2^64 (no repeated pass); the second beyond (one repeat, the reference
# raised to it); the first past exp2's range (+inf: the reference raised by 128, then its
# remaining excess raised again on the careful pass); the first beyond and the second within
# 64 of it (one repeat)
@pytest.mark.parametrize("fmt,heads", [("fp8", 32), ("fp8", 128), ("bf16", 128)])
@pytest.mark.parametrize("e1,e2", [(40.0, 60.0), (50.0, 100.0), (200.0, 100.0), (100.0, 150.0)])
def test_two_spikes_in_different_tiles(fmt, heads, e1, e2):
    inp = _small(fmt=fmt, heads=heads, topk=320, nreq=2, rows=(1, 1), ctx=(900, 1100), seed=95)
    j = 7
    realised = _plant_spikes(inp, fmt, j, [(3 * 32 + 5, e1), (7 * 32 + 11, e2)])
    for want, got in zip((e1, e2), realised):
        assert abs(got - want) < 2.0, (want, got)
    announce(f"two spikes {fmt} H={heads} excess={realised[0]:.1f},{realised[1]:.1f}")
    out, lse = gpu_decode(inp)
    o, l = oracle_decode(inp)
    compare(out, lse, o, l, what=f"two spikes {fmt} {e1}/{e2}")
