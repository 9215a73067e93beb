"""Bit-exact checks of the decode kernel's own gather and dequantization, through
sparse_mla_decode_run (the hot path), not through a helper kernel.

Two constructions make the decode's result an exactly known bf16 value:
- a row with a single valid index and no sink: its one probability is exp2(0) = 1, the
  weight sum is 1, so out[r][h] must be that entry's dequantized V, bit for bit, whatever
  q is.  With a one-hot q (head h reads dim d_h) the LSE is softmax_scale * k[d_h], which
  pins every one of the 576 dims the QK contraction reads, the rope half included;
- q = 0 over 32 or 64 valid entries (one or two full tiles): every score is 0, every
  probability 1, and out = (sum of V) / n with n a power of two.  The cache values are
  chosen so that every partial sum is exact in fp32 (UE8M0 scales of one row's entries
  within one binade per group, BF16 values on a 2^-4 grid), so the result is exact in any
  summation order and the bf16 rounding of the exact quotient is the only rounding.
  This places an entry at every one of a tile's 32 token positions.
The expected values come from the float64 oracle's decoder and decode on the same bytes.
Duplicate indices (reading: a multiset) are checked at the standard tolerance too.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import sparse_mla_oracle as orc
from sparse_mla_decode_03_amd import binding as B
from tests.gpu_util import KV, announce, compare

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda")
SCALE = 1.0 / 24.0


def _finite_codes() -> np.ndarray:
    """All 256 e4m3fn codes with the two NaN codes replaced by zeros."""
    c = np.arange(256, dtype=np.uint8)
    c[[0x7F, 0xFF]] = 0
    return c


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _zero_sign_free(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns with -0 written as +0: a sum that starts from +0 gives +0 for an
    entry whose value is -0 (code 0x80), the same number; every other pattern is compared
    as it is."""
    b = bits.copy()
    b[b == 0x8000] = 0
    return b


def _cache(fmt: str, n_slots: int, ps: int, rng, scale_bytes=None, bf16_grid=False):
    """Pages holding n_slots entries: latent codes covering every finite e4m3fn code
    (rolled per slot), the given UE8M0 bytes [n_slots, 8] (default: 10..246), rope N(0,1).
    BF16: N(0,1) values, or integers in [-255, 255] times 2^-4 (bf16_grid)."""
    npg = n_slots // ps
    codes = np.stack([np.roll(np.tile(_finite_codes(), 3)[:576], 37 * s) for s in range(n_slots)])
    if fmt == "fp8t":
        return codes.reshape(npg, 576 * ps)
    if fmt == "bf16":
        if bf16_grid:
            vals = rng.integers(-255, 256, size=(n_slots, 576)).astype(np.float32) / 16.0
        else:
            vals = rng.standard_normal((n_slots, 576)).astype(np.float32)
        return _bf16_bits(vals).view(np.uint8).reshape(npg, 1152 * ps)
    if scale_bytes is None:
        scale_bytes = rng.integers(10, 247, size=(n_slots, 8))
    rope = _bf16_bits(rng.standard_normal((n_slots, 64)).astype(np.float32))
    pages = np.zeros((npg, 648 * ps), dtype=np.uint8)
    for p in range(npg):
        sl = slice(p * ps, (p + 1) * ps)
        pages[p, : 512 * ps] = codes[sl, :512].reshape(-1)
        pages[p, 512 * ps: 640 * ps] = rope[sl].reshape(-1).view(np.uint8)
        pages[p, 640 * ps:] = np.asarray(scale_bytes[sl], dtype=np.uint8).reshape(-1)
    return pages


def _decode(pages, fmt, ps, q, idx, row_req, pt, kv_scale=1.0):
    out, lse = B.sparse_mla_decode(q.to(DEV), torch.from_numpy(pages).to(DEV),
                                   torch.from_numpy(idx).to(DEV), torch.from_numpy(row_req).to(DEV),
                                   torch.from_numpy(pt).to(DEV), None, fmt, ps, SCALE,
                                   kv_scale=kv_scale)
    torch.cuda.synchronize()
    return out, lse


def _tables(R: int, pages_per_req: int, rng):
    """One request per row, each with its own shuffled pages."""
    perm = rng.permutation(R * pages_per_req).astype(np.int32)
    return np.arange(R, dtype=np.int32), perm.reshape(R, pages_per_req)


@pytest.mark.parametrize("fmt", ["fp8", "bf16", "fp8t"])
@pytest.mark.parametrize("heads", [16, 64, 96, 128])
def test_single_entry_rows_out_is_the_entry_bit_exact(fmt, heads):
    """One valid index per row at list positions across the row (first, last, around the
    32-position tile edges), one-hot queries over all 576 dims: out == V of the entry bit
    for bit, lse == softmax_scale * k[d_h] to fp32 rounding."""
    rng = np.random.default_rng(heads + {"fp8": 0, "bf16": 1, "fp8t": 2}[fmt])
    ps, ppr, K, R = 16, 3, 96, 48
    kv_scale = 1.0 / 64 if fmt == "fp8t" else 1.0
    row_req, pt = _tables(R, ppr, rng)
    pages = _cache(fmt, R * ppr * ps, ps, rng)
    where = [0, 1, 31, 32, 33, 63, 64, 95, 17, 50]
    idx = np.full((R, K), -1, dtype=np.int32)
    tok = rng.integers(0, ppr * ps, size=R).astype(np.int32)
    for r in range(R):
        idx[r, where[r % len(where)]] = tok[r]
    q = np.zeros((R, heads, 576), dtype=np.float32)
    dims = (np.arange(R)[:, None] * heads + np.arange(heads)[None, :]) % 576
    for r in range(R):
        q[r, np.arange(heads), dims[r]] = 1.0
    qb = torch.from_numpy(q).to(torch.bfloat16)
    announce(f"single-entry rows {fmt} H={heads}")
    out, lse = _decode(pages, fmt, ps, qb, idx, row_req, pt, kv_scale)
    slots = pt[row_req, tok // ps] * ps + tok % ps
    k = orc.decode_entries(pages, KV[fmt], ps, slots, kv_scale)            # [R, 576]
    want = _bf16_bits(k[:, :512].astype(np.float32))
    assert np.array_equal(orc.bf16_bits_to_f64(want), k[:, :512]), "V not exact in bf16"
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)              # [R, H, 512]
    bad = np.nonzero(_zero_sign_free(got) != _zero_sign_free(want)[:, None, :])
    assert bad[0].size == 0, f"{bad[0].size} bit mismatches, first at {[b[0] for b in bad]}"
    lse_ref = SCALE * k[np.arange(R)[:, None], dims]                       # [R, H]
    lg = lse.cpu().double().numpy()
    # (scores of the smallest entries, 2^-126 / 24, are fp32 denormals: 1e-36 absolute)
    assert np.all(np.abs(lg - lse_ref) <= 1e-6 * np.abs(lse_ref) + 1e-36), \
        float(np.max(np.abs(lg - lse_ref) / np.maximum(np.abs(lse_ref), 1e-300)))


def _exact_sum_case(fmt, heads, seed, dup=False):
    """Rows of 32 or 64 valid entries (alternating) over a list of 128 positions, q = 0,
    no sink; values chosen so every partial sum is exact in fp32."""
    rng = np.random.default_rng(seed)
    ps, ppr, K, R = 64, 2, 128, 12
    row_req, pt = _tables(R, ppr, rng)
    n_slots = R * ppr * ps
    scale_bytes = None
    ns = [32 if r % 2 == 0 else 64 for r in range(R)]
    if fmt == "fp8":
        # per (request, group) one binade for 64-entry rows, two adjacent ones for 32-entry
        # rows: |sum| < 448 * 2^(e+1-127) * 32 = 2^23.8 units of the smallest ulp 2^(e-136).
        # e <= 239 keeps 64 * 448 * 2^(e-127) below fp32's range, e >= 16 keeps the smallest
        # nonzero mean 2^(e-136) / 64 a normal number
        scale_bytes = np.zeros((n_slots, 8), dtype=np.int64)
        base = rng.integers(16, 239, size=(R, 8))
        for r in range(R):
            slots_r = (pt[r][:, None] * ps + np.arange(ps)[None, :]).reshape(-1)
            bump = rng.integers(0, 2, size=(slots_r.size, 8)) if ns[r] == 32 else 0
            scale_bytes[slots_r] = base[r][None, :] + bump
    pages = _cache(fmt, n_slots, ps, rng, scale_bytes=scale_bytes, bf16_grid=True)
    idx = np.full((R, K), -1, dtype=np.int32)
    for r in range(R):
        pos = np.sort(rng.choice(K, size=ns[r], replace=False))
        if dup and r in (2, 3):
            toks = rng.choice(ppr * ps, size=ns[r] // 2, replace=False)
            toks = np.concatenate([toks, toks[rng.permutation(toks.size)]])   # each twice
        else:
            toks = rng.choice(ppr * ps, size=ns[r], replace=False)
        idx[r, pos] = toks
    q = torch.zeros((R, heads, 576), dtype=torch.bfloat16)
    return pages, ps, q, idx, row_req, pt, ns


@pytest.mark.parametrize("fmt", ["fp8", "bf16", "fp8t"])
@pytest.mark.parametrize("heads", [16, 64, 128])
def test_full_tiles_zero_query_exact_sums_bit_exact(fmt, heads):
    """Every token position of one or two full tiles: out == bf16(sum V / n) exactly."""
    pages, ps, q, idx, row_req, pt, ns = _exact_sum_case(fmt, heads, 200 + heads, dup=True)
    kv_scale = 1.0 / 64 if fmt == "fp8t" else 1.0
    announce(f"exact sums {fmt} H={heads}")
    out, lse = _decode(pages, fmt, ps, q, idx, row_req, pt, kv_scale)
    qbits = q.view(torch.int16).numpy().view(np.uint16)
    o, l = orc.sparse_mla_decode(qbits, pages, KV[fmt], ps, idx, row_req, pt, None, SCALE,
                                 kv_scale=kv_scale)
    # precondition: the oracle's float64 sums are exact (each row's V sum times n / n)
    for r in range(len(ns)):
        slots = orc.translate(idx[r], orc.IDX_LOGICAL, r, pt, ps, pages.shape[0])[1]
        v = orc.decode_entries(pages, KV[fmt], ps, slots, kv_scale)[:, :512]
        s32 = v.astype(np.float32).sum(0, dtype=np.float32)
        assert np.array_equal(s32.astype(np.float64), v.sum(0)), "fp32 sum not exact"
        assert np.array_equal(o[r, 0], v.sum(0) / ns[r])
    want = _bf16_bits(o.astype(np.float32))
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(_zero_sign_free(got) != _zero_sign_free(want))
    assert bad[0].size == 0, f"{bad[0].size} bit mismatches, first at {[b[0] for b in bad]}"
    lg = lse.cpu().double().numpy()
    assert np.all(np.abs(lg - np.log(np.array(ns, dtype=np.float64))[:, None]) <= 1e-6)


@pytest.mark.parametrize("fmt,heads,topk", [("fp8", 64, 256), ("fp8", 128, 256), ("bf16", 32, 16)])
def test_duplicate_indices_are_a_multiset(fmt, heads, topk):
    """Rows whose lists repeat indices: each occurrence is a term (the oracle's multiset);
    at K = 16 treating the repeats as one entry would miss the tolerance by far."""
    from sparse_mla_decode_03_amd import workloads as W
    spec = W.WorkloadSpec("dup", 3, (1, 2), heads, topk, 300, 700, fmt, page_size=16)
    inp = W.make_inputs(spec, 300 + topk)
    idx = inp.indices.clone()
    rng = np.random.default_rng(5)
    R, K = idx.shape
    idx[0, : K // 2] = idx[0, K // 2:].clone()                  # every entry twice
    idx[1, 1:9] = int(idx[1, 0])                                # one entry nine times
    idx[-1, torch.from_numpy(rng.choice(K, size=K // 4, replace=False))] = int(idx[-1, 3])
    from tests.gpu_util import gpu_decode, oracle_decode
    announce(f"duplicates {fmt} H={heads} K={topk}")
    out, lse = gpu_decode(inp, indices=idx)
    o, l = oracle_decode(inp, indices=idx)
    compare(out, lse, o, l, what=f"duplicates {fmt} K={topk}")
    if topk <= 16:
        dedup = idx.clone()
        dedup[1, 1:9] = -1
        od, _ = oracle_decode(inp, indices=dedup)
        assert np.abs(od[1] - o[1]).max() > 2e-2
