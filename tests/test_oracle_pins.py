"""Pins for the float64 oracle: it is checked against things other than itself.

- number formats against torch's own float8_e4m3fn / bfloat16 decoders and the OCP spec
  points in golden/e4m3fn_spec_points.txt;
- the cache layout against the hand-built page in golden/fp8_page_ps2.txt;
- the attention against an independent pure-Python brute force on tiny inputs, against
  torch's scaled_dot_product_attention (float64) for a dense selection, and against
  closed forms (one-hot q, q = 0, one entry, sink identity);
- invariants: -1 insertion, order, page relocation, LOGICAL vs GLOBAL, split + merge.
Planted-mistake tests at the end show that a plausible slip in the oracle fails a pin.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import sparse_mla_oracle as orc
from sparse_mla_decode_03_amd import workloads as W
from tests import brute_force
from tests.golden_io import e4m3fn_points, fp8_page_fixture

KV = {"bf16": orc.KV_BF16, "fp8": orc.KV_FP8_UE8M0, "fp8t": orc.KV_FP8_TENSOR}


def _q_bits(inp):
    return inp.q.contiguous().view(torch.int16).numpy().view(np.uint16)


def _np(inp):
    return dict(q_bits=_q_bits(inp), cache=inp.kv_cache.numpy(), kv_format=KV[inp.spec.kv_format],
                page_size=inp.spec.page_size, indices=inp.indices.numpy(),
                row_req=inp.row_req.numpy(), page_table=inp.page_table.numpy(),
                sinks=None if inp.sinks is None else inp.sinks.numpy(),
                softmax_scale=inp.spec.softmax_scale, kv_scale=inp.spec.kv_scale)


def _tiny(fmt, seed, heads=3, topk=12, ps=4, ctx=(20, 40), sinks="normal", valid="all",
          rows=(1, 2), nreq=2):
    spec = W.WorkloadSpec("tiny", nreq, rows, heads, topk, ctx[0], ctx[1], fmt, page_size=ps,
                          valid=valid, sinks=sinks,
                          kv_scale=1.0 / 64 if fmt == "fp8t" else 1.0)
    return W.make_inputs(spec, seed)


def _oracle(d, rows=None, index_mode=orc.IDX_LOGICAL, **over):
    args = dict(d)
    args.update(over)
    return orc.sparse_mla_decode(args["q_bits"], args["cache"], args["kv_format"],
                                 args["page_size"], args["indices"], args["row_req"],
                                 args["page_table"], args["sinks"], args["softmax_scale"],
                                 index_mode=index_mode, rows=rows, kv_scale=args["kv_scale"])


# ---------------------------------------------------------------- number formats

def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert set(np.nonzero(np.isnan(ours))[0].tolist()) == {0x7F, 0xFF}


def test_e4m3fn_spec_points():
    for code, val in e4m3fn_points():
        got = float(orc.e4m3fn_to_f64(np.array([code], dtype=np.uint8))[0])
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)
    assert np.nanmax(orc.e4m3fn_to_f64(np.arange(256))) == 448.0


def test_ue8m0_closed_form():
    e = np.arange(256)
    v = orc.ue8m0_to_f64(e)
    for k in range(255):
        assert v[k] == math.ldexp(1.0, k - 127)
    assert math.isnan(v[255])
    assert v[127] == 1.0 and v[130] == 8.0


def test_bf16_all_codes_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert orc.bf16_bits_to_f64(np.array([0x3F80, 0xC000], dtype=np.uint16)).tolist() == [1.0, -2.0]


# ---------------------------------------------------------------- layout

def test_fp8_layout_fixture_decodes_by_hand_values():
    page, ps, expects = fp8_page_fixture()
    buf = np.frombuffer(page, dtype=np.uint8)
    rows = orc.decode_entries(buf, orc.KV_FP8_UE8M0, ps, [0, 1])
    for slot, lo, hi, val in expects:
        seg = rows[slot, lo:hi]
        assert np.all(seg == val), (slot, lo, hi, val, seg[:4])
    # the brute force's own offsets agree on every dim
    for slot in (0, 1):
        assert rows[slot].tolist() == brute_force.entry(page, "fp8", ps, slot)


def test_fp8_tensor_page_decodes_by_hand_values():
    """Per-tensor FP8 entry: 576 e4m3fn codes in a row, each times the one tensor scale."""
    ps = 2
    page = np.zeros(576 * ps, dtype=np.uint8)
    page[0] = 0x38                  # slot 0 dim 0: 1.0
    page[511] = 0xC0                # slot 0 dim 511: -2.0
    page[512] = 0x01                # slot 0 dim 512 (first rope dim): 2^-9
    page[575] = 0x7E                # slot 0 dim 575: 448
    page[576 + 5] = 0xB4            # slot 1 dim 5: -0.75
    page[576 + 575] = 0x30          # slot 1 dim 575: 0.5
    rows = orc.decode_entries(page, orc.KV_FP8_TENSOR, ps, [0, 1], kv_scale=0.25)
    want = np.zeros((2, 576))
    want[0, 0], want[0, 511], want[0, 512], want[0, 575] = 0.25, -0.5, 2.0 ** -11, 112.0
    want[1, 5], want[1, 575] = -0.1875, 0.125
    assert np.array_equal(rows, want)
    for slot in (0, 1):
        assert rows[slot].tolist() == brute_force.entry(page.tobytes(), "fp8t", ps, slot, 0.25)


def test_fp8_tensor_equals_bf16_cache_of_the_same_values():
    """Every e4m3fn value times a power of two is a bf16 value, so a per-tensor FP8 cache
    and the BF16 cache holding its decoded values give the same attention."""
    inp = _tiny("fp8t", 4)
    d = _np(inp)
    o, lse = _oracle(d)
    npg = d["cache"].shape[0]
    ps = d["page_size"]
    vals = orc.decode_entries(d["cache"], orc.KV_FP8_TENSOR, ps, np.arange(npg * ps),
                              kv_scale=d["kv_scale"])
    bf = torch.from_numpy(vals).to(torch.bfloat16)
    assert np.array_equal(bf.double().numpy(), vals)
    d2 = dict(d, cache=bf.view(torch.uint8).reshape(npg, ps * 1152).numpy(),
              kv_format=orc.KV_BF16, kv_scale=1.0)
    o2, lse2 = _oracle(d2)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_packer_writes_fixture_layout():
    """The generator's page packer puts each region where the layout says."""
    page, ps, _ = fp8_page_fixture()
    buf = torch.frombuffer(bytearray(page), dtype=torch.uint8)
    codes = buf[:1024].reshape(2, 512)
    rope = buf[1024:1280].view(torch.bfloat16).reshape(2, 64)
    scales = buf[1280:1296].reshape(2, 8)
    packed = W.pack_fp8_pages(codes, rope, scales, ps)
    assert bytes(packed.reshape(-1).numpy().tobytes()) == page


def test_bf16_layout_slot_addressing():
    """slot -> page = slot // ps, row = slot % ps; every dim comes from its own bytes."""
    ps, npg = 4, 3
    vals = torch.arange(npg * ps * 576, dtype=torch.float32).remainder(251).sub(125)
    cache = vals.to(torch.bfloat16).view(torch.uint8).reshape(npg, ps * 1152)
    rows = orc.decode_entries(cache.numpy(), orc.KV_BF16, ps, np.arange(npg * ps))
    assert np.array_equal(rows, vals.reshape(npg * ps, 576).double().numpy())


def test_encoder_roundtrip_within_fp8_resolution():
    """Generator codes decode (by the oracle) to within half an e4m3 ulp of the drawn
    values, and no group overflows 448 before scaling."""
    g = torch.Generator().manual_seed(5)
    x = torch.randn(64, 512, generator=g) * torch.logspace(-3, 3, 64)[:, None]
    codes, sb = W.encode_fp8_groups(x)
    scale = orc.ue8m0_to_f64(sb.numpy())
    dec = orc.e4m3fn_to_f64(codes.numpy()) * np.repeat(scale, 64, axis=1)
    xs = x.double().numpy()
    # relative spacing of e4m3 is 2^-3 for normals: error <= 2^-4 |x| or the subnormal step
    err = np.abs(dec - xs)
    bound = np.maximum(np.abs(xs) * 2.0 ** -4, np.repeat(scale, 64, axis=1) * 2.0 ** -10)
    assert np.all(err <= bound)
    amax = np.abs(xs).reshape(64, 8, 64).max(-1)
    assert np.all(amax <= 448 * scale) and np.all(amax > 224 * scale)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp8t"])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_oracle_matches_brute_force(fmt, seed):
    inp = _tiny(fmt, seed, heads=2, topk=8, ctx=(9, 30))
    idx = inp.indices.clone()
    rng = np.random.default_rng(seed)
    # -1 anywhere, and one repeated index (a multiset term)
    idx[0, rng.integers(0, 8)] = -1
    idx[-1, 3] = idx[-1, 5]
    d = _np(inp)
    d["indices"] = idx.numpy()
    o, lse = _oracle(d)
    cache = inp.kv_cache.numpy().tobytes()
    pt = inp.page_table.numpy()
    ps = inp.spec.page_size
    for r in range(inp.num_rows):
        b = int(inp.row_req[r])
        slot_of = lambda t: int(pt[b, t // ps]) * ps + t % ps  # noqa: E731
        qr = [[float(x) for x in inp.q[r, h].double().tolist()] for h in range(inp.num_heads)]
        bo, bl = brute_force.decode_row(qr, cache, fmt, ps, idx[r].tolist(), slot_of,
                                        inp.spec.softmax_scale, d["sinks"], inp.spec.kv_scale)
        np.testing.assert_allclose(o[r], np.array(bo), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[r], np.array(bl), rtol=1e-12, atol=1e-14)


def test_dense_selection_matches_torch_sdpa():
    """Selecting every token of a request equals dense attention (torch SDPA, float64)."""
    inp = _tiny("fp8", 7, heads=4, topk=32, ctx=(32, 32), sinks="none", rows=(1,), nreq=1)
    idx = torch.arange(32, dtype=torch.int32)[None, :]
    d = _np(inp)
    d["indices"] = idx.numpy()
    o, lse = _oracle(d)
    pt = inp.page_table.numpy()[0]
    slots = pt[np.arange(32) // 4] * 4 + np.arange(32) % 4
    k = torch.tensor([brute_force.entry(inp.kv_cache.numpy().tobytes(), "fp8", 4, int(s))
                      for s in slots], dtype=torch.float64)
    q = inp.q[0].double()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[None], k[None], k[None, :, :512], scale=inp.spec.softmax_scale)[0]
    np.testing.assert_allclose(o[0], ref.numpy(), rtol=1e-12, atol=1e-14)
    s = inp.spec.softmax_scale * (q @ k.T)
    np.testing.assert_allclose(lse[0], torch.logsumexp(s, dim=1).numpy(), rtol=1e-13)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("dim", [0, 200, 511, 512, 575])
def test_one_hot_query_scores_one_dim(dim):
    """q = e_dim gives s_j = scale * k_j[dim]; covers latent and rope halves."""
    inp = _tiny("fp8", 11, heads=1, topk=8, ctx=(16, 16), sinks="none", rows=(1,), nreq=1)
    q = torch.zeros(1, 1, 576, dtype=torch.bfloat16)
    q[0, 0, dim] = 1.0
    d = _np(inp)
    d["q_bits"] = q.view(torch.int16).numpy().view(np.uint16)
    d["softmax_scale"] = 0.75
    o, lse = _oracle(d)
    pt = inp.page_table.numpy()[0]
    t = inp.indices.numpy()[0]
    k = orc.decode_entries(d["cache"], orc.KV_FP8_UE8M0, 4, pt[t // 4] * 4 + t % 4)
    s = 0.75 * k[:, dim]
    assert lse[0, 0] == pytest.approx(scipy.special.logsumexp(s), rel=1e-14)
    np.testing.assert_allclose(o[0, 0], scipy.special.softmax(s) @ k[:, :512], rtol=1e-12,
                               atol=1e-15)


def test_zero_query_gives_mean_and_log_n():
    inp = _tiny("bf16", 12, heads=2, topk=12, ctx=(20, 20), rows=(1,), nreq=1)
    d = _np(inp)
    d["q_bits"] = np.zeros_like(d["q_bits"])
    d["sinks"] = None
    o, lse = _oracle(d)
    pt = inp.page_table.numpy()[0]
    t = inp.indices.numpy()[0]
    k = orc.decode_entries(d["cache"], orc.KV_BF16, 4, pt[t // 4] * 4 + t % 4)
    np.testing.assert_allclose(o[0], np.broadcast_to(k[:, :512].mean(0), (2, 512)), rtol=1e-13)
    np.testing.assert_allclose(lse[0], math.log(12), rtol=1e-15)


def test_single_entry_is_exact():
    inp = _tiny("fp8", 13, heads=3, topk=4, ctx=(8, 8), sinks="none", rows=(1,), nreq=1)
    d = _np(inp)
    idx = np.full((1, 4), -1, dtype=np.int32)
    idx[0, 2] = 5
    d["indices"] = idx
    o, lse = _oracle(d)
    pt = inp.page_table.numpy()[0]
    k = brute_force.entry(d["cache"].tobytes(), "fp8", 4, int(pt[1]) * 4 + 1)
    for h in range(3):
        qh = inp.q[0, h].double().tolist()
        s = inp.spec.softmax_scale * math.fsum(a * b for a, b in zip(qh, k))
        assert o[0, h].tolist() == k[:512]
        assert lse[0, h] == pytest.approx(s, rel=1e-14, abs=1e-15)


@pytest.mark.parametrize("sig", [-3.0, 0.0, 2.0, 5.0])
def test_sink_identity(sig):
    """With a sink: o = o_plain * sigmoid(lse_plain - sigma), lse = logaddexp(lse_plain, sigma)."""
    inp = _tiny("fp8", 14, heads=3, topk=16, ctx=(30, 40))
    d = _np(inp)
    d["sinks"] = None
    o0, l0 = _oracle(d)
    d["sinks"] = np.full(3, sig, dtype=np.float32)
    o1, l1 = _oracle(d)
    np.testing.assert_allclose(o1, o0 * scipy.special.expit(l0 - sig)[..., None], rtol=1e-12,
                               atol=1e-15)
    np.testing.assert_allclose(l1, np.logaddexp(l0, sig), rtol=1e-14)


def test_sink_limits():
    inp = _tiny("bf16", 15, heads=2, topk=8, ctx=(16, 16))
    d = _np(inp)
    d["sinks"] = None
    o0, l0 = _oracle(d)
    d["sinks"] = np.full(2, -np.inf, dtype=np.float32)
    o1, l1 = _oracle(d)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    d["sinks"] = np.full(2, 200.0, dtype=np.float32)
    o2, l2 = _oracle(d)
    assert np.max(np.abs(o2)) < 1e-60
    np.testing.assert_allclose(l2, 200.0, rtol=1e-15)


# ---------------------------------------------------------------- invariants

def test_masking_and_order_invariance():
    inp = _tiny("fp8", 16, heads=2, topk=16, ctx=(40, 60))
    d = _np(inp)
    o0, l0 = _oracle(d)
    rng = np.random.default_rng(0)
    R, K = d["indices"].shape
    wide = np.full((R, 2 * K), -1, dtype=np.int32)
    for r in range(R):
        pos = np.sort(rng.choice(2 * K, size=K, replace=False))
        wide[r, pos] = rng.permutation(d["indices"][r])
    d2 = dict(d, indices=wide)
    o1, l1 = _oracle(d2)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l1, l0, rtol=1e-13)
    d3 = dict(d, indices=np.full((R, K), -1, dtype=np.int32))
    o3, l3 = _oracle(d3)
    assert np.all(o3 == 0.0)
    np.testing.assert_array_equal(l3, np.broadcast_to(d["sinks"].astype(np.float64), l3.shape))
    o4, l4 = _oracle(dict(d3, sinks=None))
    assert np.all(o4 == 0.0) and np.all(np.isneginf(l4))


def test_page_relocation_and_global_mode():
    inp = _tiny("fp8", 17, heads=2, topk=12, ctx=(20, 50))
    d = _np(inp)
    o0, l0 = _oracle(d)
    rng = np.random.default_rng(3)
    npg = d["cache"].shape[0]
    perm = rng.permutation(npg)          # new page perm[p] holds old page p
    cache2 = np.empty_like(d["cache"])
    cache2[perm] = d["cache"]
    pt2 = np.where(d["page_table"] >= 0, perm[np.maximum(d["page_table"], 0)], -1)
    o1, l1 = _oracle(dict(d, cache=cache2, page_table=pt2))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # GLOBAL mode with pre-translated slots == LOGICAL mode
    ps = d["page_size"]
    g = np.full_like(d["indices"], -1)
    for r in range(g.shape[0]):
        b = d["row_req"][r]
        t = d["indices"][r]
        v = t != -1
        g[r, v] = d["page_table"][b, t[v] // ps] * ps + t[v] % ps
    o2, l2 = _oracle(dict(d, indices=g), index_mode=orc.IDX_GLOBAL)
    assert np.array_equal(o0, o2) and np.array_equal(l0, l2)



def test_invalid_ids_are_masked_hand_worked():
    """Every id that names no cache slot is dropped like -1 (hand-worked cases): negative
    ids, a page index past the request's block-table row, a page id outside the pool, a
    request outside the table, and (GLOBAL) a slot outside the pool."""
    pt = np.array([[2, -1, 7], [5, 1, 0]], dtype=np.int32)
    num_pages = 6                                   # page id 7 is outside the pool
    row0 = np.array([3, -1, -7, 5, 9, 12, 1, 2])
    pos, slots = orc.translate(row0, orc.IDX_LOGICAL, 0, pt, 4, num_pages)
    assert pos.tolist() == [0, 6, 7] and slots.tolist() == [11, 9, 10]
    pos, slots = orc.translate(np.array([4, 11, 0]), orc.IDX_LOGICAL, 1, pt, 4, num_pages)
    assert pos.tolist() == [0, 1, 2] and slots.tolist() == [4, 3, 20]
    for req in (2, -1):
        pos, slots = orc.translate(row0, orc.IDX_LOGICAL, req, pt, 4, num_pages)
        assert pos.size == 0 and slots.size == 0
    pos, slots = orc.translate(np.array([3, -1, -7, 23, 24, 0]), orc.IDX_GLOBAL, -1, pt, 4, num_pages)
    assert pos.tolist() == [0, 3, 5] and slots.tolist() == [3, 23, 0]


def test_invalid_ids_decode_like_minus_one():
    """A row with planted bad ids decodes to the brute force over its valid ids alone."""
    inp = _tiny("fp8", 21, heads=2, topk=10, ctx=(20, 30))
    d = _np(inp)
    idx = d["indices"].copy()
    npg = d["cache"].shape[0]
    idx[0, 1] = -5
    idx[0, 4] = d["page_table"].shape[1] * 4 + 2         # past the block-table row
    pt = d["page_table"].copy()
    b1 = int(d["row_req"][-1])
    pt[b1, 0] = npg + 3                                  # a page id outside the pool
    o, lse = _oracle(dict(d, indices=idx, page_table=pt))
    cache = inp.kv_cache.numpy().tobytes()
    for r in range(inp.num_rows):
        b = int(d["row_req"][r])
        keep = [int(t) for t in idx[r] if t >= 0 and t // 4 < pt.shape[1]
                and 0 <= pt[b, t // 4] < npg]
        slot_of = lambda t: int(pt[b, t // 4]) * 4 + t % 4  # noqa: E731
        qr = [[float(x) for x in inp.q[r, h].double().tolist()] for h in range(2)]
        bo, bl = brute_force.decode_row(qr, cache, "fp8", 4, keep, slot_of, d["softmax_scale"],
                                        d["sinks"])
        np.testing.assert_allclose(o[r], np.array(bo), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lse[r], np.array(bl), rtol=1e-12, atol=1e-14)


def test_chunk_bounds_by_hand():
    """Chunk c holds list positions [c*C, (c+1)*C), C = ceil(K/S): the 16 chunks of 128
    positions of the split-16 workload, and hand-listed ragged cases whose last chunks
    are short or empty."""
    assert orc.chunk_bounds(2048, 16) == [(128 * c, 128 * c + 128) for c in range(16)]
    assert orc.chunk_bounds(24, 16) == [(2 * c, 2 * c + 2) for c in range(12)] + [(24, 24)] * 4
    assert orc.chunk_bounds(20, 8) == [(0, 3), (3, 6), (6, 9), (9, 12), (12, 15), (15, 18),
                                       (18, 20), (20, 20)]
    assert orc.chunk_bounds(5, 1) == [(0, 5)]
    assert orc.chunk_bounds(7, 7) == [(c, c + 1) for c in range(7)]


def test_partials_are_the_chunks_of_list_positions():
    """Each sink-free partial equals the brute force over exactly its chunk's list
    positions (-1 entries inside a chunk included), K = 20 in 8 chunks of 3."""
    inp = _tiny("bf16", 22, heads=2, topk=20, ctx=(40, 60), rows=(1,), nreq=2)
    d = _np(inp)
    idx = d["indices"].copy()
    idx[0, [4, 5, 19]] = -1
    oc, lc = orc.sparse_mla_decode_partials(d["q_bits"], d["cache"], d["kv_format"], 4, idx,
                                            d["row_req"], d["page_table"], d["softmax_scale"], 8)
    cache = inp.kv_cache.numpy().tobytes()
    pt = d["page_table"]
    hand = [(0, 3), (3, 6), (6, 9), (9, 12), (12, 15), (15, 18), (18, 20), (20, 20)]
    for r in range(inp.num_rows):
        b = int(d["row_req"][r])
        slot_of = lambda t: int(pt[b, t // 4]) * 4 + t % 4  # noqa: E731
        qr = [[float(x) for x in inp.q[r, h].double().tolist()] for h in range(2)]
        for c, (lo, hi) in enumerate(hand):
            bo, bl = brute_force.decode_row(qr, cache, "bf16", 4, idx[r, lo:hi].tolist(), slot_of,
                                            d["softmax_scale"], None)
            np.testing.assert_allclose(oc[r, c], np.array(bo), rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(lc[r, c], np.array(bl), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("splits", [1, 2, 3, 16, 24])
def test_split_merge_reproduces_unsplit(splits):
    inp = _tiny("fp8", 18, heads=3, topk=24, ctx=(30, 60), valid="uniform")
    d = _np(inp)
    d["indices"][0, :5] = -1                  # an empty leading chunk for large S
    o0, l0 = _oracle(d)
    oc, lc = orc.sparse_mla_decode_partials(d["q_bits"], d["cache"], d["kv_format"],
                                            d["page_size"], d["indices"], d["row_req"],
                                            d["page_table"], d["softmax_scale"], splits)
    o1, l1 = orc.merge_partials(oc, lc, d["sinks"])
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l1, l0, rtol=1e-13)
    # partials are sink-free softmax over their chunk
    bounds = orc.chunk_bounds(24, splits)
    assert len(bounds) == splits and bounds[-1][1] == 24


def test_merge_random_partitions_and_empty_chunks():
    rng = np.random.default_rng(9)
    inp = _tiny("bf16", 19, heads=2, topk=16, ctx=(40, 40), rows=(1,), nreq=1)
    d = _np(inp)
    o0, l0 = _oracle(d)
    pt = d["page_table"][0]
    t = d["indices"][0]
    k = orc.decode_entries(d["cache"], orc.KV_BF16, 4, pt[t // 4] * 4 + t % 4)
    q = orc.bf16_bits_to_f64(d["q_bits"][0])
    for _ in range(5):
        labels = rng.integers(0, 6, size=16)   # 6 parts, some may be empty
        parts = [orc.attend(q, k[labels == c], d["softmax_scale"], None) for c in range(6)]
        oc = np.stack([p[0] for p in parts])[None]
        lc = np.stack([p[1] for p in parts])[None]
        o1, l1 = orc.merge_partials(oc, lc, d["sinks"])
        np.testing.assert_allclose(o1[0], o0[0], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(l1[0], l0[0], rtol=1e-13)
    # all chunks empty, with and without sink
    oe, le = orc.merge_partials(np.zeros((1, 3, 2, 512)), np.full((1, 3, 2), -np.inf),
                                np.array([0.5, -np.inf]))
    assert np.all(oe == 0) and le[0, 0] == 0.5 and np.isneginf(le[0, 1])


# ---------------------------------------------------------------- planted mistakes

def _run_pin(check):
    """True when the pin passes; a failed assertion or an error (a slip that indexes out of
    range) both count as the pin catching the mistake."""
    try:
        check()
    except (AssertionError, IndexError, ValueError):
        return False
    return True


def test_pins_catch_planted_mistakes(monkeypatch):
    """Each mutation is a plausible slip in the oracle; some pin above must fail."""
    good_attend = orc.attend
    good_decode = orc.decode_entries
    good_e4m3 = orc.e4m3fn_to_f64

    def no_rope(q, k, scale, sink):          # contracts only the latent half
        k2 = k.copy()
        k2[:, 512:] = 0
        o, lse = good_attend(q, k2, scale, sink)
        return o, lse

    def sink_ignored(q, k, scale, sink):
        return good_attend(q, k, scale, None)

    def scale_group_32(cache, fmt, ps, slots, kv_scale=1.0):  # wrong UE8M0 group size
        rows = good_decode(cache, fmt, ps, slots, kv_scale)
        if fmt == orc.KV_FP8_UE8M0 and rows.shape[0]:
            rows = rows.copy()
            rows[:, 32:64] *= 2.0
        return rows

    def tensor_scale_on_latent_only(cache, fmt, ps, slots, kv_scale=1.0):
        rows = good_decode(cache, fmt, ps, slots, kv_scale)
        if fmt == orc.KV_FP8_TENSOR and rows.shape[0]:
            rows = rows.copy()
            rows[:, 512:] /= kv_scale
        return rows

    def e4m3_bias8(codes):
        return good_e4m3(codes) / 2.0

    def dropped_term(q, k, scale, sink):       # the last entry of the set never counts
        return good_attend(q, k[:-1], scale, sink)

    def wrong_sign(q, k, scale, sink):         # scores with the sign flipped
        return good_attend(-q, k, scale, sink)

    def value_off_by_64(q, k, scale, sink):    # V read from the wrong 512 dims (64..575)
        k2 = k.copy()
        k2[:, :512] = k[:, 64:]
        o, _ = good_attend(q, k2, scale, sink)
        return o, good_attend(q, k, scale, sink)[1]

    def lse_base2(q, k, scale, sink):          # LSE in log2 instead of the natural log
        o, lse = good_attend(q, k, scale, sink)
        return o, lse / math.log(2.0)

    def only_minus_one(idx_row, index_mode, request, page_table, page_size, num_pages):
        # masks -1 alone: other negative ids wrap through the table's last entries
        idx_row = np.asarray(idx_row, dtype=np.int64)
        pos = np.nonzero(idx_row != -1)[0]
        t = idx_row[pos]
        if index_mode == orc.IDX_GLOBAL:
            return pos, t
        row = np.asarray(page_table, dtype=np.int64)[request]
        return pos, row[t // page_size] * page_size + t % page_size

    def remainder_last(topk, num_splits):      # K // S per chunk, the remainder in the last
        c = topk // num_splits
        return [(i * c, (i + 1) * c if i < num_splits - 1 else topk) for i in range(num_splits)]

    good_merge = orc.merge_partials

    def sink_per_chunk(o_c, lse_c, sinks):     # the sink folded into every chunk's weight
        o_c = np.asarray(o_c, dtype=np.float64)
        lse_c = np.asarray(lse_c, dtype=np.float64)
        if sinks is None:
            return good_merge(o_c, lse_c, sinks)
        sig = np.broadcast_to(np.asarray(sinks, dtype=np.float64), lse_c.shape)
        with np.errstate(invalid="ignore"):
            lse2 = np.logaddexp(lse_c, sig)
        return good_merge(o_c * np.exp(lse_c - lse2)[..., None], lse2, None)

    checks = {
        "no_rope": (lambda: monkeypatch.setattr(orc, "attend", no_rope),
                    lambda: test_one_hot_query_scores_one_dim(575)),
        "sink_ignored": (lambda: monkeypatch.setattr(orc, "attend", sink_ignored),
                         lambda: test_sink_identity(2.0)),
        "scale_group": (lambda: monkeypatch.setattr(orc, "decode_entries", scale_group_32),
                        lambda: test_oracle_matches_brute_force("fp8", 1)),
        "tensor_scale_rope": (lambda: monkeypatch.setattr(orc, "decode_entries",
                                                          tensor_scale_on_latent_only),
                              lambda: test_oracle_matches_brute_force("fp8t", 1)),
        "e4m3_bias": (lambda: monkeypatch.setattr(orc, "e4m3fn_to_f64", e4m3_bias8),
                      test_e4m3fn_all_codes_match_torch),
        "dropped_term": (lambda: monkeypatch.setattr(orc, "attend", dropped_term),
                         lambda: test_oracle_matches_brute_force("bf16", 2)),
        "wrong_sign": (lambda: monkeypatch.setattr(orc, "attend", wrong_sign),
                       lambda: test_oracle_matches_brute_force("fp8", 2)),
        "value_off_by_64": (lambda: monkeypatch.setattr(orc, "attend", value_off_by_64),
                            test_single_entry_is_exact),
        "lse_base2": (lambda: monkeypatch.setattr(orc, "attend", lse_base2),
                      test_single_entry_is_exact),
        "only_minus_one_masked": (lambda: monkeypatch.setattr(orc, "translate", only_minus_one),
                                  test_invalid_ids_are_masked_hand_worked),
        "chunks_remainder_last": (lambda: monkeypatch.setattr(orc, "chunk_bounds", remainder_last),
                                  test_chunk_bounds_by_hand),
        "chunks_remainder_last_partials": (
            lambda: monkeypatch.setattr(orc, "chunk_bounds", remainder_last),
            test_partials_are_the_chunks_of_list_positions),
        "sink_per_chunk": (lambda: monkeypatch.setattr(orc, "merge_partials", sink_per_chunk),
                           lambda: test_split_merge_reproduces_unsplit(3)),
    }
    for name, (plant, check) in checks.items():
        plant()
        assert not _run_pin(check), f"planted mistake {name} went unnoticed"
        monkeypatch.undo()
    # and with nothing planted the same checks pass
    for name, (_, check) in checks.items():
        assert _run_pin(check), name


def test_oracle_package_exports():
    assert oracle.sparse_mla_decode is orc.sparse_mla_decode
