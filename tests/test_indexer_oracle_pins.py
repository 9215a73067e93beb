"""Pins of the indexer oracle (FP8 paged MQA logits and the top-k selection) against
things other than itself: pure-Python loops over torch's own e4m3fn decode, a hand-worked
page, positive homogeneity and page relocation, and numpy's argsort for the selection.
CPU only."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import indexer_oracle as io
from sparse_mla_decode_03_amd import workloads as W


def _torch_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _pages(codes: np.ndarray, scales: np.ndarray, ps: int) -> np.ndarray:
    """Pack keys [n, 128] / scales [n] (n a multiple of ps) into region-split pages."""
    n = codes.shape[0]
    pages = np.zeros((n // ps, 132 * ps), dtype=np.uint8)
    for t in range(n):
        p, r = divmod(t, ps)
        pages[p, r * 128:(r + 1) * 128] = codes[t]
        pages[p, 128 * ps + 4 * r: 128 * ps + 4 * r + 4] = np.array([scales[t]], dtype="<f4").view(np.uint8)
    return pages


def _brute(q_codes, weights, codes, scales, row_req, row_len, page_table, ps, width):
    qv = _torch_e4m3(q_codes)
    kv = _torch_e4m3(codes)
    out = np.full((q_codes.shape[0], width), -math.inf)
    for r in range(q_codes.shape[0]):
        b = int(row_req[r])
        for t in range(int(row_len[r])):
            slot = int(page_table[b, t // ps]) * ps + t % ps
            terms = []
            for h in range(q_codes.shape[1]):
                dot = math.fsum(float(qv[r, h, d]) * float(kv[slot, d]) for d in range(128))
                terms.append(float(weights[r, h]) * max(0.0, float(scales[slot]) * dot))
            out[r, t] = math.fsum(terms)
    return out


def _random_case(seed, ps=4, B=2, H=3, n_rows=(2, 1), ctx=(9, 6)):
    rng = np.random.default_rng(seed)
    pages_per = [-(-c // ps) for c in ctx]
    npages = sum(pages_per) + 2
    codes = rng.integers(0, 256, (npages * ps, 128), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x11          # no NaN codes
    scales = rng.uniform(0.01, 3.0, npages * ps).astype(np.float32)
    perm = rng.permutation(npages)
    page_table = np.full((B, max(pages_per)), -1, dtype=np.int32)
    s = 0
    for b in range(B):
        page_table[b, :pages_per[b]] = perm[s:s + pages_per[b]]
        s += pages_per[b]
    row_req = np.repeat(np.arange(B), n_rows)
    row_len = np.array([ctx[b] - (n_rows[b] - 1 - i) for b in range(B) for i in range(n_rows[b])])
    R = len(row_req)
    q = rng.integers(0, 256, (R, H, 128), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x22
    w = rng.standard_normal((R, H)).astype(np.float32)
    return q, w, codes, scales, _pages(codes, scales, ps), row_req, row_len, page_table


@pytest.mark.parametrize("seed", [1, 2])
def test_logits_match_loops_over_torch_decode(seed):
    ps, width = 4, 12
    q, w, codes, scales, pages, row_req, row_len, pt = _random_case(seed)
    want = _brute(q, w, codes, scales, row_req, row_len, pt, ps, width)
    got = io.indexer_logits(q, w, pages, ps, row_req, row_len, pt, width)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got))
    assert np.allclose(got[fin], want[fin], rtol=1e-12, atol=1e-9)


def test_hand_worked_page():
    # two heads; q head 0 = (1, 0, ...), head 1 = (0, 2, 0, ...); weights (1, -0.5)
    # key 0 = 2.0 * (0.5, -1, 0, ...): head 0 relu(2 * 0.5) = 1, head 1 relu(2 * -2) = 0
    #   -> 1 * 1 + (-0.5) * 0 = 1
    # key 1 = 0.5 * (-1, 1, 0, ...): head 0 relu(0.5 * -1) = 0, head 1 relu(0.5 * 2) = 1
    #   -> 0 + (-0.5) * 1 = -0.5
    q = np.zeros((1, 2, 128), dtype=np.uint8)
    q[0, 0, 0] = 0x38      # 1.0
    q[0, 1, 1] = 0x40      # 2.0
    codes = np.zeros((2, 128), dtype=np.uint8)
    codes[0, 0], codes[0, 1] = 0x30, 0xB8      # 0.5, -1.0
    codes[1, 0], codes[1, 1] = 0xB8, 0x38      # -1.0, 1.0
    pages = _pages(codes, np.array([2.0, 0.5], dtype=np.float32), 2)
    got = io.indexer_logits(q, np.array([[1.0, -0.5]]), pages, 2, [0], [2], np.array([[0]]), 3)
    assert got[0, 0] == 1.0 and got[0, 1] == -0.5 and got[0, 2] == -math.inf


def test_homogeneity_relu_and_relocation():
    ps, width = 4, 12
    q, w, codes, scales, pages, row_req, row_len, pt = _random_case(5)
    base = io.indexer_logits(q, w, pages, ps, row_req, row_len, pt, width)
    fin = np.isfinite(base)
    # doubling every weight doubles every logit
    assert np.allclose(io.indexer_logits(q, 2 * w, pages, ps, row_req, row_len, pt, width)[fin],
                       2 * base[fin], rtol=1e-14)
    # doubling every key scale doubles every logit (the ReLU is positively homogeneous)
    pages2 = _pages(codes, 2 * scales, ps)
    assert np.allclose(io.indexer_logits(q, w, pages2, ps, row_req, row_len, pt, width)[fin],
                       2 * base[fin], rtol=1e-14)
    # negating the queries: each head then contributes relu(-dot) instead of relu(dot), so
    # the two results sum to sum_h w_h |dot_h|, checked by the loop reference with |.|
    neg = q ^ np.uint8(0x80)
    a = io.indexer_logits(neg, w, pages, ps, row_req, row_len, pt, width)
    qv, kv = _torch_e4m3(q), _torch_e4m3(codes)
    r, t = 0, 3
    slot = int(pt[row_req[r], t // ps]) * ps + t % ps
    absum = sum(float(w[r, h]) * abs(float(scales[slot]) * float(qv[r, h] @ kv[slot])) for h in range(q.shape[1]))
    assert math.isclose(a[r, t] + base[r, t], absum, rel_tol=1e-12, abs_tol=1e-9)
    # moving the pages to other places in the pool (and the table with them) changes nothing
    perm = np.random.default_rng(9).permutation(pages.shape[0])
    moved = np.empty_like(pages)
    moved[perm] = pages
    assert np.array_equal(io.indexer_logits(q, w, moved, ps, row_req, row_len, np.where(pt >= 0, perm[pt], -1), width), base)


def test_row_lengths_and_mtp_rows():
    ps, width = 4, 12
    q, w, codes, scales, pages, row_req, row_len, pt = _random_case(3)
    lg = io.indexer_logits(q, w, pages, ps, row_req, row_len, pt, width)
    for r in range(len(row_req)):
        assert np.all(np.isfinite(lg[r, :row_len[r]])) and np.all(lg[r, row_len[r]:] == -math.inf)
    # the two rows of request 0 share their common positions' keys: with the same query
    # and weights their logits agree on the shorter row's positions
    q2, w2 = q.copy(), w.copy()
    q2[1], w2[1] = q2[0], w2[0]
    lg2 = io.indexer_logits(q2, w2, pages, ps, row_req, row_len, pt, width)
    n0 = row_len[0]
    assert np.array_equal(lg2[0, :n0], lg2[1, :n0])


def test_topk_against_argsort_on_distinct_values():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((5, 300))
    lens = np.array([300, 299, 100, 7, 0])
    got = io.indexer_topk(lg, lens, 64)
    for r in range(5):
        n = lens[r]
        want = np.sort(np.argsort(-lg[r, :n], kind="stable")[:min(64, n)])
        assert np.array_equal(got[r, :want.size], want)
        assert np.all(got[r, want.size:] == -1)


def test_topk_ties_go_to_smaller_positions():
    lg = np.array([[5.0, 3.0, 3.0, 1.0, 3.0], [2.0, 2.0, 2.0, 2.0, 2.0]])
    got = io.indexer_topk(lg, [5, 5], 2)
    assert got.tolist() == [[0, 1], [0, 1]]
    got = io.indexer_topk(lg, [5, 3], 3)
    assert got.tolist() == [[0, 1, 2], [0, 1, 2]]
    got = io.indexer_topk(lg, [2, 1], 4)
    assert got.tolist() == [[0, 1, -1, -1], [0, -1, -1, -1]]


def test_generator_layout_is_the_oracle_layout():
    inp = W.make_indexer_inputs(W.INDEXER_WORKLOADS["idx_small"], 2)
    cache = inp.key_cache.numpy()
    slots = io.row_slots(0, 70, inp.page_table.numpy(), 64)
    codes, scales = io.decode_keys(cache, 64, slots)
    # scales are amax/448 of the (unquantized) keys, so the largest code value is 448
    assert np.all(scales > 0)
    assert np.allclose(np.abs(codes).max(axis=1), 448.0)
    assert np.all(inp.row_len.numpy() <= inp.width) and inp.width % 64 == 0


# ---------------------------------------------------------------- planted mistakes

def _passes(check) -> bool:
    try:
        check()
    except AssertionError:
        return False
    return True


def test_pins_catch_planted_indexer_mistakes(monkeypatch):
    """Each mutation is a plausible slip in the indexer oracle; a pin above must fail."""
    good_logits = io.indexer_logits
    good_decode = io.decode_keys

    def mutated_logits(relu=True, reverse_weights=False):
        def f(q_codes, weights, cache, page_size, row_req, row_len, page_table, width, rows=None):
            q_codes = np.asarray(q_codes, dtype=np.uint8)
            w = np.asarray(weights, dtype=np.float64)
            if reverse_weights:
                w = w[:, ::-1]
            rows_ = range(q_codes.shape[0]) if rows is None else list(rows)
            out = np.full((len(rows_), width), -np.inf)
            for i, r in enumerate(rows_):
                n = int(row_len[r])
                if n == 0:
                    continue
                codes, scale = io.decode_keys(cache, page_size,
                                              io.row_slots(int(row_req[r]), n, page_table, page_size))
                dots = scale[None, :] * (io.e4m3fn_to_f64(q_codes[r]) @ codes.T)
                out[i, :n] = w[r] @ (np.maximum(dots, 0.0) if relu else dots)
            return out
        return f

    def no_key_scale(cache, page_size, slots):
        codes, scales = good_decode(cache, page_size, slots)
        return codes, np.ones_like(scales)

    def ties_to_larger(logits, row_len, topk):
        logits = np.asarray(logits, dtype=np.float64)
        out = np.full((logits.shape[0], topk), -1, dtype=np.int64)
        for r in range(logits.shape[0]):
            n = int(row_len[r])
            pos = np.arange(n)
            order = np.lexsort((-pos, -logits[r, :n]))
            take = np.sort(order[:min(topk, n)])
            out[r, :take.size] = take
        return out

    checks = {
        "no_relu": (lambda: monkeypatch.setattr(io, "indexer_logits", mutated_logits(relu=False)),
                    lambda: test_logits_match_loops_over_torch_decode(1)),
        "weights_reversed": (lambda: monkeypatch.setattr(io, "indexer_logits",
                                                         mutated_logits(reverse_weights=True)),
                             lambda: test_logits_match_loops_over_torch_decode(2)),
        "no_key_scale": (lambda: monkeypatch.setattr(io, "decode_keys", no_key_scale),
                         lambda: test_logits_match_loops_over_torch_decode(1)),
        "ties_to_larger_position": (lambda: monkeypatch.setattr(io, "indexer_topk", ties_to_larger),
                                    test_topk_ties_go_to_smaller_positions),
    }
    assert good_logits is io.indexer_logits
    for name, (plant, check) in checks.items():
        plant()
        assert not _passes(check), f"planted mistake {name} went unnoticed"
        monkeypatch.undo()
    for name, (_, check) in checks.items():
        assert _passes(check), name
