"""Host-only checks of the C ABI: the library loads without a GPU, exports every
function the header declares, and rejects bad arguments with the documented status
before touching the device.  No kernel is launched here."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from sparse_mla_decode_03_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_mla.h")


# The sanitizer test (test_host_sanitized.py) runs this module again in a child process
# against the CPU-only, ASan/UBSan-instrumented build of the same host code.
LIB = os.environ.get("SMLA_HOST_CHECK_LIB", B.LIB_PATH)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.skip("library not built (python -m sparse_mla_decode_03_amd.build)")
    return B.load_library(LIB)


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(sparse_mla_[a-z_0-9]+)\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("sparse_mla_decode_plan", "sparse_mla_decode_run", "sparse_mla_merge_partials"):
        assert n in names
    assert set(names) == set(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.sparse_mla_version() == 100


def test_status_strings(lib):
    for s in range(8):
        assert B.status_string(s)
    assert B.status_string(B.ERR_WORKSPACE_TOO_SMALL).startswith("workspace")
    assert B.status_string(99) == "unknown status"


def _prob(**kw):
    base = dict(num_rows=4, num_requests=2, num_heads=64, topk=2048, page_size=64, num_pages=100,
                max_pages_per_req=50, kv_format=B.KV_FP8_UE8M0, index_mode=B.IDX_LOGICAL,
                num_splits=0, flags=0, softmax_scale=1 / 24)
    base.update(kw)
    return B.make_problem(**base)


def _plan_status(lib, prob, cus=256):
    p = B.Plan()
    ws = ctypes.c_size_t(0)
    st = lib.sparse_mla_decode_plan(ctypes.byref(prob), cus, ctypes.byref(p), ctypes.byref(ws))
    return st, p, ws.value


@pytest.mark.parametrize("kw,status", [
    (dict(num_heads=8), B.ERR_UNSUPPORTED),
    (dict(num_heads=24), B.ERR_UNSUPPORTED),
    (dict(num_heads=144), B.ERR_UNSUPPORTED),
    (dict(topk=2046), B.ERR_MISALIGNED),
    (dict(topk=0), B.ERR_BAD_SHAPE),
    (dict(num_rows=-1), B.ERR_BAD_SHAPE),
    (dict(page_size=48), B.ERR_BAD_SHAPE),
    (dict(page_size=2048), B.ERR_BAD_SHAPE),
    (dict(page_size=1), B.ERR_UNSUPPORTED),
    (dict(num_pages=0), B.ERR_BAD_SHAPE),
    (dict(num_pages=1 << 26, page_size=64), B.ERR_BAD_SHAPE),
    (dict(kv_format=7), B.ERR_UNSUPPORTED),
    (dict(index_mode=3), B.ERR_UNSUPPORTED),
    (dict(flags=8), B.ERR_UNSUPPORTED),
    (dict(flags=B.F_BALANCE_ROWS | B.F_PARTIALS_ONLY, num_splits=2), B.ERR_UNSUPPORTED),
    (dict(num_requests=0), B.ERR_BAD_SHAPE),
    (dict(max_pages_per_req=0), B.ERR_BAD_SHAPE),
    (dict(num_splits=-2), B.ERR_BAD_SHAPE),
    (dict(num_splits=300), B.ERR_BAD_SHAPE),
    (dict(topk=8, num_splits=9), B.ERR_BAD_SHAPE),
    (dict(num_splits=1, topk=4096), B.ERR_UNSUPPORTED),
    (dict(softmax_scale=float("inf")), B.ERR_BAD_SHAPE),
])
def test_plan_rejects_bad_problems(lib, kw, status):
    st, _, _ = _plan_status(lib, _prob(**kw))
    assert st == status


def test_plan_null_args(lib):
    p = B.Plan()
    ws = ctypes.c_size_t(0)
    prob = _prob()
    assert lib.sparse_mla_decode_plan(None, 256, ctypes.byref(p), ctypes.byref(ws)) == B.ERR_NULL_ARG
    assert lib.sparse_mla_decode_plan(ctypes.byref(prob), 256, None, ctypes.byref(ws)) == B.ERR_NULL_ARG
    assert lib.sparse_mla_decode_plan(ctypes.byref(prob), 256, ctypes.byref(p), None) == B.ERR_NULL_ARG


def test_plan_splits_and_workspace(lib):
    # many rows: no split, no workspace
    st, p, ws = _plan_status(lib, _prob(num_rows=512, num_heads=128))
    assert st == B.OK and lib.sparse_mla_plan_num_splits(ctypes.byref(p)) == 1 and ws == 0
    # forced 16 splits over 2 rows: fp32 partials [R,S,H,512] + lse [R,S,H] in the workspace
    st, p, ws = _plan_status(lib, _prob(num_rows=2, num_heads=128, num_splits=16,
                                        kv_format=B.KV_BF16))
    assert st == B.OK and lib.sparse_mla_plan_num_splits(ctypes.byref(p)) == 16
    assert ws >= 2 * 16 * 128 * 512 * 4 + 2 * 16 * 128 * 4
    # few rows: the planner splits, with chunks of at least 128 positions
    st, p, ws = _plan_status(lib, _prob(num_rows=32))
    s = lib.sparse_mla_plan_num_splits(ctypes.byref(p))
    assert st == B.OK and 1 < s <= 2048 // 128
    # a short list of two tiles over few rows splits in two; one tile does not split
    st, p, ws = _plan_status(lib, _prob(num_rows=1, topk=64))
    assert st == B.OK and lib.sparse_mla_plan_num_splits(ctypes.byref(p)) == 2
    st, p, ws = _plan_status(lib, _prob(num_rows=1, topk=32))
    assert st == B.OK and lib.sparse_mla_plan_num_splits(ctypes.byref(p)) == 1 and ws == 0
    # partials-only keeps the partials out of the workspace
    st, p, ws = _plan_status(lib, _prob(num_rows=2, num_splits=4, flags=B.F_PARTIALS_ONLY))
    assert st == B.OK and ws == 0
    # index checking needs one word
    st, p, ws = _plan_status(lib, _prob(num_rows=512, flags=B.F_CHECK_INDICES))
    assert st == B.OK and ws == 256
    # many ragged rows: two splits by the round rule; balanced rows may split in two, each
    # row by its own count
    st, p, ws = _plan_status(lib, _prob(num_rows=627, num_heads=64))
    assert st == B.OK and lib.sparse_mla_plan_num_splits(ctypes.byref(p)) == 2
    st, p, ws = _plan_status(lib, _prob(num_rows=627, num_heads=64, flags=B.F_BALANCE_ROWS))
    assert st == B.OK and lib.sparse_mla_plan_num_splits(ctypes.byref(p)) == 2
    # balanced rows: a count, a split count and a job per row, and the job count (the
    # header's flag value is the binding's)
    st, p, ws = _plan_status(lib, _prob(num_rows=600, num_splits=1, flags=B.F_BALANCE_ROWS))
    assert st == B.OK and ws == 7424
    assert "SMLA_F_BALANCE_ROWS = 4" in open(HEADER).read() and B.F_BALANCE_ROWS == 4
    # plans are data independent and deterministic
    a = _plan_status(lib, _prob(num_rows=32))
    b = _plan_status(lib, _prob(num_rows=32))
    assert bytes(a[1].opaque) == bytes(b[1].opaque) and a[2] == b[2]
    assert lib.sparse_mla_plan_num_splits(None) == -1


FAKE = 0x10000  # never dereferenced: every call below fails validation first


def _run(lib, plan, q=FAKE, kv=FAKE, idx=FAKE, rr=FAKE, pt=FAKE, sinks=None, out=FAKE, lse=None,
         po=None, pl=None, ws=None, wsb=0):
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.sparse_mla_decode_run(ctypes.byref(plan), v(q), v(kv), v(idx), v(rr), v(pt), v(sinks),
                                     v(out), v(lse), v(po), v(pl), v(ws), ctypes.c_size_t(wsb), None)


def test_run_validation_before_launch(lib):
    st, plan, _ = _plan_status(lib, _prob(num_rows=512))
    assert st == B.OK
    bad = B.Plan()
    assert _run(lib, bad) == B.ERR_BAD_PLAN
    assert _run(lib, plan, q=None) == B.ERR_NULL_ARG
    assert _run(lib, plan, rr=None) == B.ERR_NULL_ARG
    assert _run(lib, plan, out=None) == B.ERR_NULL_ARG
    assert _run(lib, plan, q=FAKE + 8) == B.ERR_MISALIGNED
    assert _run(lib, plan, idx=FAKE + 4) == B.ERR_MISALIGNED
    assert _run(lib, plan, lse=FAKE + 2) == B.ERR_MISALIGNED
    # split plan needs its workspace
    st, plan2, wsb = _plan_status(lib, _prob(num_rows=2, num_splits=8))
    assert wsb > 0
    assert _run(lib, plan2) == B.ERR_NULL_ARG
    assert _run(lib, plan2, ws=FAKE, wsb=wsb - 1) == B.ERR_WORKSPACE_TOO_SMALL
    assert _run(lib, plan2, ws=FAKE + 16, wsb=wsb) == B.ERR_MISALIGNED
    # partials-only requires the partial buffers
    st, plan3, _ = _plan_status(lib, _prob(num_rows=2, num_splits=4, flags=B.F_PARTIALS_ONLY))
    assert _run(lib, plan3, out=None) == B.ERR_NULL_ARG
    # GLOBAL mode does not need row_req / page_table
    st, plan4, _ = _plan_status(lib, _prob(num_rows=0, index_mode=B.IDX_GLOBAL))
    assert _run(lib, plan4, rr=None, pt=None) == B.OK          # zero rows: nothing launched


def test_merge_and_gather_validation(lib):
    v = ctypes.c_void_p
    assert lib.sparse_mla_merge_partials(v(FAKE), v(FAKE), 4, 0, 8, None, v(FAKE), None, None) == B.ERR_BAD_SHAPE
    assert lib.sparse_mla_merge_partials(v(FAKE), v(FAKE), 4, 300, 8, None, v(FAKE), None, None) == B.ERR_BAD_SHAPE
    assert lib.sparse_mla_merge_partials(None, v(FAKE), 4, 2, 8, None, v(FAKE), None, None) == B.ERR_NULL_ARG
    assert lib.sparse_mla_merge_partials(v(FAKE + 4), v(FAKE), 4, 2, 8, None, v(FAKE), None, None) == B.ERR_MISALIGNED
    assert lib.sparse_mla_merge_partials(v(FAKE), v(FAKE), 0, 2, 8, None, v(FAKE), None, None) == B.OK
    assert lib.sparse_mla_gather_debug(v(FAKE), 5, 64, 10, v(FAKE), 3, v(FAKE), None) == B.ERR_UNSUPPORTED
    assert lib.sparse_mla_gather_debug(v(FAKE), 1, 48, 10, v(FAKE), 3, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert lib.sparse_mla_gather_debug(v(FAKE), 1, 64, 10, None, 3, v(FAKE), None) == B.ERR_NULL_ARG
    assert lib.sparse_mla_gather_debug(v(FAKE + 1), 1, 64, 10, v(FAKE), 3, v(FAKE), None) == B.ERR_MISALIGNED
    assert lib.sparse_mla_gather_debug(v(FAKE), 1, 64, 10, v(FAKE), 0, v(FAKE), None) == B.OK


def test_read_index_error_validation(lib):
    st, plan, _ = _plan_status(lib, _prob(num_rows=4))
    rp = (ctypes.c_int32 * 2)()
    assert lib.sparse_mla_read_index_error(ctypes.byref(B.Plan()), ctypes.c_void_p(FAKE), ctypes.byref(rp), None) == B.ERR_BAD_PLAN
    assert lib.sparse_mla_read_index_error(ctypes.byref(plan), None, ctypes.byref(rp), None) == B.ERR_NULL_ARG
    assert lib.sparse_mla_read_index_error(ctypes.byref(plan), ctypes.c_void_p(FAKE), ctypes.byref(rp), None) == B.ERR_UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 16, 576, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.sparse_mla_decode(q, torch.zeros(1, 1, dtype=torch.uint8), torch.zeros(1, 4, dtype=torch.int32),
                            None, None, None, "bf16", 64, 1.0)


def test_cache_store_validation(lib):
    v = ctypes.c_void_p
    cs = lib.sparse_mla_cache_store
    # (latent, rope, slots, n, kv_format, page_size, num_pages, kv_cache, stream)
    assert cs(v(FAKE), v(FAKE), v(FAKE), 4, 7, 64, 10, v(FAKE), None) == B.ERR_UNSUPPORTED
    assert cs(v(FAKE), v(FAKE), v(FAKE), 4, B.KV_FP8_UE8M0, 1, 10, v(FAKE), None) == B.ERR_UNSUPPORTED
    assert cs(v(FAKE), v(FAKE), v(FAKE), -1, B.KV_BF16, 64, 10, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert cs(v(FAKE), v(FAKE), v(FAKE), 4, B.KV_BF16, 48, 10, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert cs(v(FAKE), v(FAKE), v(FAKE), 4, B.KV_BF16, 64, 0, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert cs(None, v(FAKE), v(FAKE), 4, B.KV_BF16, 64, 10, v(FAKE), None) == B.ERR_NULL_ARG
    assert cs(v(FAKE), v(FAKE), v(FAKE), 4, B.KV_BF16, 64, 10, None, None) == B.ERR_NULL_ARG
    assert cs(v(FAKE + 8), v(FAKE), v(FAKE), 4, B.KV_BF16, 64, 10, v(FAKE), None) == B.ERR_MISALIGNED
    assert cs(v(FAKE), v(FAKE), v(FAKE + 2), 4, B.KV_BF16, 64, 10, v(FAKE), None) == B.ERR_MISALIGNED
    # zero tokens: nothing launched, pointers not checked
    assert cs(None, None, None, 0, B.KV_FP8_UE8M0, 64, 10, None, None) == B.OK


def test_indexer_validation(lib):
    v = ctypes.c_void_p
    il = lib.sparse_mla_indexer_logits
    # (q, weights, keys, row_len, page_table, B, next_n, heads, page_size, num_pages,
    #  max_pages, width, logits, stream)
    args = [v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), 4, 2, 64, 64, 100, 8, 512, v(FAKE), None]

    def call(**kw):
        a = list(args)
        names = ["q", "w", "k", "len", "pt", "B", "nn", "H", "ps", "np", "mp", "width", "out", "st"]
        for key, val in kw.items():
            a[names.index(key)] = val
        return il(*a)

    assert call(H=32) == B.ERR_UNSUPPORTED
    assert call(ps=16) == B.ERR_UNSUPPORTED
    assert call(nn=5) == B.ERR_UNSUPPORTED and call(nn=0) == B.ERR_UNSUPPORTED
    assert call(width=500) == B.ERR_BAD_SHAPE and call(width=0) == B.ERR_BAD_SHAPE
    assert call(mp=7) == B.ERR_BAD_SHAPE            # the table must cover the width
    # a row's bytes stay below 2^31: width at most 2^28 positions
    assert call(width=(1 << 28) + 64, mp=(1 << 22) + 1) == B.ERR_BAD_SHAPE
    assert call(np=0) == B.ERR_BAD_SHAPE and call(B=-1) == B.ERR_BAD_SHAPE
    assert call(q=None) == B.ERR_NULL_ARG and call(out=None) == B.ERR_NULL_ARG
    assert call(w=v(FAKE + 4)) == B.ERR_MISALIGNED and call(len=v(FAKE + 2)) == B.ERR_MISALIGNED
    assert call(B=0, q=None, out=None) == B.OK      # nothing to do
    tk = lib.sparse_mla_indexer_topk
    # (logits, row_len, rows, width, topk, indices, stream)
    assert tk(v(FAKE), v(FAKE), 3, 0, 16, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert tk(v(FAKE), v(FAKE), 3, 64, 0, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert tk(v(FAKE), v(FAKE), -1, 64, 16, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert tk(None, v(FAKE), 3, 64, 16, v(FAKE), None) == B.ERR_NULL_ARG
    assert tk(v(FAKE), v(FAKE), 3, 64, 16, v(FAKE + 1), None) == B.ERR_MISALIGNED
    assert tk(v(FAKE + 4), v(FAKE), 3, 64, 16, v(FAKE), None) == B.ERR_MISALIGNED
    assert tk(v(FAKE), v(FAKE), 3, 66, 16, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert tk(None, None, 0, 64, 16, None, None) == B.OK


def test_translate_validation(lib):
    v = ctypes.c_void_p
    tr = lib.sparse_mla_translate_indices
    # (indices, row_req, page_table, rows, topk, num_requests, max_pages, page_size, num_pages, slots, stream)
    assert tr(v(FAKE), v(FAKE), v(FAKE), 4, 16, 2, 8, 48, 100, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert tr(v(FAKE), v(FAKE), v(FAKE), 4, 0, 2, 8, 64, 100, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert tr(v(FAKE), v(FAKE), v(FAKE), -1, 16, 2, 8, 64, 100, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert tr(v(FAKE), v(FAKE), v(FAKE), 4, 16, 2, 8, 64, 0, v(FAKE), None) == B.ERR_BAD_SHAPE
    assert tr(None, v(FAKE), v(FAKE), 4, 16, 2, 8, 64, 100, v(FAKE), None) == B.ERR_NULL_ARG
    assert tr(v(FAKE), v(FAKE), v(FAKE), 4, 16, 2, 8, 64, 100, v(FAKE + 2), None) == B.ERR_MISALIGNED
    assert tr(None, None, None, 0, 16, 2, 8, 64, 100, None, None) == B.OK


def _run_noalloc(lib, plan, q=FAKE, kv=FAKE, idx=FAKE, rr=FAKE, pt=FAKE, sinks=None, out=FAKE, lse=None):
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.sparse_mla_decode_run_noalloc(ctypes.byref(plan), v(q), v(kv), v(idx), v(rr), v(pt),
                                             v(sinks), v(out), v(lse), None)


def test_noalloc_run_validation_before_launch(lib):
    """The allocation-free entry point: plans beyond its scratch, flags it cannot serve and
    bad pointers are all refused before any device call."""
    assert _run_noalloc(lib, B.Plan()) == B.ERR_BAD_PLAN
    # 64 rows x 16 splits x 128 heads of fp32 partials: 268 MB, beyond the 16 MiB scratch
    st, big, ws = _plan_status(lib, _prob(num_rows=64, num_heads=128, num_splits=16))
    assert st == B.OK and ws > B.NOALLOC_SCRATCH_BYTES
    assert _run_noalloc(lib, big) == B.ERR_WORKSPACE_TOO_SMALL
    for flag in (B.F_PARTIALS_ONLY, B.F_CHECK_INDICES):
        st, p, _ = _plan_status(lib, _prob(num_rows=2, num_splits=4, flags=flag))
        assert st == B.OK and _run_noalloc(lib, p) == B.ERR_UNSUPPORTED
    # a split plan that fits: argument errors come back before the scratch is looked up
    st, p, ws = _plan_status(lib, _prob(num_rows=2, num_splits=4))
    assert st == B.OK and 0 < ws <= B.NOALLOC_SCRATCH_BYTES
    assert _run_noalloc(lib, p, q=None) == B.ERR_NULL_ARG
    assert _run_noalloc(lib, p, rr=None) == B.ERR_NULL_ARG
    assert _run_noalloc(lib, p, out=None) == B.ERR_NULL_ARG
    assert _run_noalloc(lib, p, q=FAKE + 8) == B.ERR_MISALIGNED
    assert _run_noalloc(lib, p, lse=FAKE + 2) == B.ERR_MISALIGNED
    # zero rows: nothing to do
    st, z, _ = _plan_status(lib, _prob(num_rows=0))
    assert st == B.OK and _run_noalloc(lib, z, q=None, kv=None, idx=None, out=None) == B.OK
