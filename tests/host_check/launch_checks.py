"""Launch marshalling of the host API, run against the CPU-only instrumented build.

    python tests/host_check/launch_checks.py <libsparse_mla_hostcheck.so>

Run by tests/test_host_sanitized.py in a child process under AddressSanitizer and UBSan
(the launchers are stand-ins that record their arguments; no pointer is dereferenced).
Each check calls an entry point with valid arguments and asserts what it asked to launch:
which kernels, in which mode, on which buffers and with which scalar arguments.
"""

from __future__ import annotations

import ctypes
import math
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

from sparse_mla_decode_03_amd import binding as B  # noqa: E402

DECODE, MERGE, GATHER, FILL, STORE, LOGITS, TOPK, TRANSLATE, MERGE_NATIVE = range(9)
LOG2E = 1.4426950408889634
W = 0x100000          # fake workspace base (256-byte aligned); never dereferenced
P = {n: 0x200000 + 0x10000 * i for i, n in enumerate(
    ["q", "kv", "idx", "rr", "pt", "sinks", "out", "lse", "po", "pl"])}


def setup(lib):
    lib.smla_hostcheck_launches.argtypes = [ctypes.c_int]
    lib.smla_hostcheck_launches.restype = ctypes.c_int
    lib.smla_hostcheck_fake_scratch.restype = ctypes.c_uint64
    lib.smla_hostcheck_set_cus.argtypes = [ctypes.c_int]
    lib.smla_hostcheck_last_decode.argtypes = [ctypes.POINTER(ctypes.c_int32 * 13),
                                               ctypes.POINTER(ctypes.c_float * 2),
                                               ctypes.POINTER(ctypes.c_uint64 * 11)]
    lib.smla_hostcheck_last_merge.argtypes = [ctypes.POINTER(ctypes.c_int32 * 3),
                                              ctypes.POINTER(ctypes.c_uint64 * 2)]
    lib.smla_hostcheck_last_merge_scale.restype = ctypes.c_float
    lib.smla_hostcheck_last_balance.argtypes = [ctypes.POINTER(ctypes.c_int32 * 4),
                                                ctypes.POINTER(ctypes.c_uint64 * 10)]


def counts(lib):
    return [lib.smla_hostcheck_launches(k) for k in range(9)]


def last_decode(lib):
    i, f, p = (ctypes.c_int32 * 13)(), (ctypes.c_float * 2)(), (ctypes.c_uint64 * 11)()
    lib.smla_hostcheck_last_decode(ctypes.byref(i), ctypes.byref(f), ctypes.byref(p))
    names = ["R", "H", "K", "S", "chunk", "B", "ps_log2", "num_pages", "num_slots", "max_pages",
             "index_mode", "write_partials", "kv_format"]
    d = dict(zip(names, list(i)))
    d["scale_log2"], d["out_scale"] = f[0], f[1]
    d.update(zip(["q", "kv", "idx", "rr", "pt", "sinks", "out", "lse", "po", "pl", "err"], list(p)))
    return d


def last_balance(lib):
    i, p = (ctypes.c_int32 * 4)(), (ctypes.c_uint64 * 10)()
    lib.smla_hostcheck_last_balance(ctypes.byref(i), ctypes.byref(p))
    return list(i), list(p)


def last_merge(lib):
    i, p = (ctypes.c_int32 * 3)(), (ctypes.c_uint64 * 2)()
    lib.smla_hostcheck_last_merge(ctypes.byref(i), ctypes.byref(p))
    return list(i), list(p)


def prob(**kw):
    base = dict(num_rows=512, num_requests=128, num_heads=128, topk=2048, page_size=64, num_pages=90000,
                max_pages_per_req=2048, kv_format=B.KV_FP8_UE8M0, index_mode=B.IDX_LOGICAL,
                num_splits=0, flags=0, softmax_scale=1 / 24)
    base.update(kw)
    return B.make_problem(**base)


def plan(lib, pr, cus=256):
    pl, ws = B.Plan(), ctypes.c_size_t(0)
    st = lib.sparse_mla_decode_plan(ctypes.byref(pr), cus, ctypes.byref(pl), ctypes.byref(ws))
    assert st == B.OK, st
    return pl, ws.value


def run(lib, pl, ws=None, wsb=0, po=None, pl_=None):
    v = lambda x: None if x is None else ctypes.c_void_p(x)  # noqa: E731
    return lib.sparse_mla_decode_run(ctypes.byref(pl), v(P["q"]), v(P["kv"]), v(P["idx"]), v(P["rr"]),
                                     v(P["pt"]), v(P["sinks"]), v(P["out"]), v(P["lse"]), v(po), v(pl_),
                                     v(ws), ctypes.c_size_t(wsb), None)


def round_up(x, a):
    return (x + a - 1) // a * a


def check_unsplit(lib):
    lib.smla_hostcheck_reset()
    pr = prob()
    pl, ws = plan(lib, pr)
    assert ws == 0 and run(lib, pl) == B.OK
    assert counts(lib) == [1, 0, 0, 0, 0, 0, 0, 0, 0]
    d = last_decode(lib)
    assert (d["R"], d["H"], d["K"], d["S"], d["chunk"], d["B"]) == (512, 128, 2048, 1, 2048, 128)
    assert (d["ps_log2"], d["num_pages"], d["num_slots"], d["max_pages"]) == (6, 90000, 90000 * 64, 2048)
    assert (d["index_mode"], d["write_partials"], d["kv_format"]) == (0, 0, B.KV_FP8_UE8M0)
    assert math.isclose(d["scale_log2"], LOG2E / 24, rel_tol=1e-6) and d["out_scale"] == 1.0
    for n in ("q", "kv", "idx", "rr", "pt", "sinks", "out", "lse"):
        assert d[n] == P[n], n
    assert d["po"] == d["pl"] == d["err"] == 0


def check_split_merge(lib):
    lib.smla_hostcheck_reset()
    R, S, H = 2, 8, 128
    pl, ws = plan(lib, prob(num_rows=R, num_requests=2, num_splits=S, kv_format=B.KV_BF16))
    # the decode's own format: O of whole 32-head groups, then (max, sum) per head
    po_bytes = R * S * H * 512 * 4
    assert ws == round_up(po_bytes, 256) + round_up(R * S * H * 8, 256)
    assert run(lib, pl, ws=W, wsb=ws) == B.OK
    assert counts(lib) == [1, 0, 0, 0, 0, 0, 0, 0, 1]
    d = last_decode(lib)
    assert (d["S"], d["chunk"], d["write_partials"], d["kv_format"]) == (S, 256, 2, B.KV_BF16)
    assert d["po"] == W and d["pl"] == W + round_up(po_bytes, 256) and d["out"] == 0
    (mr, ms, mh), (mpo, mpl) = last_merge(lib)
    assert (mr, ms, mh) == (R, S, H) and (mpo, mpl) == (d["po"], d["pl"])
    assert lib.smla_hostcheck_last_merge_scale() == 1.0
    # 16 heads fill half of one 32-head group: the O blocks cover the whole group
    pl, ws = plan(lib, prob(num_rows=3, num_requests=3, num_heads=16, num_splits=4))
    assert ws == round_up(3 * 4 * 32 * 512 * 4, 256) + round_up(3 * 4 * 16 * 8, 256)


def check_partials_only(lib):
    lib.smla_hostcheck_reset()
    pl, ws = plan(lib, prob(num_rows=3, num_requests=3, num_splits=4, flags=B.F_PARTIALS_ONLY))
    assert ws == 0
    assert run(lib, pl, po=P["po"], pl_=P["pl"]) == B.OK
    assert counts(lib) == [1, 0, 0, 0, 0, 0, 0, 0, 0]
    d = last_decode(lib)
    assert d["write_partials"] == 1 and (d["po"], d["pl"]) == (P["po"], P["pl"]) and d["out"] == 0


def check_index_check(lib):
    lib.smla_hostcheck_reset()
    pl, ws = plan(lib, prob(flags=B.F_CHECK_INDICES))
    assert ws == 256 and run(lib, pl, ws=W, wsb=ws) == B.OK
    assert counts(lib)[:4] == [1, 0, 0, 1]           # the error word is filled first
    assert last_decode(lib)["err"] == W
    rp = (ctypes.c_int32 * 2)()
    assert lib.sparse_mla_read_index_error(ctypes.byref(pl), ctypes.c_void_p(W), ctypes.byref(rp), None) == B.OK
    assert list(rp) == [-1, -1]                      # the stand-in copy reports no bad index


def check_tensor_fp8_scales(lib):
    lib.smla_hostcheck_reset()
    pl, _ = plan(lib, prob(kv_format=B.KV_FP8_TENSOR, kv_scale=1 / 64))
    assert run(lib, pl) == B.OK
    d = last_decode(lib)
    assert math.isclose(d["scale_log2"], LOG2E / 24 / 64, rel_tol=1e-6)
    assert d["out_scale"] == 1 / 64 and d["kv_format"] == B.KV_FP8_TENSOR
    # split: the merge of the decode's own format applies the value scale
    pl, ws = plan(lib, prob(num_rows=2, num_requests=2, kv_format=B.KV_FP8_TENSOR, kv_scale=1 / 64,
                            num_splits=4))
    assert run(lib, pl, ws=W, wsb=ws) == B.OK
    assert lib.smla_hostcheck_last_merge_scale() == 1 / 64


def check_global_mode(lib):
    lib.smla_hostcheck_reset()
    pl, _ = plan(lib, prob(index_mode=B.IDX_GLOBAL))
    v = ctypes.c_void_p
    st = lib.sparse_mla_decode_run(ctypes.byref(pl), v(P["q"]), v(P["kv"]), v(P["idx"]), None, None, None,
                                   v(P["out"]), None, None, None, None, ctypes.c_size_t(0), None)
    assert st == B.OK
    d = last_decode(lib)
    assert d["index_mode"] == 1 and d["B"] == 0 and d["max_pages"] == 0 and d["rr"] == d["pt"] == 0


def check_noalloc(lib):
    lib.smla_hostcheck_reset()
    R, S, H = 2, 4, 64
    pl, ws = plan(lib, prob(num_rows=R, num_requests=2, num_heads=H, num_splits=S))
    assert 0 < ws <= B.NOALLOC_SCRATCH_BYTES
    v = ctypes.c_void_p
    for _ in range(2):                                # the second call reuses the looked-up address
        st = lib.sparse_mla_decode_run_noalloc(ctypes.byref(pl), v(P["q"]), v(P["kv"]), v(P["idx"]), v(P["rr"]),
                                               v(P["pt"]), None, v(P["out"]), v(P["lse"]), None)
        assert st == B.OK
    assert counts(lib) == [2, 0, 0, 0, 0, 0, 0, 0, 2]
    d = last_decode(lib)
    base = lib.smla_hostcheck_fake_scratch()
    assert d["po"] == base and d["pl"] == base + round_up(R * S * H * 512 * 4, 256)
    assert d["write_partials"] == 2
    # an unsplit plan needs no scratch and writes the output directly
    lib.smla_hostcheck_reset()
    pl, ws = plan(lib, prob())
    st = lib.sparse_mla_decode_run_noalloc(ctypes.byref(pl), v(P["q"]), v(P["kv"]), v(P["idx"]), v(P["rr"]),
                                           v(P["pt"]), None, v(P["out"]), v(P["lse"]), None)
    assert st == B.OK and counts(lib) == [1, 0, 0, 0, 0, 0, 0, 0, 0] and last_decode(lib)["out"] == P["out"]


def check_balance_rows(lib):
    lib.smla_hostcheck_reset()
    R, S, H = 600, 2, 64
    # counts [R], split counts [R], jobs [R * S] and the job count follow the split partials
    pl, ws = plan(lib, prob(num_rows=R, num_requests=R, num_heads=H, num_splits=S, flags=B.F_BALANCE_ROWS))
    parts = round_up(R * S * H * 512 * 4, 256) + round_up(R * S * H * 8, 256)
    assert ws == parts + round_up((2 * R + R * S + 1) * 4, 256)
    assert run(lib, pl, ws=W, wsb=ws) == B.OK
    assert lib.smla_hostcheck_launches(9) == 1 and counts(lib) == [1, 0, 0, 0, 0, 0, 0, 0, 1]
    (br, bk, bs, slots), p = last_balance(lib)
    assert (br, bk, bs, slots) == (R, 2048, S, 2 * 256) and p[0] == P["idx"]
    bc = W + parts
    assert p[1:5] == [bc, bc + 4 * R, bc + 8 * R, bc + 8 * R + 4 * R * S]
    assert p[5:9] == p[1:5] and p[9] == p[2]          # the decode and the merge see the same lists
    d = last_decode(lib)
    assert d["write_partials"] == 2 and d["po"] == W and d["out"] == P["out"] and d["lse"] == P["lse"]
    # unsplit: the lists alone, in a workspace of their own; four-wave rows take one slot per CU
    lib.smla_hostcheck_reset()
    pl, ws = plan(lib, prob(num_rows=R, num_requests=R, num_splits=1, flags=B.F_BALANCE_ROWS))
    assert ws == round_up((3 * R + 1) * 4, 256)
    assert run(lib, pl, ws=W, wsb=ws) == B.OK
    assert lib.smla_hostcheck_launches(9) == 1 and last_decode(lib)["out"] == P["out"]
    (_, _, bs, slots), p = last_balance(lib)
    assert (bs, slots) == (1, 256) and p[5:9] == [W, W + 4 * R, W + 8 * R, W + 12 * R]
    assert counts(lib)[8] == 0
    # without the flag the decode gets no lists and the merge no split counts
    lib.smla_hostcheck_reset()
    pl, ws = plan(lib, prob(num_rows=R, num_requests=R, num_heads=H, num_splits=S))
    assert run(lib, pl, ws=W, wsb=ws) == B.OK and lib.smla_hostcheck_launches(9) == 0
    assert last_balance(lib)[1][5:] == [0, 0, 0, 0, 0] and last_decode(lib)["out"] == 0
    # balancing changes the positional chunks the documented partials are defined by
    pr = prob(num_rows=4, num_requests=4, num_splits=2, flags=B.F_BALANCE_ROWS | B.F_PARTIALS_ONLY)
    pl_, wsb = B.Plan(), ctypes.c_size_t(0)
    assert lib.sparse_mla_decode_plan(ctypes.byref(pr), 256, ctypes.byref(pl_), ctypes.byref(wsb)) == B.ERR_UNSUPPORTED
    # jobs are coded as row | split << 24
    pr = prob(num_rows=1 << 24, num_requests=4, num_splits=1, flags=B.F_BALANCE_ROWS)
    assert lib.sparse_mla_decode_plan(ctypes.byref(pr), 256, ctypes.byref(pl_), ctypes.byref(wsb)) == B.ERR_BAD_SHAPE


def check_planner_cu_count(lib):
    # num_cus <= 0 asks the runtime (the stand-in reports 304 CUs): 32 rows -> ceil(304 / 32)
    lib.smla_hostcheck_set_cus(304)
    pl, _ = plan(lib, prob(num_rows=32, num_requests=32), cus=0)
    assert lib.sparse_mla_plan_num_splits(ctypes.byref(pl)) == 10
    pl, _ = plan(lib, prob(num_rows=32, num_requests=32), cus=64)
    assert lib.sparse_mla_plan_num_splits(ctypes.byref(pl)) == 2
    # top-k beyond one workgroup's positions needs splits even with many rows
    pl, _ = plan(lib, prob(topk=5000), cus=256)
    assert lib.sparse_mla_plan_num_splits(ctypes.byref(pl)) == 3


def check_other_entry_points(lib):
    lib.smla_hostcheck_reset()
    v = ctypes.c_void_p
    assert lib.sparse_mla_merge_partials(v(W), v(W + 0x1000), 4, 3, 16, None, v(P["out"]), None, None) == B.OK
    assert last_merge(lib) == ([4, 3, 16], [W, W + 0x1000])
    assert lib.sparse_mla_gather_debug(v(P["kv"]), 1, 64, 10, v(P["idx"]), 3, v(P["out"]), None) == B.OK
    assert lib.sparse_mla_cache_store(v(P["q"]), v(P["q"]), v(P["idx"]), 4, B.KV_FP8_UE8M0, 64, 10,
                                      v(P["kv"]), None) == B.OK
    assert lib.sparse_mla_indexer_logits(v(P["q"]), v(W), v(P["kv"]), v(P["rr"]), v(P["pt"]), 4, 2, 64, 64,
                                         100, 8, 512, v(P["out"]), None) == B.OK
    assert lib.sparse_mla_indexer_topk(v(P["out"]), v(P["rr"]), 3, 64, 16, v(P["idx"]), None) == B.OK
    assert lib.sparse_mla_translate_indices(v(P["idx"]), v(P["rr"]), v(P["pt"]), 4, 16, 2, 8, 64, 100,
                                            v(P["out"]), None) == B.OK
    assert counts(lib) == [0, 1, 1, 0, 1, 1, 1, 1, 0]


def main(path):
    lib = B.load_library(path)
    setup(lib)
    checks = [check_unsplit, check_split_merge, check_partials_only, check_index_check,
              check_tensor_fp8_scales, check_global_mode, check_noalloc, check_balance_rows,
              check_planner_cu_count, check_other_entry_points]
    for c in checks:
        c(lib)
        print("ok", c.__name__, flush=True)
    print("all launch checks passed")


if __name__ == "__main__":
    main(sys.argv[1])
