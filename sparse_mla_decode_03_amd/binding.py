"""ctypes binding of libsparse_mla.so (C ABI in include/sparse_mla.h).

Argument marshalling only: torch tensors supply device pointers and the current HIP
stream; every step of the decode runs in the library's kernels.  The library must be
built (python -m sparse_mla_decode_03_amd.build); loading fails loudly otherwise.
"""

from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparse_mla.so")

# status codes
OK = 0
ERR_NULL_ARG = 1
ERR_BAD_SHAPE = 2
ERR_UNSUPPORTED = 3
ERR_MISALIGNED = 4
ERR_WORKSPACE_TOO_SMALL = 5
ERR_HIP = 6
ERR_BAD_PLAN = 7

KV_BF16 = 0
KV_FP8_UE8M0 = 1
KV_FP8_TENSOR = 2
ENTRY_BYTES = {0: 1152, 1: 648, 2: 576}    # page bytes = entry bytes * page_size
IDX_LOGICAL = 0
IDX_GLOBAL = 1
F_PARTIALS_ONLY = 1
F_CHECK_INDICES = 2
F_BALANCE_ROWS = 4

EXPORTED = [
    "sparse_mla_decode_plan", "sparse_mla_plan_num_splits", "sparse_mla_decode_run",
    "sparse_mla_merge_partials", "sparse_mla_gather_debug", "sparse_mla_read_index_error",
    "sparse_mla_cache_store",
    "sparse_mla_status_string", "sparse_mla_version",
    "sparse_mla_indexer_logits",
    "sparse_mla_indexer_topk",
    "sparse_mla_translate_indices",
    "sparse_mla_decode_run_noalloc",
]
NOALLOC_SCRATCH_BYTES = 16 << 20


class Problem(ctypes.Structure):
    _fields_ = [
        ("num_rows", ctypes.c_int32), ("num_requests", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("max_pages_per_req", ctypes.c_int32), ("kv_format", ctypes.c_int32),
        ("index_mode", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("flags", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("kv_scale", ctypes.c_float),
    ]


class Plan(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_uint8 * 256)]


class SparseMLAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sparse_mla_decode_03_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, f32p, i32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p
    lib.sparse_mla_decode_plan.argtypes = [ctypes.POINTER(Problem), i32, ctypes.POINTER(Plan),
                                           ctypes.POINTER(ctypes.c_size_t)]
    lib.sparse_mla_decode_plan.restype = ctypes.c_int
    lib.sparse_mla_plan_num_splits.argtypes = [ctypes.POINTER(Plan)]
    lib.sparse_mla_plan_num_splits.restype = i32
    lib.sparse_mla_decode_run.argtypes = [ctypes.POINTER(Plan), vp, vp, i32p, i32p, i32p, f32p, vp,
                                          f32p, f32p, f32p, vp, ctypes.c_size_t, vp]
    lib.sparse_mla_decode_run.restype = ctypes.c_int
    lib.sparse_mla_decode_run_noalloc.argtypes = [ctypes.POINTER(Plan), vp, vp, i32p, i32p, i32p, f32p,
                                                  vp, f32p, vp]
    lib.sparse_mla_decode_run_noalloc.restype = ctypes.c_int
    lib.sparse_mla_merge_partials.argtypes = [f32p, f32p, i32, i32, i32, f32p, vp, f32p, vp]
    lib.sparse_mla_merge_partials.restype = ctypes.c_int
    lib.sparse_mla_gather_debug.argtypes = [vp, i32, i32, i32, i32p, i32, vp, vp]
    lib.sparse_mla_gather_debug.restype = ctypes.c_int
    lib.sparse_mla_cache_store.argtypes = [vp, vp, i32p, i32, i32, i32, i32, vp, vp]
    lib.sparse_mla_indexer_logits.argtypes = [vp, f32p, vp, i32p, i32p, i32, i32, i32, i32, i32, i32,
                                              i32, f32p, vp]
    lib.sparse_mla_indexer_topk.argtypes = [f32p, i32p, i32, i32, i32, i32p, vp]
    lib.sparse_mla_translate_indices.argtypes = [i32p, i32p, i32p, i32, i32, i32, i32, i32, i32, i32p, vp]
    lib.sparse_mla_translate_indices.restype = ctypes.c_int
    lib.sparse_mla_indexer_logits.restype = ctypes.c_int
    lib.sparse_mla_indexer_topk.restype = ctypes.c_int
    lib.sparse_mla_cache_store.restype = ctypes.c_int
    lib.sparse_mla_read_index_error.argtypes = [ctypes.POINTER(Plan), vp, ctypes.POINTER(i32 * 2), vp]
    lib.sparse_mla_read_index_error.restype = ctypes.c_int
    lib.sparse_mla_status_string.argtypes = [ctypes.c_int32]
    lib.sparse_mla_status_string.restype = ctypes.c_char_p
    lib.sparse_mla_version.argtypes = []
    lib.sparse_mla_version.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().sparse_mla_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != OK:
        raise SparseMLAError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


@dataclass
class PlanInfo:
    plan: Plan
    workspace_bytes: int
    num_splits: int
    problem: Problem


def make_problem(num_rows, num_requests, num_heads, topk, page_size, num_pages,
                 max_pages_per_req, kv_format, index_mode=IDX_LOGICAL, num_splits=0, flags=0,
                 softmax_scale=1.0 / math.sqrt(576.0), kv_scale=1.0) -> Problem:
    return Problem(int(num_rows), int(num_requests), int(num_heads), int(topk), int(page_size),
                   int(num_pages), int(max_pages_per_req), int(kv_format), int(index_mode),
                   int(num_splits), int(flags), float(softmax_scale), float(kv_scale))


def plan(problem: Problem, num_cus: int = 0) -> PlanInfo:
    lib = load_library()
    p = Plan()
    ws = ctypes.c_size_t(0)
    _check("sparse_mla_decode_plan",
           lib.sparse_mla_decode_plan(ctypes.byref(problem), int(num_cus), ctypes.byref(p),
                                      ctypes.byref(ws)))
    return PlanInfo(p, int(ws.value), int(lib.sparse_mla_plan_num_splits(ctypes.byref(p))), problem)


def run(info: PlanInfo, q, kv_cache, indices, row_req, page_table, sinks, out, lse=None,
        partial_o=None, partial_lse=None, workspace=None, stream=None) -> None:
    """Raw run: every tensor is caller-allocated on the GPU."""
    lib = load_library()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("sparse_mla_decode_run",
           lib.sparse_mla_decode_run(ctypes.byref(info.plan), _ptr(q), _ptr(kv_cache), _ptr(indices),
                                     _ptr(row_req), _ptr(page_table), _ptr(sinks), _ptr(out),
                                     _ptr(lse), _ptr(partial_o), _ptr(partial_lse), _ptr(workspace),
                                     ctypes.c_size_t(ws_bytes), _stream(stream)))


def run_noalloc(info: PlanInfo, q, kv_cache, indices, row_req, page_table, sinks, out, lse=None,
                stream=None) -> None:
    """Raw run through the allocation-free entry point (no workspace; split partials in the
    library's own per-GPU scratch)."""
    lib = load_library()
    _check("sparse_mla_decode_run_noalloc",
           lib.sparse_mla_decode_run_noalloc(ctypes.byref(info.plan), _ptr(q), _ptr(kv_cache),
                                             _ptr(indices), _ptr(row_req), _ptr(page_table),
                                             _ptr(sinks), _ptr(out), _ptr(lse), _stream(stream)))


def _kv_format_of(kv_format) -> int:
    if isinstance(kv_format, str):
        return {"fp8": KV_FP8_UE8M0, "fp8t": KV_FP8_TENSOR, "bf16": KV_BF16}[kv_format]
    return int(kv_format)


def _require(t: torch.Tensor, name: str, dtype, dev):
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def sparse_mla_decode(q: torch.Tensor, kv_cache: torch.Tensor, indices: torch.Tensor,
                      row_req: Optional[torch.Tensor], page_table: Optional[torch.Tensor],
                      sinks: Optional[torch.Tensor], kv_format, page_size: int,
                      softmax_scale: float, index_mode: int = IDX_LOGICAL, num_splits: int = 0,
                      flags: int = 0, num_cus: int = 0, stream=None, return_info: bool = False,
                      kv_scale: float = 1.0):
    """Convenience wrapper: plan, allocate out/lse/workspace with torch, run.

    q bf16 [R,H,576]; kv_cache uint8 [num_pages, page_bytes]; indices int32 [R,K];
    row_req int32 [R] and page_table int32 [B,P] (LOGICAL mode); sinks fp32 [H] or None.
    Returns (out bf16 [R,H,512], lse fp32 [R,H]) - or, with F_PARTIALS_ONLY,
    (partial_o fp32 [R,S,H,512], partial_lse fp32 [R,S,H]).
    """
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("sparse_mla_decode runs on the GPU only")
    _require(q, "q", torch.bfloat16, dev)
    _require(kv_cache, "kv_cache", torch.uint8, dev)
    _require(indices, "indices", torch.int32, dev)
    R, H, D = q.shape
    if D != 576:
        raise ValueError("q must be [R, H, 576]")
    K = indices.shape[1]
    if indices.shape[0] != R:
        raise ValueError("indices must be [R, K]")
    if index_mode == IDX_LOGICAL:
        _require(row_req, "row_req", torch.int32, dev)
        _require(page_table, "page_table", torch.int32, dev)
        B, P = page_table.shape
    else:
        B, P = 0, 0
    if index_mode == IDX_LOGICAL and row_req.numel() != R:
        raise ValueError("row_req must hold one request id per row")
    if sinks is not None:
        _require(sinks, "sinks", torch.float32, dev)
        if sinks.numel() != H:
            raise ValueError("sinks must hold one value per head")
    kvf = _kv_format_of(kv_format)
    if kv_cache.dim() != 2 or kv_cache.shape[1] != ENTRY_BYTES[kvf] * page_size:
        raise ValueError("kv_cache must be [num_pages, page_bytes] for this format and page size")
    prob = make_problem(R, B, H, K, page_size, kv_cache.shape[0], P, kvf,
                        index_mode, num_splits, flags, softmax_scale, kv_scale)
    with torch.cuda.device(dev):
        info = plan(prob, num_cus)
        ws = (torch.empty(info.workspace_bytes, dtype=torch.uint8, device=dev)
              if info.workspace_bytes > 0 else None)
        if flags & F_PARTIALS_ONLY:
            po = torch.empty((R, info.num_splits, H, 512), dtype=torch.float32, device=dev)
            pl = torch.empty((R, info.num_splits, H), dtype=torch.float32, device=dev)
            run(info, q, kv_cache, indices, row_req, page_table, sinks, None, None, po, pl, ws, stream)
            res = (po, pl)
        else:
            out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=dev)
            lse = torch.empty((R, H), dtype=torch.float32, device=dev)
            run(info, q, kv_cache, indices, row_req, page_table, sinks, out, lse, None, None, ws, stream)
            res = (out, lse)
    if return_info:
        return res + (info, ws)
    return res


def merge_partials(partial_o: torch.Tensor, partial_lse: torch.Tensor,
                   sinks: Optional[torch.Tensor], stream=None):
    """LSE-merge partials [R,S,H,512] / [R,S,H] with the sink; returns (out, lse)."""
    lib = load_library()
    dev = partial_o.device
    _require(partial_o, "partial_o", torch.float32, dev)
    _require(partial_lse, "partial_lse", torch.float32, dev)
    R, S, H, D = partial_o.shape
    if D != 512 or tuple(partial_lse.shape) != (R, S, H):
        raise ValueError("partials must be [R,S,H,512] and [R,S,H]")
    if sinks is not None:
        _require(sinks, "sinks", torch.float32, dev)
    out = torch.empty((R, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check("sparse_mla_merge_partials",
               lib.sparse_mla_merge_partials(_ptr(partial_o), _ptr(partial_lse), R, S, H,
                                             _ptr(sinks), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def gather_debug(kv_cache: torch.Tensor, kv_format, page_size: int, slots: torch.Tensor,
                 stream=None) -> torch.Tensor:
    """Dequantize cache slots to bf16 [n, 576] with the library's plain reference decoder
    (a test helper; not the decode kernel's LDS gather)."""
    lib = load_library()
    dev = kv_cache.device
    _require(kv_cache, "kv_cache", torch.uint8, dev)
    _require(slots, "slots", torch.int32, dev)
    if kv_cache.dim() != 2 or kv_cache.shape[1] != ENTRY_BYTES[_kv_format_of(kv_format)] * page_size:
        raise ValueError("kv_cache must be [num_pages, page_bytes] for this format and page size")
    n = slots.numel()
    out = torch.empty((n, 576), dtype=torch.bfloat16, device=dev)
    with torch.cuda.device(dev):
        _check("sparse_mla_gather_debug",
               lib.sparse_mla_gather_debug(_ptr(kv_cache), _kv_format_of(kv_format), int(page_size),
                                           int(kv_cache.shape[0]), _ptr(slots), int(n), _ptr(out),
                                           _stream(stream)))
    return out


def cache_store(kv_cache: torch.Tensor, kv_format, page_size: int, latent: torch.Tensor,
                rope: torch.Tensor, slots: torch.Tensor, stream=None) -> None:
    """Write tokens (bf16 latent [n, 512], bf16 rope [n, 64], int32 slots [n]) into the
    paged cache in place: FP8 e4m3fn + UE8M0 per 64 elements, or plain bf16."""
    lib = load_library()
    dev = kv_cache.device
    _require(kv_cache, "kv_cache", torch.uint8, dev)
    _require(latent, "latent", torch.bfloat16, dev)
    _require(rope, "rope", torch.bfloat16, dev)
    _require(slots, "slots", torch.int32, dev)
    kvf = _kv_format_of(kv_format)
    if kv_cache.dim() != 2 or kv_cache.shape[1] != (648 if kvf == KV_FP8_UE8M0 else 1152) * page_size:
        raise ValueError("kv_cache must be [num_pages, page_bytes] for this format and page size")
    n = slots.numel()
    if tuple(latent.shape) != (n, 512) or tuple(rope.shape) != (n, 64):
        raise ValueError("latent must be [n, 512] and rope [n, 64]")
    with torch.cuda.device(dev):
        _check("sparse_mla_cache_store",
               lib.sparse_mla_cache_store(_ptr(latent), _ptr(rope), _ptr(slots), int(n), kvf,
                                          int(page_size), int(kv_cache.shape[0]), _ptr(kv_cache),
                                          _stream(stream)))


def indexer_logits(q_codes: torch.Tensor, weights: torch.Tensor, key_cache: torch.Tensor,
                   row_len: torch.Tensor, page_table: torch.Tensor, next_n: int, width: int,
                   page_size: int = 64, logits: torch.Tensor = None, stream=None) -> torch.Tensor:
    """FP8 paged MQA logits: q_codes uint8 [R, 64, 128] (e4m3fn), weights fp32 [R, 64],
    key_cache uint8 [num_pages, 132 * page_size], row_len int32 [R], page_table int32
    [B, max_pages] with R = B * next_n.  Returns fp32 logits [R, width]; positions at or
    past a row's length are left as they were in `logits` (allocated empty if None)."""
    lib = load_library()
    dev = q_codes.device
    _require(q_codes, "q_codes", torch.uint8, dev)
    _require(weights, "weights", torch.float32, dev)
    _require(key_cache, "key_cache", torch.uint8, dev)
    _require(row_len, "row_len", torch.int32, dev)
    _require(page_table, "page_table", torch.int32, dev)
    R = int(q_codes.shape[0])
    B = int(page_table.shape[0])
    if q_codes.dim() != 3 or tuple(q_codes.shape[1:]) != (64, 128) or tuple(weights.shape) != (R, 64):
        raise ValueError("q_codes must be [R, 64, 128] and weights [R, 64]")
    if R != B * next_n or tuple(row_len.shape) != (R,):
        raise ValueError("rows must be num_requests * next_n, request-major, with one length each")
    if key_cache.dim() != 2 or key_cache.shape[1] != 132 * page_size:
        raise ValueError("key_cache must be [num_pages, 132 * page_size]")
    if logits is None:
        logits = torch.empty((R, width), dtype=torch.float32, device=dev)
    _require(logits, "logits", torch.float32, dev)
    if tuple(logits.shape) != (R, width):
        raise ValueError("logits must be [R, width]")
    with torch.cuda.device(dev):
        _check("sparse_mla_indexer_logits",
               lib.sparse_mla_indexer_logits(_ptr(q_codes), _ptr(weights), _ptr(key_cache), _ptr(row_len),
                                             _ptr(page_table), B, int(next_n), 64, int(page_size),
                                             int(key_cache.shape[0]), int(page_table.shape[1]), int(width),
                                             _ptr(logits), _stream(stream)))
    return logits


def indexer_topk(logits: torch.Tensor, row_len: torch.Tensor, topk: int, out: torch.Tensor = None,
                 stream=None) -> torch.Tensor:
    """Top-k positions of each row's logits (ascending positions, -1 padded): int32 [R, topk]."""
    lib = load_library()
    dev = logits.device
    _require(logits, "logits", torch.float32, dev)
    _require(row_len, "row_len", torch.int32, dev)
    R, width = int(logits.shape[0]), int(logits.shape[1])
    if tuple(row_len.shape) != (R,):
        raise ValueError("row_len must be [R]")
    if out is None:
        out = torch.empty((R, topk), dtype=torch.int32, device=dev)
    _require(out, "out", torch.int32, dev)
    if tuple(out.shape) != (R, topk):
        raise ValueError("out must be [R, topk]")
    with torch.cuda.device(dev):
        _check("sparse_mla_indexer_topk",
               lib.sparse_mla_indexer_topk(_ptr(logits), _ptr(row_len), R, width, int(topk), _ptr(out),
                                           _stream(stream)))
    return out


def translate_indices(indices: torch.Tensor, row_req: torch.Tensor, page_table: torch.Tensor,
                      page_size: int, num_pages: int, out: torch.Tensor = None, stream=None) -> torch.Tensor:
    """Request-local top-k positions -> global slots (int32 [R, K], -1 where masked)."""
    lib = load_library()
    dev = indices.device
    _require(indices, "indices", torch.int32, dev)
    _require(row_req, "row_req", torch.int32, dev)
    _require(page_table, "page_table", torch.int32, dev)
    R, K = int(indices.shape[0]), int(indices.shape[1])
    if out is None:
        out = torch.empty((R, K), dtype=torch.int32, device=dev)
    _require(out, "out", torch.int32, dev)
    with torch.cuda.device(dev):
        _check("sparse_mla_translate_indices",
               lib.sparse_mla_translate_indices(_ptr(indices), _ptr(row_req), _ptr(page_table), R, K,
                                                int(page_table.shape[0]), int(page_table.shape[1]),
                                                int(page_size), int(num_pages), _ptr(out), _stream(stream)))
    return out


def read_index_error(info: PlanInfo, workspace: torch.Tensor, stream=None):
    lib = load_library()
    rp = (ctypes.c_int32 * 2)()
    _check("sparse_mla_read_index_error",
           lib.sparse_mla_read_index_error(ctypes.byref(info.plan), _ptr(workspace), ctypes.byref(rp),
                                           _stream(stream)))
    return int(rp[0]), int(rp[1])
