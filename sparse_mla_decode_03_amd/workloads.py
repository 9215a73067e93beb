"""Seeded synthetic inputs for sparse MLA decode.

This module only draws random numbers and lays bytes out in the paged cache format; it
holds none of the decode arithmetic (no dequantisation, no dot products, no softmax).
Both the HIP path and the float64 oracle consume what it produces.

Five workloads, following the shapes used for the DeepSeek-V4 sparse decode on the
source pages (576-wide latent KV shared by all heads, top-k lists of 2048, page size 64,
MTP rows with their own index lists):
  tiny_bf16     1 request x 1 row, 16 heads, BF16 cache of 4 pages (identity table),
                64 distinct indices out of 256 tokens with the last 8 set to -1, no sink.
  b32_h64_fp8   32 requests x 1 row, 64 heads, context ~ U[4096, 32768], FP8+UE8M0,
                2048 distinct indices per row, sinks ~ N(0,1).
  b128_mtp4_h128_fp8
                128 requests x 4 rows (independent lists), 128 heads,
                context ~ U[8192, 131072], FP8+UE8M0, sinks ~ N(0,1).
  b2_h128_bf16_split16
                2 requests x 1 row, 128 heads, context 131072, BF16, 16 forced splits.
  ragged_b256_h64_fp8
                256 requests with next_n in {1,2,4}, 64 heads, context 4096 each over a
                shuffled pool of 16384 pages, valid count ~ U[1, 2048] padded with -1,
                about 10% of requests share their first 32 pages with another request,
                sinks -inf on heads 0..31 and ~ N(0,1) on 32..63.

Draw order (numpy.random.default_rng(seed)): context lengths, rows per request, page
permutation, shared-page copies, then per row (valid count, indices), then q, then
sinks.  The cache is drawn by torch.Generator(device).manual_seed(seed) in chunks of
pages, so it can be produced directly on the GPU for the large workloads.

FP8 encoding of the latent (the cache producer, not the decode path): per token and
per group of 64 dims, k = the smallest integer with amax <= 448 * 2^k (k = 0 for an
all-zero group); scale byte = k + 127; code = round-to-nearest-even e4m3fn of x / 2^k
(torch's float8_e4m3fn cast; |x / 2^k| <= 448 so nothing saturates).
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

KV_BF16 = "bf16"
KV_FP8 = "fp8"
KV_FP8T = "fp8t"        # per-tensor FP8: e4m3fn [576] per entry, one scale for the cache

LATENT = 512
ROPE = 64
WIDTH = 576
GROUPS = 8


@dataclass(frozen=True)
class WorkloadSpec:
    name: str
    num_requests: int
    rows_per_request: tuple          # choices drawn uniformly per request
    num_heads: int
    topk: int
    ctx_lo: int
    ctx_hi: int
    kv_format: str
    page_size: int = 64
    valid: str = "all"               # "all" | "tail8_masked" | "uniform"
    sinks: str = "normal"            # "none" | "normal" | "half_neg_inf"
    shared_frac: float = 0.0         # fraction of requests whose first pages are shared
    shared_pages: int = 32
    permute_pages: bool = True
    num_splits: int = 0              # 0 = planner decides
    softmax_scale: float = 1.0 / math.sqrt(576.0)
    causal: bool = False             # row i of n rows draws from positions < ctx - n + 1 + i
    kv_scale: float = 1.0            # per-tensor FP8: the cache's one scale
    flags: int = 0                   # run flags that suit the batch (4: balanced rows)

    def scaled(self, **kw) -> "WorkloadSpec":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_bf16": WorkloadSpec("tiny_bf16", 1, (1,), 16, 64, 256, 256, KV_BF16,
                              valid="tail8_masked", sinks="none", permute_pages=False),
    "b32_h64_fp8": WorkloadSpec("b32_h64_fp8", 32, (1,), 64, 2048, 4096, 32768, KV_FP8),
    "b128_mtp4_h128_fp8": WorkloadSpec("b128_mtp4_h128_fp8", 128, (4,), 128, 2048, 8192,
                                       131072, KV_FP8),
    "b2_h128_bf16_split16": WorkloadSpec("b2_h128_bf16_split16", 2, (1,), 128, 2048, 131072,
                                         131072, KV_BF16, num_splits=16),
    "ragged_b256_h64_fp8": WorkloadSpec("ragged_b256_h64_fp8", 256, (1, 2, 4), 64, 2048, 4096,
                                        4096, KV_FP8, valid="uniform", sinks="half_neg_inf",
                                        shared_frac=0.1, flags=4),
    # prefill chunks and decode rows in one launch: requests with 1, 4 or 256 query rows,
    # each row with its own causal top-k list
    # the headline shape over the contiguous per-tensor FP8 cache
    "b128_mtp4_h128_fp8t": WorkloadSpec("b128_mtp4_h128_fp8t", 128, (4,), 128, 2048, 8192,
                                        131072, KV_FP8T, kv_scale=1.0 / 64),
    "mixed_b24_h128_fp8": WorkloadSpec("mixed_b24_h128_fp8", 24, (1, 4, 256), 128, 2048, 8192,
                                       65536, KV_FP8, causal=True),
}
# Order of the workloads as they are numbered in the documentation (1..5).
WORKLOAD_ORDER = ["tiny_bf16", "b32_h64_fp8", "b128_mtp4_h128_fp8", "b2_h128_bf16_split16",
                  "ragged_b256_h64_fp8"]


@dataclass
class Inputs:
    spec: WorkloadSpec
    q: torch.Tensor                  # bf16 [R, H, 576]
    kv_cache: torch.Tensor           # uint8 [num_pages, page_bytes]
    indices: torch.Tensor            # int32 [R, K]
    row_req: torch.Tensor            # int32 [R]
    page_table: torch.Tensor         # int32 [B, max_pages]
    sinks: Optional[torch.Tensor]    # fp32 [H] or None
    context_lens: torch.Tensor       # int32 [B]
    meta: dict = field(default_factory=dict)

    @property
    def num_rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.kv_cache.shape[0])

    def num_valid(self) -> int:
        return int((self.indices != -1).sum().item())

    def to(self, device) -> "Inputs":
        mv = lambda t: None if t is None else t.to(device)  # noqa: E731
        return Inputs(self.spec, mv(self.q), mv(self.kv_cache), mv(self.indices),
                      mv(self.row_req), mv(self.page_table), mv(self.sinks),
                      mv(self.context_lens), dict(self.meta))


def page_bytes(kv_format: str, page_size: int) -> int:
    return {KV_FP8: 648, KV_FP8T: 576, KV_BF16: 1152}[kv_format] * page_size


def encode_fp8_groups(x: torch.Tensor):
    """Encode float32 latents [n, 512] as e4m3fn codes [n, 512] and UE8M0 bytes [n, 8]."""
    n = x.shape[0]
    g = x.reshape(n, GROUPS, LATENT // GROUPS)
    amax = g.abs().amax(dim=-1)
    lim = torch.full_like(amax, 448.0)
    pos = amax > 0
    k = torch.where(pos, torch.ceil(torch.log2(torch.where(pos, amax, lim) / 448.0)),
                    torch.zeros_like(amax))
    # log2 and the division round; settle k exactly with power-of-two products.
    k = torch.where(pos & (amax > torch.ldexp(lim, k)), k + 1, k)
    k = torch.where(pos & (amax <= torch.ldexp(lim, k - 1)), k - 1, k)
    y = g * torch.ldexp(torch.ones_like(amax), -k)[..., None]
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(n, LATENT)
    sbytes = (k + 127).clamp(0, 254).to(torch.uint8)
    return codes, sbytes


def pack_fp8_pages(codes: torch.Tensor, rope_bf16: torch.Tensor, scale_bytes: torch.Tensor,
                   page_size: int) -> torch.Tensor:
    """Region-split FP8 pages: latent [ps][512] | rope bf16 [ps][64] | scales [ps][8]."""
    n = codes.shape[0]
    assert n % page_size == 0
    npg = n // page_size
    out = torch.empty((npg, 648 * page_size), dtype=torch.uint8, device=codes.device)
    out[:, : 512 * page_size] = codes.reshape(npg, 512 * page_size)
    out[:, 512 * page_size: 640 * page_size] = (
        rope_bf16.contiguous().view(torch.uint8).reshape(npg, 128 * page_size))
    out[:, 640 * page_size:] = scale_bytes.reshape(npg, 8 * page_size)
    return out


def make_cache(num_pages: int, page_size: int, kv_format: str, seed: int,
               device="cpu", chunk_pages: int = 2048, kv_scale: float = 1.0) -> torch.Tensor:
    """Random paged cache: N(0,1) values, FP8+UE8M0 latent with bf16 rope, or plain bf16."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    pb = page_bytes(kv_format, page_size)
    cache = torch.empty((num_pages, pb), dtype=torch.uint8, device=device)
    for p0 in range(0, num_pages, chunk_pages):
        p1 = min(num_pages, p0 + chunk_pages)
        ntok = (p1 - p0) * page_size
        if kv_format == KV_BF16:
            vals = torch.randn((ntok, WIDTH), generator=gen, device=device, dtype=torch.float32)
            cache[p0:p1] = vals.to(torch.bfloat16).view(torch.uint8).reshape(p1 - p0, pb)
        elif kv_format == KV_FP8T:
            vals = torch.randn((ntok, WIDTH), generator=gen, device=device, dtype=torch.float32)
            codes = (vals / kv_scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
            cache[p0:p1] = codes.view(torch.uint8).reshape(p1 - p0, pb)
        else:
            lat = torch.randn((ntok, LATENT), generator=gen, device=device, dtype=torch.float32)
            rope = torch.randn((ntok, ROPE), generator=gen, device=device, dtype=torch.float32)
            codes, sb = encode_fp8_groups(lat)
            cache[p0:p1] = pack_fp8_pages(codes, rope.to(torch.bfloat16), sb, page_size)
    return cache


def _bf16_from_normal(rng: np.random.Generator, shape) -> torch.Tensor:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(torch.bfloat16)


def make_inputs(spec: WorkloadSpec, seed: int, device="cpu", cache_device=None) -> Inputs:
    """Draw one workload.  Small tensors are drawn on the host with numpy and moved to
    `device`; the cache is drawn on `cache_device` (default: `device`)."""
    cache_device = device if cache_device is None else cache_device
    rng = np.random.default_rng(seed)
    B, ps, K = spec.num_requests, spec.page_size, spec.topk
    ctx = rng.integers(spec.ctx_lo, spec.ctx_hi + 1, size=B)
    nrows = rng.choice(np.asarray(spec.rows_per_request), size=B)
    pages_per_req = -(-ctx // ps)
    num_pages = int(pages_per_req.sum())
    max_pages = int(pages_per_req.max())
    perm = rng.permutation(num_pages) if spec.permute_pages else np.arange(num_pages)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    start = 0
    for b in range(B):
        page_table[b, : pages_per_req[b]] = perm[start: start + pages_per_req[b]]
        start += pages_per_req[b]
    shared = []
    n_shared = int(round(spec.shared_frac * B))
    if n_shared > 0:
        takers = rng.choice(B, size=n_shared, replace=False)
        for b in takers:
            donor = int(rng.integers(0, B - 1))
            donor = donor + 1 if donor >= b else donor
            npg = min(spec.shared_pages, pages_per_req[b], pages_per_req[donor])
            page_table[b, :npg] = page_table[donor, :npg]
            shared.append((int(b), donor, int(npg)))
    R = int(nrows.sum())
    row_req = np.repeat(np.arange(B, dtype=np.int32), nrows)
    indices = np.full((R, K), -1, dtype=np.int32)
    first_row = np.concatenate([[0], np.cumsum(nrows)[:-1]])
    for r in range(R):
        c = int(ctx[row_req[r]])
        if spec.causal:
            b = int(row_req[r])
            c -= int(nrows[b]) - 1 - (r - int(first_row[b]))
        if spec.valid == "uniform":
            count = int(rng.integers(1, K + 1))
        else:
            count = K
        count = min(count, c)
        indices[r, :count] = rng.choice(c, size=count, replace=False)
        if spec.valid == "tail8_masked":
            indices[r, K - 8:] = -1
    q = _bf16_from_normal(rng, (R, spec.num_heads, WIDTH))
    if spec.sinks == "none":
        sinks = None
    else:
        sinks = rng.standard_normal(size=spec.num_heads).astype(np.float32)
        if spec.sinks == "half_neg_inf":
            sinks[: spec.num_heads // 2] = -np.inf
        sinks = torch.from_numpy(sinks)
    cache = make_cache(num_pages, ps, spec.kv_format, seed, device=cache_device, kv_scale=spec.kv_scale)
    mv = lambda t: None if t is None else t.to(device)  # noqa: E731
    return Inputs(spec, mv(q), cache, mv(torch.from_numpy(indices)), mv(torch.from_numpy(row_req)),
                  mv(torch.from_numpy(page_table)), mv(sinks),
                  mv(torch.from_numpy(ctx.astype(np.int32))), {"seed": seed, "shared": shared})


def compulsory_bytes(inp: Inputs) -> int:
    """Bytes the method must move once: q, gathered entries, indices, page-table rows
    of the requests, out (bf16) and lse (fp32), sinks."""
    R, H, K = inp.num_rows, inp.num_heads, inp.spec.topk
    entry = {KV_FP8: 648, KV_FP8T: 576, KV_BF16: 1152}[inp.spec.kv_format]
    n = inp.num_valid()
    ctx = inp.context_lens.cpu().numpy().astype(np.int64)
    pt = int((-(-ctx // inp.spec.page_size)).sum()) * 4
    sinks = 0 if inp.sinks is None else 4 * H
    return R * H * 1152 + n * entry + R * K * 4 + pt + R * H * (1024 + 4) + sinks


def algorithmic_flops(inp: Inputs) -> int:
    """2*H*(576+512) per attended entry: the QK and PV contractions."""
    return 2 * inp.num_heads * (WIDTH + LATENT) * inp.num_valid()


# ---------------------------------------------------------------------------------------
# Indexer inputs: FP8 index keys (128 e4m3fn codes + an fp32 scale per token, paged like
# the latent cache), FP8 index queries and fp32 per-head weights, next_n rows per request.
# ---------------------------------------------------------------------------------------

INDEX_DIM = 128


@dataclass(frozen=True)
class IndexerSpec:
    name: str
    num_requests: int
    next_n: int
    num_heads: int
    topk: int
    ctx_lo: int
    ctx_hi: int
    page_size: int = 64
    permute_pages: bool = True

    def scaled(self, **kw) -> "IndexerSpec":
        return dataclasses.replace(self, **kw)


INDEXER_WORKLOADS = {
    # the index lists of the headline decode workload: 128 requests x 4 MTP rows
    "idx_b128_mtp4_h64": IndexerSpec("idx_b128_mtp4_h64", 128, 4, 64, 2048, 8192, 131072),
    "idx_b32_n1_h64": IndexerSpec("idx_b32_n1_h64", 32, 1, 64, 2048, 4096, 32768),
    "idx_small": IndexerSpec("idx_small", 3, 2, 64, 256, 200, 1500),
}


@dataclass
class IndexerInputs:
    spec: IndexerSpec
    q_codes: torch.Tensor            # uint8 [R, H, 128] e4m3fn
    weights: torch.Tensor            # fp32 [R, H]
    key_cache: torch.Tensor          # uint8 [num_pages, 132 * page_size]
    row_req: torch.Tensor            # int32 [R]
    row_len: torch.Tensor            # int32 [R]: positions 0 .. len-1 are visible
    page_table: torch.Tensor         # int32 [B, max_pages]
    context_lens: torch.Tensor       # int32 [B]
    width: int                       # logits row stride (>= max row_len, multiple of 64)

    @property
    def num_rows(self) -> int:
        return int(self.q_codes.shape[0])


def encode_keys(x: torch.Tensor):
    """float32 keys [n, 128] -> e4m3fn codes [n, 128] and fp32 scales [n] (amax / 448,
    1 for an all-zero key)."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    codes = (x / scale[:, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


def pack_key_pages(codes: torch.Tensor, scales: torch.Tensor, page_size: int) -> torch.Tensor:
    """Region-split key pages: codes [ps][128] | scales fp32 [ps]."""
    n = codes.shape[0]
    assert n % page_size == 0
    npg = n // page_size
    out = torch.empty((npg, (INDEX_DIM + 4) * page_size), dtype=torch.uint8, device=codes.device)
    out[:, : INDEX_DIM * page_size] = codes.reshape(npg, INDEX_DIM * page_size)
    out[:, INDEX_DIM * page_size:] = scales.contiguous().view(torch.uint8).reshape(npg, 4 * page_size)
    return out


def make_key_cache(num_pages: int, page_size: int, seed: int, device="cpu",
                   chunk_pages: int = 4096) -> torch.Tensor:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 7919)
    cache = torch.empty((num_pages, (INDEX_DIM + 4) * page_size), dtype=torch.uint8, device=device)
    for p0 in range(0, num_pages, chunk_pages):
        p1 = min(num_pages, p0 + chunk_pages)
        x = torch.randn(((p1 - p0) * page_size, INDEX_DIM), generator=gen, device=device,
                        dtype=torch.float32)
        codes, scales = encode_keys(x)
        cache[p0:p1] = pack_key_pages(codes, scales, page_size)
    return cache


def make_indexer_inputs(spec: IndexerSpec, seed: int, device="cpu", cache_device=None) -> IndexerInputs:
    """Requests with contexts U[ctx_lo, ctx_hi]; row i of a request's next_n rows sees
    positions 0 .. ctx - next_n + i (the MTP rows are the request's last next_n tokens).
    Queries N(0,1) cast to e4m3fn, weights N(0,1)/sqrt(H), keys N(0,1) quantized per token."""
    cache_device = device if cache_device is None else cache_device
    rng = np.random.default_rng(seed)
    B, ps, nn, H = spec.num_requests, spec.page_size, spec.next_n, spec.num_heads
    ctx = rng.integers(spec.ctx_lo, spec.ctx_hi + 1, size=B)
    pages_per_req = -(-ctx // ps)
    num_pages = int(pages_per_req.sum())
    perm = rng.permutation(num_pages) if spec.permute_pages else np.arange(num_pages)
    page_table = np.full((B, int(pages_per_req.max())), -1, dtype=np.int32)
    start = 0
    for b in range(B):
        page_table[b, : pages_per_req[b]] = perm[start: start + pages_per_req[b]]
        start += pages_per_req[b]
    R = B * nn
    row_req = np.repeat(np.arange(B, dtype=np.int32), nn)
    row_len = np.array([ctx[b] - (nn - 1 - i) for b in range(B) for i in range(nn)], dtype=np.int32)
    q = torch.from_numpy(rng.standard_normal(size=(R, H, INDEX_DIM), dtype=np.float32))
    q_codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
    weights = torch.from_numpy((rng.standard_normal(size=(R, H)) / math.sqrt(H)).astype(np.float32))
    width = int(-(-int(row_len.max()) // 64) * 64)
    cache = make_key_cache(num_pages, ps, seed, device=cache_device)
    mv = lambda t: t.to(device)  # noqa: E731
    return IndexerInputs(spec, mv(q_codes), mv(weights), cache, mv(torch.from_numpy(row_req)),
                         mv(torch.from_numpy(row_len)), mv(torch.from_numpy(page_table)),
                         mv(torch.from_numpy(ctx.astype(np.int32))), width)


def indexer_algorithmic_bytes(inp: IndexerInputs) -> int:
    """Each request's keys read once (132 B per position up to its longest row), the
    queries (128 B per head) and weights (4 B per head) of every row, the page-table rows,
    and the logits written (4 B per visible position)."""
    lens = inp.row_len.cpu().numpy().astype(np.int64)
    rr = inp.row_req.cpu().numpy()
    per_req = np.zeros(inp.spec.num_requests, dtype=np.int64)
    np.maximum.at(per_req, rr, lens)
    H = inp.spec.num_heads
    return int(per_req.sum() * 132 + inp.num_rows * H * 132
               + (-(-per_req // inp.spec.page_size)).sum() * 4 + lens.sum() * 4)


def indexer_algorithmic_flops(inp: IndexerInputs) -> int:
    """2 * H * 128 per (row, visible position)."""
    return int(2 * inp.spec.num_heads * INDEX_DIM * inp.row_len.cpu().numpy().astype(np.int64).sum())
