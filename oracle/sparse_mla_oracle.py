"""Float64 CPU oracle for top-k sparse MLA decode with attention sinks and split-KV merge.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this module.  It shares no code with the HIP library: it reads
the same packed input bytes and decodes them with its own code, written from the
definitions below.

Sources (prhub.com.cn summaries of serving-engine pull requests):
  [vllm#43477]  "DSv4 and GLM-5.1 inference on Blackwell SM120" - key code excerpts:
                FlashInferMLASparseSM120Impl.forward_mqa (block-table translation of the
                top-k positions, output [tokens, heads, kv_lora_rank] in q's dtype, one
                latent KV head shared by all query heads via get_kv_cache_shape).
  [sglang#24692] "SM120 desktop Blackwell support for DeepSeek-V4" - implementation
                breakdown items 2-3: gather and dequantize paged entries with in-page
                addressing, tiled online softmax, merge of partial results, attention
                sink applied as its own step; review highlights: invalid ids (-1) are
                never dereferenced.
  [vllm#43827]  "FlashInfer TRTLLM-gen sparse MLA backend for DSv4" - key code excerpts:
                init_layer_buffers (bmm1 scale = softmax scale * q_scale * kv_scale with
                unit FP8 scales, so the logit scale is the softmax scale).
The pages never write the formula out.  What is computed here is the plain reading
of those passages, stated at each function that takes one.

Definitions implemented (natural exp/log; float64 throughout):
  k_j = dequantized cache entry (576), v_j = k_j[:512]
  s_j = scale * <q_h, k_j>;  sigma = sink_h or -inf;  m = max(max_j s_j, sigma)
  Z = exp(sigma - m) + sum_j exp(s_j - m);  o = sum_j exp(s_j - m) v_j / Z;  lse = m + ln Z
  empty row: o = 0, lse = sigma.
  chunk partials (sink-free): o_c = softmax-weighted mean over the chunk, lse_c = ln sum exp(s_j)
  merge: M = max(max_c lse_c, sigma), w_c = exp(lse_c - M), o = sum w_c o_c / (sum w_c + exp(sigma - M))
"""

from __future__ import annotations

import numpy as np

QK_DIM = 576
V_DIM = 512
ROPE_DIM = 64
SCALE_GROUP = 64
NUM_GROUPS = V_DIM // SCALE_GROUP  # 8
FP8_ENTRY_BYTES = 648
BF16_ENTRY_BYTES = 1152

KV_BF16 = 0
KV_FP8_UE8M0 = 1
KV_FP8_TENSOR = 2
FP8_TENSOR_ENTRY_BYTES = 576
IDX_LOGICAL = 0
IDX_GLOBAL = 1


# ---------------------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------------------

def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("e4m3fn"): sign bit, 4 exponent bits with bias 7, 3 mantissa bits.

    Normal (exponent field e in 1..15): (-1)^s * (1 + m/8) * 2^(e-7).
    Subnormal (e == 0):                 (-1)^s * (m/8) * 2^(-6).
    S.1111.111 is NaN; there are no infinities, so S.1111.110 = +-448 is the maximum.
    The FP8 latent of the paged cache is this format (vllm#43827 key code excerpts,
    _resolve_dsv4_kv_cache_dtype returns torch.float8_e4m3fn for the fp8 cache).
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def ue8m0_to_f64(codes: np.ndarray) -> np.ndarray:
    """UE8M0 scale byte: an unsigned biased exponent, value 2^(e-127); 255 is NaN.

    The pages name the UE8M0 paged layout of the fp8 cache (vllm#43827 motivation and
    key code excerpts) without spelling it out; this is the OCP MX E8M0 definition.
    """
    e = np.asarray(codes).astype(np.int64)
    val = np.exp2((e - 127).astype(np.float64))
    return np.where(e == 255, np.nan, val)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32: widen the 16 bits and read them."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------
# Cache layout and index translation
# ---------------------------------------------------------------------------------------

def page_bytes(kv_format: int, page_size: int) -> int:
    entry = {KV_BF16: BF16_ENTRY_BYTES, KV_FP8_UE8M0: FP8_ENTRY_BYTES,
             KV_FP8_TENSOR: FP8_TENSOR_ENTRY_BYTES}[kv_format]
    return entry * page_size


def decode_entries(cache: np.ndarray, kv_format: int, page_size: int, slots,
                   kv_scale: float = 1.0) -> np.ndarray:
    """Dequantize cache slots into float64 rows k[n, 576].

    `cache` is the whole paged buffer as bytes (any shape; it is flattened).  A slot is
    page = slot // page_size, row = slot % page_size.  The FP8 page holds three regions
    that the kernel of sglang#24692 reads through fp8 / uint8 / bf16 views of the same
    buffer (implementation breakdown item 2): e4m3fn latent [ps][512] at byte 0, bf16
    rope [ps][64] at byte 512*ps, UE8M0 scales [ps][8] at byte 640*ps.  The BF16 page
    is bf16 [ps][576].  The per-tensor FP8 page (the contiguous fp8_e4m3 cache of
    vllm#43827, implementation breakdown 1 and 4) is e4m3fn [ps][576], every value times
    the one tensor scale `kv_scale`.
    """
    flat = np.ascontiguousarray(cache).reshape(-1).view(np.uint8)
    slots = np.asarray(slots, dtype=np.int64).reshape(-1)
    n = slots.shape[0]
    pb = page_bytes(kv_format, page_size)
    page = slots // page_size
    row = slots % page_size
    base = page * pb
    out = np.empty((n, QK_DIM), dtype=np.float64)
    if n == 0:
        return out
    if kv_format == KV_BF16:
        offs = base + row * BF16_ENTRY_BYTES
        raw = flat[offs[:, None] + np.arange(BF16_ENTRY_BYTES)[None, :]]
        out[:] = bf16_bits_to_f64(raw.view(np.uint16).reshape(n, QK_DIM))
        return out
    if kv_format == KV_FP8_TENSOR:
        offs = base + row * FP8_TENSOR_ENTRY_BYTES
        codes = flat[offs[:, None] + np.arange(FP8_TENSOR_ENTRY_BYTES)[None, :]]
        out[:] = e4m3fn_to_f64(codes) * float(kv_scale)
        return out
    if kv_format != KV_FP8_UE8M0:
        raise ValueError(f"unknown kv_format {kv_format}")
    lat_off = base + row * 512
    rope_off = base + 512 * page_size + row * (2 * ROPE_DIM)
    sc_off = base + 640 * page_size + row * NUM_GROUPS
    lat = flat[lat_off[:, None] + np.arange(512)[None, :]]
    rope = flat[rope_off[:, None] + np.arange(2 * ROPE_DIM)[None, :]]
    sc = flat[sc_off[:, None] + np.arange(NUM_GROUPS)[None, :]]
    scale = ue8m0_to_f64(sc)  # [n, 8]
    out[:, :V_DIM] = e4m3fn_to_f64(lat) * np.repeat(scale, SCALE_GROUP, axis=1)
    out[:, V_DIM:] = bf16_bits_to_f64(np.ascontiguousarray(rope).view(np.uint16).reshape(n, ROPE_DIM))
    return out


def translate(idx_row: np.ndarray, index_mode: int, request: int, page_table, page_size: int,
              num_pages: int):
    """Request-local top-k positions -> (list positions kept, global slots).

    LOGICAL mode is the block-table translation that vllm#43477 runs before its kernel
    (triton_convert_req_index_to_global_index over req_id_per_token and block_table):
    slot = block_table[request][t // page_size] * page_size + t % page_size.
    GLOBAL mode takes t as the slot.  Invalid ids are dropped and never dereferenced
    (sglang#24692 review highlights: invalid ids): -1, and with it every entry that names
    no cache slot - a negative t, a page index past the request's block-table row, a page
    id outside [0, num_pages), a request outside the table, or (GLOBAL) a slot outside
    [0, num_pages * page_size).
    """
    idx_row = np.asarray(idx_row, dtype=np.int64)
    keep = idx_row >= 0
    if index_mode == IDX_GLOBAL:
        keep &= idx_row < num_pages * page_size
        pos = np.nonzero(keep)[0]
        return pos, idx_row[pos]
    pt = np.asarray(page_table, dtype=np.int64)
    if not 0 <= request < pt.shape[0]:
        return np.zeros(0, dtype=np.int64), np.zeros(0, dtype=np.int64)
    row = pt[request]
    pi = np.where(keep, idx_row // page_size, 0)
    keep &= pi < row.shape[0]
    page = np.where(keep, row[np.where(keep, pi, 0)], -1)
    keep &= (page >= 0) & (page < num_pages)
    pos = np.nonzero(keep)[0]
    t = idx_row[pos]
    return pos, page[pos] * page_size + t % page_size


# ---------------------------------------------------------------------------------------
# Attention over a set of decoded entries
# ---------------------------------------------------------------------------------------

def attend(q: np.ndarray, k: np.ndarray, scale: float, sink) -> tuple[np.ndarray, np.ndarray]:
    """Softmax-with-sink attention of H query vectors over n entries.

    q: float64 [H, 576]; k: float64 [n, 576]; sink: float64 [H] or None.
    Returns o [H, 512] and lse [H] (natural log), both float64.
    """
    H = q.shape[0]
    sig = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    o = np.zeros((H, V_DIM))
    if k.shape[0] == 0:
        return o, sig.copy()
    s = scale * (q @ k.T)                                   # [H, n]
    m = np.maximum(s.max(axis=1), sig)                      # finite: s is finite
    e = np.exp(s - m[:, None])
    es = np.exp(sig - m)                                    # 0 for a -inf sink
    z = e.sum(axis=1) + es
    o = (e @ k[:, :V_DIM]) / z[:, None]
    lse = m + np.log(z)
    return o, lse


def _row_inputs(r, q_bits, cache, kv_format, page_size, indices, row_req, page_table, index_mode,
                kv_scale=1.0):
    req = int(row_req[r]) if index_mode == IDX_LOGICAL else -1
    flat_bytes = np.asarray(cache).nbytes
    pos, slots = translate(indices[r], index_mode, req, page_table, page_size,
                           flat_bytes // page_bytes(kv_format, page_size))
    k = decode_entries(cache, kv_format, page_size, slots, kv_scale)
    q = bf16_bits_to_f64(q_bits[r])
    return q, pos, k


def sparse_mla_decode(q_bits, cache, kv_format, page_size, indices, row_req, page_table,
                      sinks, softmax_scale, index_mode=IDX_LOGICAL, rows=None, kv_scale=1.0):
    """Final decode output for the given rows.

    q_bits: uint16 [R, H, 576] (bf16 bit patterns); cache: uint8 paged buffer;
    indices: int32 [R, K]; row_req: int32 [R]; page_table: int32 [B, P];
    sinks: float32 [H] or None.  Returns o float64 [len(rows), H, 512], lse [len(rows), H].
    """
    q_bits = np.asarray(q_bits)
    indices = np.asarray(indices)
    R, H = q_bits.shape[0], q_bits.shape[1]
    rows = range(R) if rows is None else list(rows)
    sink = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    outs = np.zeros((len(rows), H, V_DIM))
    lses = np.zeros((len(rows), H))
    for i, r in enumerate(rows):
        q, _, k = _row_inputs(r, q_bits, cache, kv_format, page_size, indices, row_req,
                              page_table, index_mode, kv_scale)
        outs[i], lses[i] = attend(q, k, softmax_scale, sink)
    return outs, lses


def chunk_bounds(topk: int, num_splits: int):
    """Split-KV chunks are contiguous ranges of list positions of C = ceil(K/S) each."""
    c = -(-topk // num_splits)
    return [(min(i * c, topk), min((i + 1) * c, topk)) for i in range(num_splits)]


def sparse_mla_decode_partials(q_bits, cache, kv_format, page_size, indices, row_req,
                               page_table, softmax_scale, num_splits, index_mode=IDX_LOGICAL,
                               rows=None, kv_scale=1.0):
    """Sink-free per-chunk partials o_c [n_rows, S, H, 512] and lse_c [n_rows, S, H]."""
    q_bits = np.asarray(q_bits)
    indices = np.asarray(indices)
    R, H, K = q_bits.shape[0], q_bits.shape[1], indices.shape[1]
    rows = range(R) if rows is None else list(rows)
    bounds = chunk_bounds(K, num_splits)
    o_c = np.zeros((len(rows), num_splits, H, V_DIM))
    lse_c = np.full((len(rows), num_splits, H), -np.inf)
    for i, r in enumerate(rows):
        q, pos, k = _row_inputs(r, q_bits, cache, kv_format, page_size, indices, row_req,
                                page_table, index_mode, kv_scale)
        for c, (lo, hi) in enumerate(bounds):
            sel = (pos >= lo) & (pos < hi)
            o_c[i, c], lse_c[i, c] = attend(q, k[sel], softmax_scale, None)
    return o_c, lse_c


def merge_partials(o_c, lse_c, sinks):
    """LSE merge of sink-free partials with the sink applied once.

    o_c [..., S, H, 512], lse_c [..., S, H]; sinks [H] or None.  Chunks with
    lse_c = -inf get weight 0.  Returns o [..., H, 512], lse [..., H].
    """
    o_c = np.asarray(o_c, dtype=np.float64)
    lse_c = np.asarray(lse_c, dtype=np.float64)
    H = lse_c.shape[-1]
    sig = np.full(H, -np.inf) if sinks is None else np.asarray(sinks, dtype=np.float64)
    sig = np.broadcast_to(sig, lse_c.shape[:-2] + (H,))
    m = np.maximum(lse_c.max(axis=-2), sig)                 # [..., H]
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.where(np.isneginf(lse_c), 0.0, np.exp(lse_c - m_safe[..., None, :]))
    ws = np.where(np.isneginf(sig), 0.0, np.exp(sig - m_safe))
    z = w.sum(axis=-2) + ws
    z_safe = np.where(empty, 1.0, z)
    o = (w[..., None] * o_c).sum(axis=-3) / z_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, m_safe + np.log(z_safe))
    return o, lse
