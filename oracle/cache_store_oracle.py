"""Float64 CPU oracle for writing new tokens into the paged latent KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import this module.  It shares no code with the HIP library.

Sources (prhub.com.cn summaries of serving-engine pull requests):
  [vllm#43827]  "FlashInfer TRTLLM-gen sparse MLA backend for DSv4" - motivation and key
                code excerpts: the FP8 paged cache whose latent is e4m3fn with UE8M0
                power-of-two scales per 64 elements and whose rope part stays bf16; the
                compressor writes new tokens into it and the full-cache store is tested.
  [sglang#24692] implementation breakdown 2: entries are addressed inside their page
                (the region-split page read by the decode path).
The pages name the format but not the scale choice.  The reading taken here: the scale of
a group is the smallest power of two that keeps every code finite, i.e.

  group g = dims 64g .. 64g+63 of one token, amax = max |x|;
  e = 127 when amax == 0, else the smallest integer with 448 * 2^(e - 127) >= amax,
      clamped to [0, 254] (the UE8M0 byte);
  code[d] = the e4m3fn code whose value is nearest to x[d] / 2^(e - 127), a tie going to
      the code with an even mantissa;
  the latent codes, the token's 64 bf16 rope values and its 8 scale bytes are written to
  the token's slot of the region-split page; a BF16 cache stores the 576 bf16 values;
  slots that are negative or past the cache are skipped.
The per-tensor FP8 cache ([vllm#43827] implementation breakdown 4 and 5: the compressor
writes a contiguous per-tensor FP8 cache given the tensor's fp8 scale) stores all 576 values
of a token as e4m3fn codes.  The reading taken here, in the kernel's precision:

  y[d] = float32(x[d]) / float32(kv_scale), an IEEE float32 division (correctly rounded);
  y clamped to [-448, 448] (the saturating conversion of FP8 quantizers);
  code[d] = the e4m3fn code nearest to y[d], ties to the even code.

The float32 quotient decides the code, so the oracle forms it in float32 as the kernel does.
Inputs are bf16 (the model's latent and rope rows), decoded exactly to float64.
"""

from __future__ import annotations

import numpy as np

from .sparse_mla_oracle import (BF16_ENTRY_BYTES, FP8_ENTRY_BYTES, FP8_TENSOR_ENTRY_BYTES,
                                KV_BF16, KV_FP8_TENSOR, KV_FP8_UE8M0, bf16_bits_to_f64,
                                e4m3fn_to_f64)

LATENT = 512
ROPE = 64
GROUP = 64
E4M3_MAX = 448.0


def _e4m3fn_table():
    """Values of the 127 non-negative finite codes 0x00..0x7E, in code order."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return e4m3fn_to_f64(codes)


_POS = _e4m3fn_table()


def e4m3fn_nearest(y: np.ndarray) -> np.ndarray:
    """e4m3fn code nearest to each y (|y| <= 448), ties to the even code.

    Written as a search over the table of representable values, not as bit arithmetic:
    for |y| the two neighbouring table entries are compared and the closer one wins; an
    exact tie picks the code whose last bit (the mantissa LSB) is 0.  The sign bit is
    copied from y (so -0.0 gives 0x80).
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(a > E4M3_MAX) or np.any(~np.isfinite(a)):
        raise ValueError("e4m3fn_nearest expects finite |y| <= 448")
    hi = np.searchsorted(_POS, a, side="left")          # first table value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS[lo]
    d_hi = _POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _POS[lo], lo, code).astype(np.uint8)    # exact hits
    return np.where(np.signbit(y), code | 0x80, code).astype(np.uint8)


def ue8m0_for_amax(amax: np.ndarray) -> np.ndarray:
    """Scale byte e: 127 for amax == 0, else the smallest e with 448 * 2^(e-127) >= amax,
    clamped to [0, 254]."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, 127, dtype=np.int64)
    pos = amax > 0
    # a first guess from log2, then settled by exact power-of-two comparisons
    k = np.zeros(amax.shape, dtype=np.int64)
    k[pos] = np.ceil(np.log2(amax[pos] / E4M3_MAX)).astype(np.int64)
    for _ in range(3):
        too_small = pos & (E4M3_MAX * np.exp2(k.astype(np.float64)) < amax)
        k = np.where(too_small, k + 1, k)
        can_lower = pos & (E4M3_MAX * np.exp2((k - 1).astype(np.float64)) >= amax)
        k = np.where(can_lower, k - 1, k)
    out[pos] = k[pos] + 127
    return np.clip(out, 0, 254).astype(np.uint8)


def quantize_fp8_ue8m0(latent_bits: np.ndarray):
    """bf16 latent rows [n, 512] (uint16 bit patterns) -> e4m3fn codes [n, 512] and UE8M0
    scale bytes [n, 8]."""
    x = bf16_bits_to_f64(np.asarray(latent_bits, dtype=np.uint16)).reshape(-1, LATENT // GROUP, GROUP)
    amax = np.abs(x).max(axis=-1)
    e = ue8m0_for_amax(amax)
    y = x / np.exp2(e.astype(np.float64) - 127.0)[..., None]
    codes = e4m3fn_nearest(y).reshape(-1, LATENT)
    return codes, e


def quantize_fp8_tensor(latent_bits: np.ndarray, rope_bits: np.ndarray, kv_scale: float):
    """bf16 latent [n, 512] and rope [n, 64] (uint16 bit patterns) -> e4m3fn codes [n, 576]
    of the per-tensor FP8 cache with the one scale `kv_scale`."""
    if not (np.isfinite(kv_scale) and kv_scale > 0):
        raise ValueError("kv_scale must be finite and > 0")
    lat = bf16_bits_to_f64(np.asarray(latent_bits, dtype=np.uint16)).reshape(-1, LATENT)
    rope = bf16_bits_to_f64(np.asarray(rope_bits, dtype=np.uint16)).reshape(-1, ROPE)
    x = np.concatenate([lat, rope], axis=1).astype(np.float32)      # exact: bf16 values
    y = np.divide(x, np.float32(kv_scale), dtype=np.float32)
    y = np.clip(y.astype(np.float64), -E4M3_MAX, E4M3_MAX)
    return e4m3fn_nearest(y)


def cache_store(cache: np.ndarray, kv_format: int, page_size: int, latent_bits: np.ndarray,
                rope_bits: np.ndarray, slots: np.ndarray, kv_scale: float = 1.0) -> np.ndarray:
    """Return a copy of `cache` ([num_pages, page bytes] uint8) with the tokens written.

    Tokens are applied in order, so a slot named twice keeps the last token's bytes.
    """
    out = np.array(cache, dtype=np.uint8, copy=True)
    num_pages = out.shape[0]
    latent_bits = np.asarray(latent_bits, dtype=np.uint16).reshape(-1, LATENT)
    rope_bits = np.asarray(rope_bits, dtype=np.uint16).reshape(-1, ROPE)
    slots = np.asarray(slots, dtype=np.int64).reshape(-1)
    if kv_format == KV_FP8_UE8M0:
        codes, scales = quantize_fp8_ue8m0(latent_bits)
    elif kv_format == KV_FP8_TENSOR:
        codes = quantize_fp8_tensor(latent_bits, rope_bits, kv_scale)
    for t, slot in enumerate(slots):
        if slot < 0 or slot >= num_pages * page_size:
            continue
        page, r = divmod(int(slot), page_size)
        if kv_format == KV_FP8_UE8M0:
            out[page, r * LATENT:(r + 1) * LATENT] = codes[t]
            rb = LATENT * page_size + r * 2 * ROPE
            out[page, rb:rb + 2 * ROPE] = rope_bits[t].astype("<u2").view(np.uint8)
            sb = (LATENT + 2 * ROPE) * page_size + r * 8
            out[page, sb:sb + 8] = scales[t]
        elif kv_format == KV_BF16:
            row = np.concatenate([latent_bits[t], rope_bits[t]]).astype("<u2").view(np.uint8)
            out[page, r * BF16_ENTRY_BYTES:(r + 1) * BF16_ENTRY_BYTES] = row
        elif kv_format == KV_FP8_TENSOR:
            out[page, r * FP8_TENSOR_ENTRY_BYTES:(r + 1) * FP8_TENSOR_ENTRY_BYTES] = codes[t]
        else:
            raise ValueError("unknown kv_format")
    assert FP8_ENTRY_BYTES == LATENT + 2 * ROPE + 8
    return out
