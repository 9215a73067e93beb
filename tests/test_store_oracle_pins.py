"""Pins of the cache-store oracle (FP8 e4m3fn + UE8M0 quantization and the page write)
against things other than itself: torch's float8_e4m3fn cast (round to nearest even), the
OCP closed form of the scale rule, the decoder of the decode oracle, and hand-worked
values.  CPU only."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle import cache_store_oracle as cso
from oracle import sparse_mla_oracle as orc
from sparse_mla_decode_03_amd import workloads as W


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_exact_values_encode_to_their_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = orc.e4m3fn_to_f64(codes)
    assert np.array_equal(cso.e4m3fn_nearest(vals), codes)


def test_rounding_matches_torch_cast_including_ties():
    rng = np.random.default_rng(7)
    y = rng.uniform(-448, 448, 20000)
    # exact midpoints between neighbouring codes: ties must go to the even code
    pos = orc.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    y = np.concatenate([y, mids, -mids, [0.0, -0.0, 448.0, -448.0]])
    ref = torch.from_numpy(y.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # float32 holds every midpoint exactly, so the cast sees the same ties
    assert np.array_equal(cso.e4m3fn_nearest(y), ref)


def test_tie_examples_by_hand():
    # 1.0625 lies halfway between 1.0 (0x38, even) and 1.125 (0x39): goes to 1.0
    # 1.1875 lies halfway between 1.125 (0x39) and 1.25 (0x3A, even): goes to 1.25
    # 2^-10 lies halfway between 0 and the smallest subnormal 2^-9 (0x01): goes to 0
    assert cso.e4m3fn_nearest(np.array([1.0625, 1.1875, 2.0 ** -10])).tolist() == [0x38, 0x3A, 0x00]


@pytest.mark.parametrize("amax,e", [
    (0.0, 127),                  # empty group: scale 1
    (448.0, 127),                # exactly the largest code at scale 1
    (450.0, 128),                # next bf16 above 448 needs one more power of two
    (1.0, 119),                  # 448 * 2^-8 = 1.75 >= 1 > 448 * 2^-9
    (1.75, 119),
    (1.7578125, 120),            # next bf16 above 1.75
    (2.0 ** -140, 0),            # tiny: clamped at the smallest scale
])
def test_scale_rule_examples(amax, e):
    assert int(cso.ue8m0_for_amax(np.array([amax]))[0]) == e


def test_scale_rule_is_the_smallest_finite_power_of_two():
    rng = np.random.default_rng(3)
    amax = np.abs(rng.standard_normal(5000)) * np.exp2(rng.integers(-30, 30, 5000))
    amax = orc.bf16_bits_to_f64(_bf16_bits(amax))
    e = cso.ue8m0_for_amax(amax).astype(np.float64)
    assert np.all(448.0 * np.exp2(e - 127) >= amax)
    assert np.all(448.0 * np.exp2(e - 128) < amax)


def test_quantize_round_trip_and_generator_agreement():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    x[3, :64] = 0.0                      # an all-zero group
    x[5, 64:128] *= 1e-3                 # a small-magnitude group
    bits = _bf16_bits(x)
    xb = orc.bf16_bits_to_f64(bits).reshape(64, 512)
    codes, scales = cso.quantize_fp8_ue8m0(bits)
    deq = orc.e4m3fn_to_f64(codes) * np.repeat(orc.ue8m0_to_f64(scales), 64, axis=1)
    # within half an e4m3 step (3 mantissa bits) of each value, or of the subnormal step
    step = np.maximum(np.abs(xb) * 2.0 ** -3, np.repeat(orc.ue8m0_to_f64(scales), 64, axis=1) * 2.0 ** -9)
    assert np.all(np.abs(deq - xb) <= step / 2 + 1e-300)
    assert np.all(codes[3, :64] == 0) and scales[3, 0] == 127
    # the seeded input generator implements the same reading of the scale rule
    g_codes, g_scales = W.encode_fp8_groups(torch.from_numpy(xb.astype(np.float32)))
    assert np.array_equal(g_codes.numpy(), codes)
    assert np.array_equal(g_scales.numpy(), scales)


@pytest.mark.parametrize("kv_format", [oracle.KV_FP8_UE8M0, oracle.KV_BF16, oracle.KV_FP8_TENSOR])
def test_store_then_decode_gives_the_quantized_rows(kv_format):
    rng = np.random.default_rng(5)
    ps, npages, n = 4, 6, 9
    pb = orc.page_bytes(kv_format, ps)
    cache = rng.integers(0, 255, (npages, pb), dtype=np.uint8)
    lat = _bf16_bits(rng.standard_normal((n, 512)))
    rope = _bf16_bits(rng.standard_normal((n, 64)))
    slots = rng.choice(npages * ps, n, replace=False).astype(np.int64)
    slots[2] = -1                        # skipped
    slots[4] = npages * ps               # past the cache: skipped
    kv_scale = 0.0125
    out = cso.cache_store(cache, kv_format, ps, lat, rope, slots, kv_scale=kv_scale)
    written = [int(s) for s in slots if 0 <= s < npages * ps]
    rows = orc.decode_entries(out, kv_format, ps, np.array(written), kv_scale=kv_scale)
    keep = [t for t, s in enumerate(slots) if 0 <= s < npages * ps]
    if kv_format == oracle.KV_FP8_TENSOR:
        # every value comes back within half an e4m3 step of itself (3 mantissa bits, or the
        # subnormal step 2^-9 in code units), the rope included
        x = np.concatenate([orc.bf16_bits_to_f64(lat), orc.bf16_bits_to_f64(rope)], axis=1)[keep]
        step = np.maximum(np.abs(x) * 2.0 ** -3, kv_scale * 2.0 ** -9)
        assert np.all(np.abs(rows - x) <= step / 2 * (1 + 1e-6))
        codes = cso.quantize_fp8_tensor(lat, rope, kv_scale)
        assert np.array_equal(rows, orc.e4m3fn_to_f64(codes[keep]) * kv_scale)
    elif kv_format == oracle.KV_FP8_UE8M0:
        codes, scales = cso.quantize_fp8_ue8m0(lat)
        want_lat = orc.e4m3fn_to_f64(codes) * np.repeat(orc.ue8m0_to_f64(scales), 64, axis=1)
    else:
        want_lat = orc.bf16_bits_to_f64(lat)
    if kv_format != oracle.KV_FP8_TENSOR:
        assert np.array_equal(rows[:, :512], want_lat[keep])
        assert np.array_equal(rows[:, 512:], orc.bf16_bits_to_f64(rope)[keep])
    # every byte outside the written entries is untouched
    mask = np.ones_like(cache, dtype=bool)
    for s in written:
        page, r = divmod(s, ps)
        if kv_format == oracle.KV_FP8_UE8M0:
            mask[page, r * 512:(r + 1) * 512] = False
            mask[page, 512 * ps + r * 128: 512 * ps + (r + 1) * 128] = False
            mask[page, 640 * ps + r * 8: 640 * ps + (r + 1) * 8] = False
        elif kv_format == oracle.KV_FP8_TENSOR:
            mask[page, r * 576:(r + 1) * 576] = False
        else:
            mask[page, r * 1152:(r + 1) * 1152] = False
    assert np.array_equal(out[mask], cache[mask])


def test_fp8_store_fixture_bytes_by_hand():
    # latent 1.0 everywhere except dim 0 = -3.0 and the second group all 0.5
    lat = np.full(512, 1.0)
    lat[0] = -3.0
    lat[64:128] = 0.5
    codes, scales = cso.quantize_fp8_ue8m0(_bf16_bits(lat[None]))
    # group 0: amax 3.0, smallest e with 448 * 2^(e-127) >= 3 is e - 127 = -7 (3.5);
    # 1.0 / 2^-7 = 128 = 1.0 * 2^7 -> e4m3 exponent field 7 + 7 = 14, mantissa 0 -> 0x70;
    # -3.0 / 2^-7 = -384 = -1.5 * 2^8 -> 0x80 | (15 << 3) | 4 = 0xFC
    assert scales[0, 0] == 120 and codes[0, 1] == 0x70 and codes[0, 0] == 0xFC
    # group 1: amax 0.5 -> e - 127 = -9 (448 * 2^-9 = 0.875), 0.5 / 2^-9 = 256 -> 0x78
    assert scales[0, 1] == 118 and codes[0, 64] == 0x78


# ---------------------------------------------------------------- per-tensor FP8 store

def test_fp8_tensor_store_by_hand():
    # kv_scale 0.25: 1.0 -> 4.0 = 0x48; -3.0 -> -12 = -1.5 * 2^3 -> 0x80 | (10 << 3) | 4 = 0xD4;
    # 1000 -> 4000, saturated at 448 = 0x7E; 2^-12 -> 2^-10, half the smallest subnormal:
    # a tie, to the even code 0x00; -0.0 -> 0x80; bf16(0.3) = 0.30078125 -> 1.203125, nearer
    # 1.25 (0x3A) than 1.125 (0x39).  The rope (dims 512..575) is quantized the same way.
    lat = np.zeros(512)
    lat[:6] = [1.0, -3.0, 1000.0, 2.0 ** -12, -0.0, 0.3]
    rope = np.zeros(64)
    rope[0], rope[63] = -1000.0, 0.5
    codes = cso.quantize_fp8_tensor(_bf16_bits(lat[None]), _bf16_bits(rope[None]), 0.25)
    assert codes[0, :6].tolist() == [0x48, 0xD4, 0x7E, 0x00, 0x80, 0x3A]
    assert codes[0, 512] == 0xFE and codes[0, 575] == 0x40       # -448 and 2.0
    assert np.all(codes[0, 6:512] == 0) and np.all(codes[0, 513:575] == 0)


@pytest.mark.parametrize("kv_scale", [1.0, 0.25, 1.0 / 64, 0.037, 3.3])
def test_fp8_tensor_store_matches_torch_cast_of_the_float32_quotient(kv_scale):
    """The reading's two steps against library routines: torch's float32 division, clamp,
    and round-to-nearest-even cast to float8_e4m3fn."""
    rng = np.random.default_rng(int(kv_scale * 1000))
    x = rng.standard_normal((40, 576)) * np.exp2(rng.integers(-12, 12, (40, 1)))
    bits = _bf16_bits(x)
    codes = cso.quantize_fp8_tensor(bits[:, :512], bits[:, 512:], kv_scale)
    xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    ref = torch.clamp(xt / torch.tensor(kv_scale, dtype=torch.float32), -448.0, 448.0)
    assert np.array_equal(codes, ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy())


def test_fp8_tensor_store_rejects_bad_scales():
    lat, rope = _bf16_bits(np.zeros((1, 512))), _bf16_bits(np.zeros((1, 64)))
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            cso.quantize_fp8_tensor(lat, rope, bad)
