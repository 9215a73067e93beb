"""GPU parity of the cache store (sparse_mla_cache_store through the C ABI) against the
cache-store oracle: the written cache must be bit-identical (codes, scale bytes, rope
bytes, untouched bytes elsewhere)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle import cache_store_oracle as cso
from oracle import sparse_mla_oracle as orc
from sparse_mla_decode_03_amd import binding as B
from tests.gpu_util import announce

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda")


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def _latent_with_edge_groups(n: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((n, 512), generator=g)
    x[0, :64] = 0.0                                    # all-zero group
    x[0, 64:128] = -0.0                                # negative zeros
    if n > 1:
        x[1, :64] *= 1e-30                             # tiny values (subnormal codes)
        x[1, 64:128] *= 1e20                           # large values
        # a group whose scale is exactly 1 (amax 448) with values on code midpoints: ties
        pos = torch.from_numpy(orc.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))).float()
        mids = ((pos[:-1] + pos[1:]) / 2)[-63:]
        x[1, 128:192] = torch.cat([torch.tensor([448.0]), mids])
    if n > 2:
        x[2, :] = torch.linspace(-448.0, 448.0, 512)
    if n > 3:
        # every midpoint between consecutive positive codes (subnormal ones included), then
        # their negatives, four groups of scale 1 (each led by 448)
        pos = torch.from_numpy(orc.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))).float()
        mids = (pos[:-1] + pos[1:]) / 2                # 126 ties
        for k, part in enumerate((mids[:63], mids[63:], -mids[:63], -mids[63:])):
            x[3, 64 * k:64 * k + 64] = torch.cat([torch.tensor([448.0]), part])
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("fmt,ps", [("fp8", 2), ("fp8", 64), ("bf16", 1), ("bf16", 64)])
def test_store_bit_exact_against_oracle(fmt, ps):
    kvf = B.KV_FP8_UE8M0 if fmt == "fp8" else B.KV_BF16
    n = 37 if ps > 2 else 9
    npages = max(7, 2 * n // ps + 1)
    rng = np.random.default_rng(ps + kvf)
    pb = orc.page_bytes(kvf, ps)
    cache0 = rng.integers(0, 256, (npages, pb), dtype=np.uint8)
    lat = _latent_with_edge_groups(n, 3 + ps)
    rope = torch.randn((n, 64), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    slots = rng.choice(npages * ps, n, replace=False).astype(np.int32)
    slots[n // 2] = -1
    slots[n // 3] = npages * ps + 5                    # past the cache: skipped
    announce(f"cache_store {fmt} ps={ps} n={n}")
    cache = torch.from_numpy(cache0).to(DEV)
    B.cache_store(cache, fmt, ps, lat.to(DEV), rope.to(DEV), torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    want = cso.cache_store(cache0, kvf, ps, _bits(lat), _bits(rope), slots)
    got = cache.cpu().numpy()
    assert np.array_equal(got, want), f"{int((got != want).sum())} bytes differ"


def test_store_then_gather_reads_the_quantized_rows():
    ps, npages, n = 64, 16, 500
    kvf = B.KV_FP8_UE8M0
    cache = torch.zeros((npages, orc.page_bytes(kvf, ps)), dtype=torch.uint8, device=DEV)
    lat = torch.randn((n, 512), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    rope = torch.randn((n, 64), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    slots = torch.randperm(npages * ps, generator=torch.Generator().manual_seed(3))[:n].to(torch.int32)
    announce("cache_store then gather_debug")
    B.cache_store(cache, "fp8", ps, lat.to(DEV), rope.to(DEV), slots.to(DEV))
    rows = B.gather_debug(cache, "fp8", ps, slots.to(DEV)).cpu().double().numpy()
    codes, scales = cso.quantize_fp8_ue8m0(_bits(lat))
    want = orc.e4m3fn_to_f64(codes) * np.repeat(orc.ue8m0_to_f64(scales), 64, axis=1)
    assert np.array_equal(rows[:, :512], want)
    assert np.array_equal(rows[:, 512:], rope.double().numpy())


def test_store_full_size_sampled():
    """One decode step's worth of new tokens for the 128-request MTP workload (512 tokens)
    and a prefill-sized batch (65 536 tokens) into a 5.7 GB-sized pool; sampled tokens are
    checked bit-exactly."""
    ps, npages = 64, 137714
    kvf = B.KV_FP8_UE8M0
    cache = torch.zeros((npages, orc.page_bytes(kvf, ps)), dtype=torch.uint8, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(4)
    for n in (512, 65536):
        lat = torch.randn((n, 512), generator=g, device=DEV).to(torch.bfloat16)
        rope = torch.randn((n, 64), generator=g, device=DEV).to(torch.bfloat16)
        slots = torch.randperm(npages * ps, generator=g, device=DEV)[:n].to(torch.int32)
        announce(f"cache_store full size n={n}")
        B.cache_store(cache, "fp8", ps, lat, rope, slots)
        torch.cuda.synchronize()
        pick = np.random.default_rng(n).choice(n, 64, replace=False)
        sl = slots.cpu().numpy()[pick]
        codes, scales = cso.quantize_fp8_ue8m0(_bits(lat[pick]))
        pages = torch.from_numpy(sl // ps).long().to(DEV)
        got = cache.index_select(0, pages).cpu().numpy()
        for i, s in enumerate(sl):
            r = int(s) % ps
            assert np.array_equal(got[i, r * 512:(r + 1) * 512], codes[i])
            assert np.array_equal(got[i, 640 * ps + r * 8: 640 * ps + (r + 1) * 8], scales[i])
            assert np.array_equal(got[i, 512 * ps + r * 128: 512 * ps + (r + 1) * 128],
                                  _bits(rope[pick[i]:pick[i] + 1]).view(np.uint8).reshape(-1))
