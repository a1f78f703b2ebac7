"""Pins for the oracle's KV write and its E4M3 codec (CPU only).

Write: the page's statement is that a token's K/V land in its slot (physical
block, offset) and nothing else is touched ("PagedAttention, clearly
explained"; "What problem does PagedAttention solve...", section "The paging
idea").  The check views the cache [NB, H, bs, D] as [NB*bs, H, D] slots with a
numpy transpose/reshape, so it does not reuse the oracle's index arithmetic.

Codec: decode is checked against torch's float8_e4m3fn (a library decoder of
the same OCP format) and a few values fixed by the format; encode is checked by
brute force (nearest of the 256 codes, ties to the even code, saturation) over
every bfloat16 bit pattern at several scales, and against torch's cast.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_from_f32, bf16_to_f32


def _slots_view(cache: np.ndarray) -> np.ndarray:
    NB, H, bs, D = cache.shape
    return cache.transpose(0, 2, 1, 3).reshape(NB * bs, H, D)


@pytest.mark.parametrize("elem", ["f32", "bf16"])
def test_write_places_rows_in_their_slots_and_nothing_else(elem):
    rng = np.random.default_rng(20)
    NB, H, bs, D, T = 9, 3, 16, 8, 40
    x = rng.standard_normal((T, H, D)).astype(np.float32)
    y = rng.standard_normal((T, H, D)).astype(np.float32)
    if elem == "bf16":
        x, y = bf16_bits_from_f32(x), bf16_bits_from_f32(y)
    cache_k = rng.standard_normal((NB, H, bs, D)).astype(np.float32)
    cache_v = rng.standard_normal((NB, H, bs, D)).astype(np.float32)
    if elem == "bf16":
        cache_k, cache_v = bf16_bits_from_f32(cache_k), bf16_bits_from_f32(cache_v)
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int32)
    slots[[3, 17]] = -1  # padding tokens are skipped
    before_k, before_v = cache_k.copy(), cache_v.copy()
    oracle.paged_kv_write(x, y, slots, cache_k, cache_v)
    live = slots >= 0
    assert np.array_equal(_slots_view(cache_k)[slots[live]].view(np.uint8),
                          x[live].view(np.uint8))
    assert np.array_equal(_slots_view(cache_v)[slots[live]].view(np.uint8),
                          y[live].view(np.uint8))
    untouched = np.ones(NB * bs, bool)
    untouched[slots[live]] = False
    assert np.array_equal(_slots_view(cache_k)[untouched].view(np.uint8),
                          _slots_view(before_k)[untouched].view(np.uint8))
    assert np.array_equal(_slots_view(cache_v)[untouched].view(np.uint8),
                          _slots_view(before_v)[untouched].view(np.uint8))


def test_write_rejects_slot_outside_pool():
    k = np.zeros((2, 1, 4), np.float32)
    cache = np.zeros((2, 1, 16, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.paged_kv_write(k, k, np.array([0, 32], np.int32), cache, cache.copy())


def test_write_quantizes_with_f32_product_then_rounds():
    rng = np.random.default_rng(21)
    NB, H, bs, D, T = 6, 2, 16, 32, 50
    x = bf16_bits_from_f32(rng.standard_normal((T, H, D)).astype(np.float32) * 3)
    x[0, 0, :4] = bf16_bits_from_f32(np.array([1e6, -1e6, 0.0, -0.0], np.float32))
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int32)
    ck = np.full((NB, H, bs, D), 0x7F, np.uint8)
    cv = ck.copy()
    scale = np.float32(0.0173)
    oracle.paged_kv_write(x, x, slots, ck, cv, k_scale=float(scale), v_scale=float(scale))
    inv = np.float32(1.0) / scale
    y = bf16_to_f32(x) * inv  # float32 product, round to nearest even
    lib = torch.from_numpy(np.clip(y, -448.0, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(_slots_view(ck)[slots], lib.numpy())
    assert np.array_equal(ck, cv)
    assert _slots_view(ck)[slots[0], 0, 0] == 0x7E and _slots_view(ck)[slots[0], 0, 1] == 0xFE
    assert _slots_view(ck)[slots[0], 0, 2] == 0x00 and _slots_view(ck)[slots[0], 0, 3] == 0x80


def test_e4m3_decode_matches_library_and_format():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], lib[~nan])
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6 and ours[0x38] == 1.0
    assert ours[0x80] == 0.0 and np.signbit(ours[0x80])


def _brute_force_encode(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code by search: ties go to the code with an even mantissa,
    magnitudes beyond the largest finite saturate, NaN gives 0x7F."""
    mags = _finite_magnitudes()
    a = np.abs(y.astype(np.float64))
    idx = np.searchsorted(mags, a)  # mags[idx-1] < a <= mags[idx]
    idx = np.clip(idx, 1, len(mags) - 1)
    lo, hi = mags[idx - 1], mags[idx]
    dlo, dhi = a - lo, hi - a
    pick = np.where(dlo < dhi, idx - 1, idx)
    tie = dlo == dhi
    pick = np.where(tie & ((idx - 1) % 2 == 0), idx - 1, np.where(tie, idx, pick))
    pick = np.where(a >= mags[-1], len(mags) - 1, pick)
    pick = np.where(a <= mags[0], 0, pick)
    code = pick.astype(np.uint8) | np.where(np.signbit(y), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(y), np.uint8(0x7F), code).astype(np.uint8)


def _finite_magnitudes():
    # the 127 non-negative finite codes 0x00..0x7E, in increasing order; their
    # values come from torch's decoder, so code index = position in the list
    codes = np.arange(0x7F, dtype=np.uint8)
    return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("scale", [1.0, 0.0173, 1.0 / 448.0, 3.5, 2.0 ** -10])
def test_e4m3_encode_brute_force_over_all_bf16(scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bf16_to_f32(bits)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(invalid="ignore", over="ignore"):
        y = (x * inv).astype(np.float32)
    ours = oracle.e4m3_encode(y)
    ref = _brute_force_encode(y)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"first mismatch y={y[bad[0]]!r} ours={ours[bad[0]]:#x} ref={ref[bad[0]]:#x}"


def test_e4m3_encode_matches_library_in_range_and_round_trips():
    rng = np.random.default_rng(22)
    y = (rng.standard_normal(200000) * 40).astype(np.float32)
    y = y[np.abs(y) < 448]
    ours = oracle.e4m3_encode(y)
    lib = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, lib)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    back = oracle.e4m3_encode(oracle.e4m3_decode(finite).astype(np.float32))
    assert np.array_equal(back, finite)


def test_write_uses_product_with_f32_inverse():
    # bf16 0x3b90 at scale 0.3: the f32 product x * (1/scale) and the correctly
    # rounded quotient x / scale land on different E4M3 codes; the write uses the
    # product (inverse formed once in f32)
    x = np.array([[[0x3B90, 0xBB90]]], np.uint16)
    s = np.float32(0.3)
    ck = np.zeros((1, 1, 16, 2), np.uint8)
    cv = ck.copy()
    oracle.paged_kv_write(x, x, np.array([5], np.int32), ck, cv, k_scale=float(s),
                          v_scale=float(s))
    xf = bf16_to_f32(x[0, 0])
    prod = (xf * (np.float32(1.0) / s)).astype(np.float32)
    quot = (xf.astype(np.float64) / np.float64(s)).astype(np.float32)
    lib = lambda a: torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert not np.array_equal(lib(prod), lib(quot))
    assert np.array_equal(ck[0, 0, 5], lib(prod))
