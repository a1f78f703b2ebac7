"""GPU parity of the slot-mapped KV write: bit-exact against the oracle.

Every byte of both pools is compared, including the untouched (poisoned)
slots, so a write outside its slot or a skipped padding token shows up."""
import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


def _compare_pools(g: gu.GpuCase, kc, vc, what):
    gk, gv = gu.host(g.kc), gu.host(g.vc)
    assert np.array_equal(gk.view(np.uint8), kc.view(np.uint8)), f"{what}: key pool differs"
    assert np.array_equal(gv.view(np.uint8), vc.view(np.uint8)), f"{what}: value pool differs"


def test_c1_f32_write_of_every_token():
    case = workloads.c1_tiny_f32()
    g = gu.GpuCase(case)
    g.fill_and_step_writes()
    kc, vc = gu.oracle_caches(case)
    _compare_pools(g, kc, vc, "c1")


# head dims 64 / 128 / 256 take the row kernel (power-of-two block sizes by
# shift, others by division); 96 takes the general kernel
@pytest.mark.parametrize("elem,bs,H,D", [("bf16", 16, 4, 128), ("bf16", 32, 8, 64),
                                         ("f32", 16, 2, 128), ("bf16", 64, 1, 128),
                                         ("bf16", 24, 3, 128), ("f32", 12, 2, 64),
                                         ("bf16", 16, 2, 96), ("f32", 8, 2, 256),
                                         ("bf16", 16, 2, 256)])
def test_random_slots_with_padding(elem, bs, H, D):
    rng = np.random.default_rng(bs * 7 + H)
    NB, T = 97, 700
    npdt = np.float32 if elem == "f32" else np.uint16
    poison = workloads.F32_NAN_BITS.view(np.float32) if elem == "f32" else workloads.BF16_NAN
    kc = np.full((NB, H, bs, D), poison, npdt)
    vc = kc.copy()
    k = np.empty((T, H, D), npdt)
    v = np.empty_like(k)
    workloads.fill_normal(k, 1.0, 5, 1)
    workloads.fill_normal(v, 1.0, 5, 2)
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int32)
    slots[rng.choice(T, size=31, replace=False)] = -1
    case = workloads.PagedCase(name="w", cache_dtype=elem, q=np.zeros((0, 1, D), npdt),
                               key_cache=kc, value_cache=vc,
                               block_tables=np.zeros((0, 1), np.int32),
                               context_lens=np.zeros(0, np.int32), block_size=bs, scale=1.0,
                               k_new=k, v_new=v, slot_mapping=slots)
    g = gu.GpuCase(case)
    g.fill_and_step_writes()
    okc, ovc = gu.oracle_caches(case)
    _compare_pools(g, okc, ovc, f"{elem} bs{bs}")


# 1e-39 is a subnormal scale: 1 / scale overflows to inf in f32, so zeros
# quantize to NaN (0x7F); head dim 96 takes the general kernel
@pytest.mark.parametrize("scale", [1.0, 0.0173, 1.0 / 448.0, 3.5, 2.0 ** -10, 0.3, 1e-39])
@pytest.mark.parametrize("elem", ["bf16", "f32"])
@pytest.mark.parametrize("bs,D", [(16, 128), (12, 64), (32, 256), (16, 96)])
def test_e4m3_quantizing_write_over_every_bf16_value(scale, elem, bs, D):
    # all 65536 bf16 bit patterns (NaN, inf, subnormals, both zeros) as rows of
    # D values, one per token, quantized with the per-tensor scale
    T = -(-65536 // D)  # rows of D values covering every pattern (wrapping around)
    bits = (np.arange(T * D, dtype=np.uint32) % 65536).astype(np.uint16)
    if elem == "f32":
        vals = workloads.bf16_to_f32(bits)
    else:
        vals = bits
    k = vals.reshape(T, 1, D)
    v = k[::-1].copy()
    NB = (T + bs - 1) // bs + 8
    slots = np.random.default_rng(1).choice(NB * bs, size=T, replace=False).astype(np.int32)
    kc = np.full((NB, 1, bs, D), 0x7F, np.uint8)
    vc = kc.copy()
    case = workloads.PagedCase(name="e4m3", cache_dtype="fp8_e4m3", q=np.zeros((0, 1, D), np.uint16),
                               key_cache=kc, value_cache=vc,
                               block_tables=np.zeros((0, 1), np.int32),
                               context_lens=np.zeros(0, np.int32), block_size=bs, scale=1.0,
                               k_scale=scale, v_scale=scale * 2, k_new=k, v_new=v,
                               slot_mapping=slots)
    g = gu.GpuCase(case)
    g.fill_and_step_writes()
    okc, ovc = gu.oracle_caches(case)
    _compare_pools(g, okc, ovc, f"e4m3 scale {scale}")


def test_c5_prefill_chunk_and_whole_fill_full_size():
    # the whole-pool fill (528k tokens quantized to E4M3) and the 4096-token
    # bf16 prefill chunk into random free slots: every byte of both pools
    case = workloads.c5_fp8()
    g = gu.GpuCase(case)
    g.fill_and_step_writes()
    okc, ovc = gu.oracle_caches(case)
    assert case.block_size == 16 and case.slot_mapping.size == 4096
    _compare_pools(g, okc, ovc, "c5 fill + chunk")
