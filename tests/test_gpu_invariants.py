"""Bit-level invariants of the HIP decode path, from the pages: output is
identical given the same reduction order, wherever the blocks sit
("pipe-paged-block-allocation-kv-cache", section "In and out"); slots past a
sequence and recycled blocks never reach the output ("PagedAttention, clearly
explained").  Also determinism across repeated launches."""
import math

import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

MODES = [("single", 0, 4, 0), ("partitioned", 64, 2, 0), ("partitioned", 512, 4, 0),
         ("balanced", 0, 0, 0), ("balanced", 0, 0, 13)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


def _case(poison=True, dtype="bf16", seed=21):
    return workloads.build_case("inv", seed=seed, context_lens=[1, 33, 200, 1000, 47, 16],
                                num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                                cache_dtype=dtype, std=0.5, scale=1.0 / math.sqrt(128),
                                poison=poison)


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_physical_block_permutation_is_bit_identical(dtype):
    case = _case(dtype=dtype)
    g = gu.GpuCase(case)
    g.fill_and_step_writes()
    kc, vc = gu.host(g.kc), gu.host(g.vc)
    pi = np.random.default_rng(2).permutation(case.num_blocks).astype(np.int32)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi], vc2[pi] = kc, vc
    g2 = gu.GpuCase(case)
    g2.kc, g2.vc = gu.dev(kc2), gu.dev(vc2)
    g2.tables = gu.dev(pi[case.block_tables])
    for m in MODES:
        a = gu.host(g.decode_mode(m)).copy()
        b = gu.host(g2.decode_mode(m))
        assert np.array_equal(a, b), m


def test_poisoned_tails_and_free_blocks_do_not_change_bits():
    poisoned = gu.GpuCase(_case(poison=True))
    clean = gu.GpuCase(_case(poison=False))
    poisoned.fill_and_step_writes()
    clean.fill_and_step_writes()
    for m in MODES:
        a = gu.host(poisoned.decode_mode(m)).copy()
        b = gu.host(clean.decode_mode(m))
        assert np.array_equal(a, b), m
        assert np.all(np.isfinite(gu.as_f64(a)))


def test_repeated_launches_are_deterministic():
    g = gu.GpuCase(_case())
    g.fill_and_step_writes()
    for m in MODES:
        first = gu.host(g.decode_mode(m)).copy()
        for _ in range(3):
            assert np.array_equal(gu.host(g.decode_mode(m)), first)


def test_contiguous_table_gives_the_same_bits():
    case = _case()
    g = gu.GpuCase(case)
    g.fill_and_step_writes()
    kc, vc = gu.host(g.kc), gu.host(g.vc)
    nbs = (case.context_lens.astype(np.int64) + 15) // 16
    order = np.concatenate([case.block_tables[s, :nbs[s]] for s in range(case.num_seqs)])
    t2 = np.zeros_like(case.block_tables)
    c = 0
    for s in range(case.num_seqs):
        t2[s, :nbs[s]] = np.arange(c, c + nbs[s])
        c += nbs[s]
    g2 = gu.GpuCase(case)
    g2.kc, g2.vc, g2.tables = gu.dev(kc[order]), gu.dev(vc[order]), gu.dev(t2)
    for m in MODES:
        assert np.array_equal(gu.host(g.decode_mode(m)).copy(), gu.host(g2.decode_mode(m)))
