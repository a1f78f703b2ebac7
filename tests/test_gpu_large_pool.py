"""Pools larger than 2^31 elements and 4 GiB: every kernel addresses blocks with
64-bit offsets.

A small seeded case is laid out as usual, and the oracle runs on its compact
pool.  On the GPU the same blocks sit at the top of a pool of NB_BIG blocks:
physical id b becomes b + shift, so every block the kernels touch starts past
element 2^31 and past byte 2^32.  That is a relabelling of physical ids, under
which the results are unchanged (writes and copies bit for bit, attention
within the usual tolerance).  Covered: the KV write, decode in every mode, the
one-call append step, the shared-prefix decode, chunked prefill, copy-on-write
copies and the swap gather and scatter."""
import math

import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
torch = gu.torch
import paged_kv_cache_135_amd as pkv  # noqa: E402

HKV, BS, D = 2, 16, 128
ELEMS_PER_BLOCK = HKV * BS * D  # 4,096
# bf16: 540,000 blocks of 8 KiB (4.4 GB per pool); E4M3: 1,100,000 blocks of 4 KiB (4.5 GB)
NB_BIG = {"bf16": 540_000, "fp8_e4m3": 1_100_000}
TORCH_DT = {"bf16": torch.bfloat16, "fp8_e4m3": torch.uint8}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


class BigPool:
    """The case's pool placed at the top of an NB_BIG-block pool on the GPU."""

    def __init__(self, case):
        dt = case.cache_dtype
        self.case = case
        nb = case.key_cache.shape[0]
        self.shift = NB_BIG[dt] - nb
        first = self.shift * ELEMS_PER_BLOCK
        assert first > 2**31 and first * case.key_cache.itemsize > 2**32
        shape = (NB_BIG[dt], HKV, BS, D)
        self.kc = torch.empty(shape, dtype=TORCH_DT[dt], device="cuda")
        self.vc = torch.empty_like(self.kc)
        self.kc[self.shift:].copy_(gu.dev(case.key_cache).view(TORCH_DT[dt]))
        self.vc[self.shift:].copy_(gu.dev(case.value_cache).view(TORCH_DT[dt]))
        self.tables = gu.dev(case.block_tables + np.int32(self.shift))
        self.lens = gu.dev(case.context_lens)
        self.q = gu.dev(case.q)

    def slots(self, slots):
        s = slots.astype(np.int64)
        return gu.dev(np.where(s >= 0, s + self.shift * BS, s).astype(slots.dtype))

    def top(self, t):
        """The relabelled part of a pool, in the case's dtype, on the host."""
        x = t[self.shift:]
        if self.case.cache_dtype == "bf16":
            return gu.host(x)
        return x.cpu().numpy()

    def write(self, k, v, slots):
        c = self.case
        pkv.paged_kv_write(gu.dev(k), gu.dev(v), self.slots(slots), self.kc, self.vc,
                           k_scale=c.k_scale, v_scale=c.v_scale)

    def free(self):
        del self.kc, self.vc
        torch.cuda.empty_cache()


def _decode_case(dt, shared_prefix_blocks=0, seed=71):
    lens = [1, 17, 300, 1000, 2049, 64] if not shared_prefix_blocks else [130, 200, 64, 333]
    return workloads.build_case(f"large_pool_{dt}", seed=seed, context_lens=lens,
                                num_q_heads=8, num_kv_heads=HKV, head_dim=D, block_size=BS,
                                cache_dtype=dt, std=0.5, scale=1.0 / math.sqrt(D),
                                shared_prefix_blocks=shared_prefix_blocks, fill_via_write=True)


@pytest.fixture(scope="module", params=["bf16", "fp8_e4m3"])
def written(request):
    """(case, big pool after the case's writes, oracle pools after the same writes)."""
    case = _decode_case(request.param)
    big = BigPool(case)
    if case.fill_k is not None:
        big.write(case.fill_k, case.fill_v, case.fill_slots)
    if case.k_new is not None:
        big.write(case.k_new, case.v_new, case.slot_mapping)
    torch.cuda.synchronize()
    okc, ovc = gu.oracle_caches(case)
    yield case, big, okc, ovc
    big.free()


def test_write_lands_past_4gib(written):
    case, big, okc, ovc = written
    assert np.array_equal(big.top(big.kc), okc)
    assert np.array_equal(big.top(big.vc), ovc)


@pytest.mark.parametrize("mode", [("auto", 0, 0, 0), ("single", 0, 4, 0),
                                  ("partitioned", 512, 4, 0), ("balanced", 0, 0, 64)])
def test_decode_modes(written, mode):
    case, big, okc, ovc = written
    kc, vc = big.kc, big.vc
    name, part, waves, workers = mode
    out = torch.empty_like(big.q)
    pkv.paged_attention_decode(out, big.q, kc, vc, big.tables, big.lens, case.scale, BS,
                               k_scale=case.k_scale, v_scale=case.v_scale,
                               mode=None if name == "auto" else name, partition_size=part,
                               waves_per_group=waves, num_workers=workers)
    gu.assert_close(gu.host(out), gu.oracle_decode(case, okc, ovc), case.cache_dtype,
                    f"decode {name}")


@pytest.mark.parametrize("dt", ["bf16", "fp8_e4m3"])
def test_append_step(dt):
    """The step's write folded into the decode, at slots past 4 GiB."""
    case = _decode_case(dt, seed=72)
    big = BigPool(case)
    try:
        if case.fill_k is not None:
            big.write(case.fill_k, case.fill_v, case.fill_slots)
        kc, vc = big.kc, big.vc
        out = torch.empty_like(big.q)
        pkv.paged_attention_decode_append(out, big.q, gu.dev(case.k_new), gu.dev(case.v_new),
                                          big.slots(case.slot_mapping), kc, vc, big.tables,
                                          big.lens, case.scale, BS, k_scale=case.k_scale,
                                          v_scale=case.v_scale)
        okc, ovc = gu.oracle_caches(case)
        gu.assert_close(gu.host(out), gu.oracle_decode(case, okc, ovc), dt, "append step")
        assert np.array_equal(big.top(big.kc), okc)
        assert np.array_equal(big.top(big.vc), ovc)
    finally:
        big.free()


def test_shared_prefix_decode():
    case = _decode_case("bf16", shared_prefix_blocks=4, seed=73)
    big = BigPool(case)
    try:
        big.write(case.fill_k, case.fill_v, case.fill_slots)
        big.write(case.k_new, case.v_new, case.slot_mapping)
        out = torch.empty_like(big.q)
        pkv.paged_attention_decode_shared_prefix(out, big.q, big.kc, big.vc, big.tables,
                                                 big.lens, 4 * BS, case.scale, BS)
        okc, ovc = gu.oracle_caches(case)
        gu.assert_close(gu.host(out), gu.oracle_decode(case, okc, ovc), "bf16",
                        "shared-prefix decode")
    finally:
        big.free()


def test_chunked_prefill():
    import oracle
    case = workloads.build_prefill_case("large_pool_prefill", seed=74,
                                        prefix_lens=[0, 100, 517], chunk_lens=[40, 77, 129],
                                        num_q_heads=8, num_kv_heads=HKV, head_dim=D,
                                        block_size=BS, cache_dtype="bf16", std=0.5,
                                        scale=1.0 / math.sqrt(D))
    big = BigPool(case)
    try:
        if case.fill_k is not None:
            big.write(case.fill_k, case.fill_v, case.fill_slots)
        if case.k_new is not None:
            big.write(case.k_new, case.v_new, case.slot_mapping)
        out = torch.empty_like(big.q)
        mql = int(np.diff(case.query_start).max())
        pkv.paged_attention_prefill(out, big.q, big.kc, big.vc, big.tables, big.lens,
                                    gu.dev(case.query_start), mql, case.scale, BS)
        okc, ovc = gu.oracle_caches(case)
        ref = oracle.paged_attention_prefill(case.q, okc, ovc, case.block_tables,
                                             case.context_lens, case.query_start, case.scale,
                                             BS, case.k_scale, case.v_scale)
        gu.assert_close(gu.host(out), ref, "bf16", "prefill")
    finally:
        big.free()


def test_copy_and_swap_blocks(written):
    """Copy-on-write pairs and the swap gather / scatter between ids past 4 GiB."""
    case, big, okc, ovc = written
    rng = np.random.default_rng(75)
    nb = okc.shape[0]
    ids = rng.permutation(nb).astype(np.int32)
    src, dst = ids[:6], ids[6:12]
    # gather: staging slot i holds block src[i]
    sk = torch.empty((len(src), HKV, BS, D), dtype=big.kc.dtype, device="cuda")
    sv = torch.empty_like(sk)
    kc, vc = big.kc, big.vc
    pkv.paged_kv_gather_blocks(kc, vc, gu.dev(src + np.int32(big.shift)), sk, sv)
    assert np.array_equal(gu.host(sk).reshape(okc[src].shape), okc[src])
    assert np.array_equal(gu.host(sv).reshape(ovc[src].shape), ovc[src])
    # copy-on-write: dst becomes a copy of src
    pairs = np.stack([src, dst], axis=1).astype(np.int32) + np.int32(big.shift)
    pkv.paged_kv_copy_blocks(kc, vc, gu.dev(pairs))
    want_k, want_v = okc.copy(), ovc.copy()
    want_k[dst], want_v[dst] = okc[src], ovc[src]
    assert np.array_equal(big.top(big.kc), want_k)
    assert np.array_equal(big.top(big.vc), want_v)
    # scatter: blocks ids[12:18] receive the staged copies of src
    dst2 = ids[12:18]
    pkv.paged_kv_scatter_blocks(sk, sv, gu.dev(dst2 + np.int32(big.shift)), kc, vc)
    want_k[dst2], want_v[dst2] = okc[src], ovc[src]
    assert np.array_equal(big.top(big.kc), want_k)
    assert np.array_equal(big.top(big.vc), want_v)
    # put the written pool back for the fixture's other tests
    big.kc[big.shift:].copy_(gu.dev(okc).view(big.kc.dtype))
    big.vc[big.shift:].copy_(gu.dev(ovc).view(big.vc.dtype))
