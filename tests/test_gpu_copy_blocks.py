"""GPU parity of the copy-on-write block copy: byte-exact against the oracle,
and the fork -> copy -> write -> decode sequence against the oracle doing the
same steps."""
import math

import numpy as np
import pytest

import oracle
import paged_kv_cache_135_amd as pkv
import workloads
from paged_kv_cache_135_amd import BlockPool
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


@pytest.mark.parametrize("elem,H,bs,D", [("bf16", 4, 16, 128), ("f32", 2, 32, 64),
                                         ("fp8_e4m3", 8, 16, 128)])
def test_copy_blocks_bit_exact(elem, H, bs, D):
    rng = np.random.default_rng(40)
    NB = 300
    npdt = {"bf16": np.uint16, "f32": np.float32, "fp8_e4m3": np.uint8}[elem]
    kc = rng.integers(0, 256, size=(NB, H, bs, D) + ((4,) if elem == "f32" else (2,) if elem == "bf16" else ()),
                      dtype=np.uint8).view(npdt).reshape(NB, H, bs, D)
    vc = rng.integers(0, 256, size=kc.nbytes, dtype=np.uint8).view(npdt).reshape(NB, H, bs, D)
    perm = rng.permutation(NB).astype(np.int32)
    pairs = np.stack([perm[:100], perm[100:200]], axis=1)
    pairs[[5, 17], 0] = -1          # padding rows
    pairs[40, 1] = pairs[40, 0]     # no-op row
    pkv.validate_block_pairs(pairs, NB)
    gk, gv = gu.dev(kc), gu.dev(vc)
    pkv.paged_kv_copy_blocks(gk, gv, gu.dev(pairs))
    ok, ov = kc.copy(), vc.copy()
    oracle.copy_blocks(ok, ov, pairs)
    assert np.array_equal(gu.host(gk).view(np.uint8), ok.view(np.uint8))
    assert np.array_equal(gu.host(gv).view(np.uint8), ov.view(np.uint8))


def test_fork_copy_on_write_write_decode():
    # 5 answers to one 1990-token prompt (refcount 5 on the prompt blocks); each
    # branch generates 3 tokens; copies, writes and decodes run on the GPU and
    # in the oracle, each from its own pool
    rng = np.random.default_rng(41)
    Hq, H, D, bs, NB = 32, 8, 128, 16, 256
    pool = BlockPool(NB, bs)
    prompt_k = np.empty((1990, H, D), np.uint16)
    prompt_v = np.empty_like(prompt_k)
    workloads.fill_normal(prompt_k, 0.5, 41, 1)
    workloads.fill_normal(prompt_v, 0.5, 41, 2)
    kc = np.full((NB, H, bs, D), workloads.BF16_NAN, np.uint16)
    vc = kc.copy()
    gk, gv = gu.dev(kc), gu.dev(vc)
    slots = pool.allocate("p", 1990)
    pkv.paged_kv_write(gu.dev(prompt_k), gu.dev(prompt_v), gu.dev(slots), gk, gv)
    oracle.paged_kv_write(prompt_k, prompt_v, slots, kc, vc)
    seqs = ["p"] + [f"f{i}" for i in range(4)]
    for q in seqs[1:]:
        pool.fork("p", q)
    q = np.empty((5, Hq, D), np.uint16)
    workloads.fill_normal(q, 0.5, 41, 3)
    out = gu.torch.empty_like(gu.dev(q))
    n_copies = 0
    for step in range(3):
        new_slots, pairs = [], []
        for name in seqs:
            sl, cow = pool.append(name)
            new_slots.append(sl[0])
            pairs += cow
        n_copies += len(pairs)
        if pairs:
            pr = np.array(pairs, np.int32)
            pkv.validate_block_pairs(pr, NB)
            pkv.paged_kv_copy_blocks(gk, gv, gu.dev(pr))
            oracle.copy_blocks(kc, vc, pr)
        nk = np.empty((5, H, D), np.uint16)
        nv = np.empty_like(nk)
        workloads.fill_normal(nk, 0.5, 41, 10 + step)
        workloads.fill_normal(nv, 0.5, 41, 20 + step)
        ns = np.array(new_slots, np.int32)
        pkv.paged_kv_write(gu.dev(nk), gu.dev(nv), gu.dev(ns), gk, gv)
        oracle.paged_kv_write(nk, nv, ns, kc, vc)
        tables = pool.block_tables(seqs)
        lens = pool.context_lens(seqs)
        pkv.paged_attention_decode(out, gu.dev(q), gk, gv, gu.dev(tables), gu.dev(lens),
                                   1 / math.sqrt(D), bs)
        ref = oracle.paged_attention_decode(q, kc, vc, tables, lens, 1 / math.sqrt(D), bs)
        gu.assert_close(gu.host(out), ref, "bf16", f"step {step}")
        assert np.array_equal(gu.host(gk), kc) and np.array_equal(gu.host(gv), vc)
    assert n_copies == 4  # the partly filled last prompt block, once per extra branch
