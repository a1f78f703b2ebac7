"""GPU parity over seeded random configurations, against the fp64 oracle.

Each case draws its shape and launch at random from a fixed seed: cache format
(f32, bf16, E4M3 with a per-tensor scale), head dim 64 or 128, block size 16,
32 or 64, 1-8 KV heads with group sizes 1-8, 1-24 sequences whose lengths mix
empty, single-token, tile-edge and ragged contexts, and one decode launch
(single pass with 1-8 wavefronts, split-K partitions, the balanced split with
its default or a small worker count, auto), with or without streaming pool
reads.  A second set draws near the supported limits: 9-16 query heads per KV
head and blocks of 128 or 256 tokens.  The step's KV write is done either by paged_kv_write followed by the
decode or folded into paged_attention_decode_append; both must leave the
oracle's written pool bit for bit and give the oracle's output on that pool,
within the format's tolerance, and empty sequences must give zero rows.  The cases complement the
hand-picked small cases and the full-size workloads with combinations nobody
chose."""
import math

import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
torch = gu.torch
import paged_kv_cache_135_amd as pkv  # noqa: E402

NUM_CASES = 160
NUM_NEAR_LIMITS = 48


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


def _lengths(rng, n, block_size):
    """A mix of empty, one-token, tile-edge and ragged contexts."""
    kinds = rng.integers(0, 6, size=n)
    out = []
    for k in kinds:
        if k == 0:
            out.append(0)
        elif k == 1:
            out.append(1)
        elif k == 2:
            out.append(16 * int(rng.integers(1, 20)) + int(rng.integers(-1, 2)))
        elif k == 3:
            out.append(block_size * int(rng.integers(1, 10)))
        else:
            out.append(int(rng.integers(2, 1500)))
    if max(out) == 0:
        out[0] = int(rng.integers(1, 300))
    return out


def _draw(seed, near_limits=False):
    rng = np.random.default_rng([seed, 4242 if not near_limits else 4343])
    dtype = ["f32", "bf16", "bf16", "fp8_e4m3"][int(rng.integers(0, 4))]
    D = [64, 128][int(rng.integers(0, 2))]
    if near_limits:
        # the largest group sizes (up to 16 query heads per KV head) and block
        # sizes (up to 256 tokens, 16 tiles a block)
        bs = [128, 256, 256][int(rng.integers(0, 3))]
        Hkv = [1, 2, 3][int(rng.integers(0, 3))]
        G = int(rng.integers(9, 17))
    else:
        bs = [16, 32, 64][int(rng.integers(0, 3))]
        Hkv = [1, 2, 4, 8][int(rng.integers(0, 4))]
        G = [1, 2, 4, 7, 8][int(rng.integers(0, 5))]
    S = int(rng.integers(1, 25))
    lens = _lengths(rng, S, bs)
    modes = [("single", 0, 1, 0), ("single", 0, 4, 0), ("single", 0, 8, 0),
             ("partitioned", 16 * int(rng.integers(1, 9)), int(rng.choice([0, 1, 2, 4])), 0),
             ("partitioned", 512, 1, 0), ("balanced", 0, 0, 0),
             ("balanced", 0, 0, int(rng.integers(1, 40))), ("auto", 0, 0, 0)]
    mode = modes[int(rng.integers(0, len(modes)))]
    stream_kv = bool(rng.integers(0, 2))
    append = bool(rng.integers(0, 2))
    case = workloads.build_case(f"random{seed}", seed=1000 + seed, context_lens=lens,
                                num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                                cache_dtype=dtype, std=1.0 if dtype == "f32" else 0.5,
                                scale=1.0 / math.sqrt(D))
    return case, mode, stream_kv, append


def _rows_per_sequence(case):
    """This step's new rows as [S, Hkv, D] plus slots [S] (-1 where len == 0)."""
    S = case.num_seqs
    live = np.nonzero(case.context_lens > 0)[0]
    k = np.zeros((S,) + case.k_new.shape[1:], case.k_new.dtype)
    v = np.zeros_like(k)
    slots = np.full(S, -1, np.int32)
    k[live], v[live], slots[live] = case.k_new, case.v_new, case.slot_mapping
    return k, v, slots


@pytest.mark.parametrize("near_limits,seed",
                         [(False, s) for s in range(NUM_CASES)] + [(True, s) for s in range(NUM_NEAR_LIMITS)])
def test_random_configuration(near_limits, seed):
    case, (mode, part, waves, workers), stream_kv, append = _draw(seed, near_limits)
    what = (f"seed {seed}: {case.cache_dtype} D={case.head_dim} bs={case.block_size} "
            f"Hq={case.num_q_heads} Hkv={case.num_kv_heads} S={case.num_seqs} "
            f"{mode}/{part}/{waves}/{workers} stream_kv={stream_kv} append={append}")
    print(what, flush=True)
    g = gu.GpuCase(case)
    kw = dict(k_scale=case.k_scale, v_scale=case.v_scale, mode=mode, partition_size=part,
              waves_per_group=waves, num_workers=workers, stream_kv=stream_kv)
    out = torch.full_like(g.q, float("nan"))
    if append:
        if case.fill_k is not None:
            g.write(case.fill_k, case.fill_v, case.fill_slots)
        k, v, slots = _rows_per_sequence(case)
        pkv.paged_attention_decode_append(out, g.q, gu.dev(k), gu.dev(v), gu.dev(slots), g.kc, g.vc,
                                          g.tables, g.lens, case.scale, case.block_size, **kw)
    else:
        g.fill_and_step_writes()
        pkv.paged_attention_decode(out, g.q, g.kc, g.vc, g.tables, g.lens, case.scale,
                                   case.block_size, **kw)
    torch.cuda.synchronize()
    got = gu.host(out)
    kc, vc = gu.oracle_caches(case)
    ref = gu.oracle_decode(case, kc, vc)
    gu.assert_close(got, ref, case.cache_dtype, what)
    # the write, by either route, leaves the oracle's pool bit for bit
    bits = lambda a: a.view(np.uint32) if a.dtype == np.float32 else a
    assert np.array_equal(bits(gu.host(g.kc)), bits(kc)), what + ": key pool"
    assert np.array_equal(bits(gu.host(g.vc)), bits(vc)), what + ": value pool"
    empty = case.context_lens == 0
    if empty.any():
        assert np.all(gu.as_f64(got[empty]) == 0.0), what
