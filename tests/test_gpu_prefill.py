"""GPU parity of chunked-prefill paged attention against the fp64 oracle.

Small batches cover every element type, both head dims, group sizes 1 to 16,
block sizes 16 to 64, chunks of 0, 1 and many tokens, prompts with no cached
prefix, chunks that are the whole context, NaN-poisoned free blocks and tails,
and every rows-per-wavefront choice.  The full-size Qwen-shaped prefill batch
is checked on whole sequences the oracle computes in seconds."""
import math

import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
torch = gu.torch
import paged_kv_cache_135_amd as pkv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


CASES = {
    # name: (prefix lengths, chunk lengths, Hq, Hkv, D, block size, cache dtype)
    "g7_d128_bf16": ([0, 100, 37, 511, 16, 3], [40, 1, 77, 200, 0, 33], 28, 4, 128, 16, "bf16"),
    "g1_d64_bs32_bf16": ([5, 0, 64], [59, 130, 1], 4, 4, 64, 32, "bf16"),
    "g16_d128_bs64_bf16": ([70, 0], [9, 64], 16, 1, 128, 64, "bf16"),
    "g2_d64_f32": ([0, 17, 40], [23, 5, 60], 4, 2, 64, 16, "f32"),
    "g4_d128_f32": ([100, 0], [31, 48], 8, 2, 128, 32, "f32"),
    "g4_d128_e4m3": ([300, 0, 20], [50, 90, 1], 32, 8, 128, 16, "fp8_e4m3"),
    "g8_d64_e4m3": ([33, 7], [40, 70], 16, 2, 64, 16, "fp8_e4m3"),
}


def _case(name, seed=13):
    pre, chk, Hq, Hkv, D, bs, dt = CASES[name]
    return workloads.build_prefill_case(name, seed=seed, prefix_lens=pre, chunk_lens=chk,
                                        num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                                        block_size=bs, cache_dtype=dt,
                                        std=0.5 if dt != "f32" else 1.0,
                                        scale=1.0 / math.sqrt(D))


def _oracle(case, kc, vc):
    import oracle
    return oracle.paged_attention_prefill(case.q, kc, vc, case.block_tables, case.context_lens,
                                          case.query_start, case.scale, case.block_size,
                                          case.k_scale, case.v_scale)


def _run(g, case, qs_dev, rows_per_wave=0, out=None):
    out = torch.empty_like(g.q) if out is None else out
    mql = int(np.diff(case.query_start).max()) if case.num_seqs else 0
    pkv.paged_attention_prefill(out, g.q, g.kc, g.vc, g.tables, g.lens, qs_dev, mql, case.scale,
                                case.block_size, k_scale=case.k_scale, v_scale=case.v_scale,
                                rows_per_wave=rows_per_wave)
    return out


_prep = {}


def _prepared(name):
    if name not in _prep:
        case = _case(name)
        pkv.validate_prefill_inputs(case.query_start, case.block_tables, case.context_lens,
                                    case.num_blocks, case.block_size, case.q.shape[0],
                                    int(np.diff(case.query_start).max()))
        g = gu.GpuCase(case)
        g.fill_and_step_writes()
        kc, vc = gu.oracle_caches(case)
        _prep[name] = (case, g, gu.dev(case.query_start), _oracle(case, kc, vc))
    return _prep[name]


@pytest.mark.parametrize("rpw", [16, 32, 64])
@pytest.mark.parametrize("name", list(CASES))
def test_small_cases(name, rpw):
    case, g, qs, ref = _prepared(name)
    if rpw == 64 and (case.cache_dtype == "f32" or case.head_dim != 64):
        with pytest.raises(pkv.PagedKVError):
            _run(g, case, qs, rpw)
        return
    got = gu.host(_run(g, case, qs, rpw))
    gu.assert_close(got, ref, case.cache_dtype, f"{name} rows/wave {rpw}")


def test_deterministic_and_independent_of_physical_placement():
    case, g, qs, _ = _prepared("g7_d128_bf16")
    a = gu.host(_run(g, case, qs)).copy()
    b = gu.host(_run(g, case, qs))
    assert np.array_equal(a, b)
    # relabel every physical block: move contents, rewrite tables
    rng = np.random.default_rng(9)
    pi = rng.permutation(case.num_blocks)
    inv = torch.from_numpy(np.argsort(pi)).to(g.kc.device)
    kc2 = g.kc[inv].contiguous()
    vc2 = g.vc[inv].contiguous()
    tables2 = gu.dev(np.ascontiguousarray(pi[case.block_tables].astype(np.int32)))
    out = torch.empty_like(g.q)
    mql = int(np.diff(case.query_start).max())
    pkv.paged_attention_prefill(out, g.q, kc2, vc2, tables2, g.lens, qs, mql, case.scale,
                                case.block_size)
    assert np.array_equal(gu.host(out), a)


def test_last_chunk_rows_agree_with_decode():
    """A chunk's last query is a decode query over the whole context."""
    case, g, qs, ref = _prepared("g7_d128_bf16")
    got = gu.host(_run(g, case, qs))
    live = np.nonzero(np.diff(case.query_start) > 0)[0]
    last_rows = case.query_start[1:][live] - 1
    qd = g.q[torch.from_numpy(last_rows.astype(np.int64)).to(g.q.device)].contiguous()
    out = torch.empty_like(qd)
    pkv.paged_attention_decode(out, qd, g.kc, g.vc, g.tables[live].contiguous(),
                               g.lens[live].contiguous(), case.scale, case.block_size,
                               mode="single")
    gu.assert_close(gu.host(out), ref[last_rows], "bf16", "decode at the chunk's last row")
    gu.assert_close(got[last_rows], ref[last_rows], "bf16", "prefill at the chunk's last row")


def test_small_max_query_len_still_covers_every_row():
    """max_query_len only sizes the launch: a smaller value loses nothing."""
    case, g, qs, ref = _prepared("g7_d128_bf16")
    out = torch.empty_like(g.q)
    pkv.paged_attention_prefill(out, g.q, g.kc, g.vc, g.tables, g.lens, qs, 1, case.scale,
                                case.block_size)
    gu.assert_close(gu.host(out), ref, "bf16", "max_query_len 1")


def test_full_size_qwen_prefill_on_sampled_sequences():
    case = workloads.p1_chunked_prefill()
    g = gu.GpuCase(case)
    qs = gu.dev(case.query_start)
    got = gu.host(_run(g, case, qs))
    import oracle
    for s in (0, 6):  # one short and the longest context
        a, b = int(case.query_start[s]), int(case.query_start[s + 1])
        sub_q = np.ascontiguousarray(case.q[a:b])
        ref = oracle.paged_attention_prefill(
            sub_q, case.key_cache, case.value_cache,
            np.ascontiguousarray(case.block_tables[s:s + 1]),
            np.ascontiguousarray(case.context_lens[s:s + 1]),
            np.array([0, b - a], np.int32), case.scale, case.block_size)
        gu.assert_close(got[a:b], ref, "bf16", f"full-size prefill, sequence {s}")


def test_largest_block_size_and_long_chunk():
    """block_size 256 and a 1,100-token chunk after a 300-token prefix."""
    case = workloads.build_prefill_case("bs256", seed=47, prefix_lens=[300, 0],
                                        chunk_lens=[1100, 257], num_q_heads=16, num_kv_heads=2,
                                        head_dim=128, block_size=256, cache_dtype="bf16",
                                        std=0.5, scale=1.0 / math.sqrt(128))
    g = gu.GpuCase(case)
    qs = gu.dev(case.query_start)
    ref = _oracle(case, case.key_cache, case.value_cache)
    for rpw in (16, 32):
        gu.assert_close(gu.host(_run(g, case, qs, rpw)), ref, "bf16", f"bs 256 rows/wave {rpw}")


@pytest.mark.parametrize("num_seqs", [600, 900])
def test_many_short_sequences(num_seqs):
    """Hundreds of sequences, zero-length chunks among them.  At head dim 64
    the job ranking holds up to 635 sequences' lengths in LDS: 600 takes that
    path (each thread of the ranking owns a run of the sequences, and with
    more jobs than threads the counting sort finds each round's job), 900 the
    one that reads the lengths from global memory in every pass."""
    rng = np.random.default_rng(71)
    pre = [int(x) for x in rng.integers(0, 200, num_seqs)]
    chk = [int(x) for x in rng.integers(0, 13, num_seqs)]
    case = workloads.build_prefill_case("many", seed=71, prefix_lens=pre, chunk_lens=chk,
                                        num_q_heads=8, num_kv_heads=2, head_dim=64,
                                        block_size=16, cache_dtype="bf16", std=0.5,
                                        scale=1.0 / math.sqrt(64))
    g = gu.GpuCase(case)
    qs = gu.dev(case.query_start)
    ref = _oracle(case, case.key_cache, case.value_cache)
    gu.assert_close(gu.host(_run(g, case, qs)), ref, "bf16", f"{num_seqs} sequences")


def test_more_rounds_than_one_plan_covers():
    """400 one-job sequences on 4 KV heads: 1,600 items, seven rounds of a
    256-workgroup grid.  Each ranking plans four rounds, so every workgroup
    ranks again mid-kernel; with at most 512 jobs the ranks are counted
    directly.  Chunks of 1..20 tokens over prefixes of 0..300 tokens."""
    rng = np.random.default_rng(83)
    pre = [int(x) for x in rng.integers(0, 301, 400)]
    chk = [int(x) for x in rng.integers(1, 21, 400)]
    case = workloads.build_prefill_case("rounds", seed=83, prefix_lens=pre, chunk_lens=chk,
                                        num_q_heads=16, num_kv_heads=4, head_dim=128,
                                        block_size=16, cache_dtype="bf16", std=0.5,
                                        scale=1.0 / math.sqrt(128))
    g = gu.GpuCase(case)
    qs = gu.dev(case.query_start)
    ref = _oracle(case, case.key_cache, case.value_cache)
    gu.assert_close(gu.host(_run(g, case, qs)), ref, "bf16", "400 sequences x 4 KV heads")


@pytest.mark.parametrize("scale", [-0.9 / math.sqrt(128), 0.0])
def test_negative_and_zero_scale(scale):
    """The kernel folds a positive factor into the exponent: a negative scale
    flips q's sign bits, a zero scale averages the visible V rows."""
    case = workloads.build_prefill_case("scale", seed=5, prefix_lens=[90, 0, 33],
                                        chunk_lens=[40, 70, 1], num_q_heads=16,
                                        num_kv_heads=4, head_dim=128, block_size=16,
                                        cache_dtype="bf16", std=0.5, scale=scale)
    g = gu.GpuCase(case)
    qs = gu.dev(case.query_start)
    ref = _oracle(case, case.key_cache, case.value_cache)
    for rpw in (16, 32):
        gu.assert_close(gu.host(_run(g, case, qs, rpw)), ref, "bf16", f"scale {scale} rows/wave {rpw}")
