"""Pins for the oracle's chunked-prefill attention (CPU only).

Chunked prefill: each sequence's new query tokens are the last positions of
its context (their K/V written first) and attend causally to every position up
to their own, the cached prefix read through the block table ("What problem
does PagedAttention solve for the KV cache in vLLM?", section "Sharing, the
second dividend": reused prefix blocks skip that part of prefill).  The oracle
is checked against what it does not compute itself:
  * torch's scaled_dot_product_attention in float64 with an explicit boolean
    causal mask aligned to the end of the context, on contiguous K/V from which
    the paged pool was built by numpy reshapes;
  * the decode oracle: a chunk's last query is a decode query over the whole
    context, and a one-token chunk is exactly decode;
  * closed forms and invariances: the first token of a prompt with no prefix
    returns its own V row; physical block ids do not matter; keys after a
    query's position never reach it.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests.test_oracle_decode import _as_f64, _make
from workloads import bf16_bits_from_f32

pytestmark = pytest.mark.filterwarnings("ignore")


def _queries(rng, chunks, Hq, D, elem):
    T = int(np.sum(chunks))
    x = rng.standard_normal((T, Hq, D)).astype(np.float32)
    q = x if elem == "f32" else bf16_bits_from_f32(x)
    qs = np.zeros(len(chunks) + 1, np.int32)
    qs[1:] = np.cumsum(chunks)
    return q, qs


def _sdpa_causal(q, qs, Ks, Vs, lens, scale):
    """float64 attention per sequence, queries at the last positions, with an
    explicit position mask and torch's grouped-query mapping."""
    out = np.zeros(q.shape, np.float64)
    for s in range(len(lens)):
        a, b = int(qs[s]), int(qs[s + 1])
        if a == b:
            continue
        n = int(lens[s])
        pos = np.arange(n - (b - a), n)
        mask = torch.from_numpy(np.arange(n)[None, :] <= pos[:, None])
        qq = torch.from_numpy(_as_f64(q[a:b])).permute(1, 0, 2)[None]
        k = torch.from_numpy(_as_f64(Ks[s]))[None]
        v = torch.from_numpy(_as_f64(Vs[s]))[None]
        o = F.scaled_dot_product_attention(qq, k, v, attn_mask=mask, scale=scale, enable_gqa=True)
        out[a:b] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("elem", ["f32", "bf16"])
@pytest.mark.parametrize("bs,G,D", [(1, 1, 8), (2, 2, 16), (16, 7, 32), (32, 4, 64)])
def test_matches_library_causal_attention(elem, bs, G, D):
    rng = np.random.default_rng(bs * 100 + G * 10 + D + 5)
    Hkv = 2
    lens = [1, bs + 1, 3 * bs - 1, 40, 7]
    chunks = [min(c, n) for c, n in zip([1, bs + 1, 5, 17, 0], lens)]
    _, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, len(lens), Hkv * G, Hkv, D, bs, lens, elem)
    q, qs = _queries(rng, chunks, Hkv * G, D, elem)
    scale = 1.0 / math.sqrt(D)
    got = oracle.paged_attention_prefill(q, kc, vc, tables, lens, qs, scale, bs)
    ref = _sdpa_causal(q, qs, Ks, Vs, lens, float(np.float32(scale)))
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_last_query_and_one_token_chunks_are_decode():
    rng = np.random.default_rng(21)
    Hq, Hkv, D, bs = 8, 2, 32, 16
    lens = [5, 33, 64, 100]
    chunks = [5, 4, 1, 30]
    _, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 4, Hq, Hkv, D, bs, lens, "bf16")
    q, qs = _queries(rng, chunks, Hq, D, "bf16")
    got = oracle.paged_attention_prefill(q, kc, vc, tables, lens, qs, 0.2, bs)
    last = np.ascontiguousarray(q[qs[1:] - 1])
    dec = oracle.paged_attention_decode(last, kc, vc, tables, lens, 0.2, bs)
    np.testing.assert_allclose(got[qs[1:] - 1], dec, rtol=1e-13, atol=1e-14)
    assert np.array_equal(got[qs[2]], dec[2])  # the one-token chunk, bit for bit


def test_first_prompt_token_returns_its_value_row():
    rng = np.random.default_rng(3)
    _, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 2, 4, 2, 16, 16, [20, 9])
    q, qs = _queries(rng, [20, 9], 4, 16, "f32")
    got = oracle.paged_attention_prefill(q, kc, vc, tables, lens, qs, 0.7, 16)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(got[qs[s], h], Vs[s][h // 2, 0].astype(np.float64))


def test_physical_ids_do_not_matter_and_later_keys_never_leak():
    rng = np.random.default_rng(4)
    Hq, Hkv, D, bs = 6, 3, 16, 16
    lens_l = [50, 17, 64]
    chunks = [20, 17, 8]
    _, Ks, Vs, kc, vc, tables, lens, free = _make(rng, 3, Hq, Hkv, D, bs, lens_l, "bf16")
    q, qs = _queries(rng, chunks, Hq, D, "bf16")
    base = oracle.paged_attention_prefill(q, kc, vc, tables, lens, qs, 0.25, bs)
    # relabel every physical block
    NB = kc.shape[0]
    pi = rng.permutation(NB).astype(np.int32)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi], vc2[pi] = kc, vc
    got = oracle.paged_attention_prefill(q, kc2, vc2, np.ascontiguousarray(pi[tables]), lens, qs,
                                         0.25, bs)
    assert np.array_equal(got, base)
    # overwrite the keys and values after the first query of sequence 0 (position 30)
    kc3, vc3 = kc.copy(), vc.copy()
    for t in range(31, 50):
        blk, off = tables[0, t // bs], t % bs
        kc3[blk, :, off] = bf16_bits_from_f32(np.full((Hkv, D), 3.0, np.float32))
        vc3[blk, :, off] = bf16_bits_from_f32(np.full((Hkv, D), -9.0, np.float32))
    got3 = oracle.paged_attention_prefill(q, kc3, vc3, tables, lens, qs, 0.25, bs)
    assert np.array_equal(got3[0], base[0])
    assert not np.array_equal(got3[1], base[1])


def test_range_errors():
    rng = np.random.default_rng(5)
    _, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 2, 4, 2, 16, 16, [10, 9])
    q, qs = _queries(rng, [11, 2], 4, 16, "f32")  # 11 queries but only 10 tokens
    with pytest.raises(ValueError):
        oracle.paged_attention_prefill(q, kc, vc, tables, lens, qs, 0.5, 16)
