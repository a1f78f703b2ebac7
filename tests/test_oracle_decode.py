"""Pins for the oracle's decode attention (CPU only).

The oracle is checked against things it does not compute itself:
  * torch's scaled_dot_product_attention in float64 on contiguous K/V (a library
    attention, with its own grouped-query head mapping), where the paged cache
    is built from the contiguous tensors with numpy reshapes, not with the
    oracle's index arithmetic;
  * closed forms: one token gives that token's V, a zero scale gives the mean
    of V, one overwhelming key gives its V, an empty context gives zeros;
  * invariances the pages state: physical block ids do not matter, only the
    logical order does ("pipe-paged-block-allocation-kv-cache", sections "In
    and out" and "Concept"); unwritten tail slots and free blocks never reach
    the output ("PagedAttention, clearly explained": slots past the sequence
    are never written, blocks are recycled).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import bf16_bits_from_f32, bf16_to_f32

pytestmark = pytest.mark.filterwarnings("ignore")


def _as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def _make(rng, S, Hq, Hkv, D, bs, lens, elem="f32", spare=3, poison=True):
    """Contiguous per-sequence K/V plus a paged copy built by reshapes."""
    lens = np.asarray(lens, dtype=np.int64)
    nbs = (lens + bs - 1) // bs
    NB = int(nbs.sum()) + spare
    perm = rng.permutation(NB).astype(np.int32)
    maxb = max(1, int(nbs.max()))
    free = perm[int(nbs.sum()):]
    tables = np.full((S, maxb), free[0] if free.size else 0, dtype=np.int32)
    c = 0
    for s in range(S):
        tables[s, :nbs[s]] = perm[c:c + nbs[s]]
        c += nbs[s]
    npdt = np.float32 if elem == "f32" else np.uint16
    fill = np.float32(np.nan) if elem == "f32" else np.uint16(0x7FC0)

    def draw(shape):
        x = rng.standard_normal(shape).astype(np.float32)
        return x if elem == "f32" else bf16_bits_from_f32(x)

    q = draw((S, Hq, D))
    Ks = [draw((Hkv, int(n), D)) for n in lens]
    Vs = [draw((Hkv, int(n), D)) for n in lens]
    kc = np.full((NB, Hkv, bs, D), fill if poison else 0, dtype=npdt)
    vc = np.full((NB, Hkv, bs, D), fill if poison else 0, dtype=npdt)
    for s in range(S):
        n, nb = int(lens[s]), int(nbs[s])
        if nb == 0:
            continue
        for src, dst in ((Ks[s], kc), (Vs[s], vc)):
            padded = np.full((Hkv, nb * bs, D), fill if poison else 0, dtype=npdt)
            padded[:, :n] = src
            dst[tables[s, :nb]] = padded.reshape(Hkv, nb, bs, D).transpose(1, 0, 2, 3)
    return q, Ks, Vs, kc, vc, tables, lens.astype(np.int32), free


def _sdpa(q, Ks, Vs, scale):
    """float64 attention per sequence with torch's grouped-query mapping."""
    outs = []
    for s in range(q.shape[0]):
        qs = torch.from_numpy(_as_f64(q[s]))[None, :, None, :]
        if Ks[s].shape[1] == 0:
            outs.append(np.zeros((q.shape[1], q.shape[2])))
            continue
        k = torch.from_numpy(_as_f64(Ks[s]))[None]
        v = torch.from_numpy(_as_f64(Vs[s]))[None]
        o = F.scaled_dot_product_attention(qs, k, v, scale=scale, enable_gqa=True)
        outs.append(o[0, :, 0, :].numpy())
    return np.stack(outs)


def _close(a, b, rtol=1e-11, atol=1e-12):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


@pytest.mark.parametrize("elem", ["f32", "bf16"])
@pytest.mark.parametrize("bs,G,D", [(1, 1, 8), (2, 2, 16), (16, 2, 64), (16, 7, 32), (32, 4, 64)])
def test_matches_library_attention(elem, bs, G, D):
    rng = np.random.default_rng(bs * 100 + G * 10 + D)
    Hkv = 2
    lens = [1, bs + 1, 3 * bs - 1, 40, 2]
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, len(lens), Hkv * G, Hkv, D, bs, lens, elem)
    scale = 1.0 / math.sqrt(D)
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, scale, bs)
    _close(got, _sdpa(q, Ks, Vs, float(np.float32(scale))))


def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(1)
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 3, 4, 2, 16, 16, [1, 1, 1])
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.7, 16)
    for s in range(3):
        for h in range(4):
            assert np.array_equal(got[s, h], Vs[s][h // 2, 0].astype(np.float64))


def test_empty_context_gives_zeros():
    rng = np.random.default_rng(2)
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 3, 2, 1, 8, 16, [0, 5, 0])
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.3, 16)
    assert np.array_equal(got[0], np.zeros((2, 8)))
    assert np.array_equal(got[2], np.zeros((2, 8)))
    assert np.all(np.isfinite(got[1]))


def test_zero_scale_gives_mean_of_values():
    rng = np.random.default_rng(3)
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 2, 6, 3, 16, 16, [37, 64])
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.0, 16)
    for s in range(2):
        for h in range(6):
            _close(got[s, h], Vs[s][h // 2].astype(np.float64).mean(axis=0))


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(4)
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 1, 2, 1, 8, 16, [29])
    Ks[0][:] = Ks[0][:, :1]
    kc2 = kc.copy()
    nb = 2
    padded = np.full((1, nb * 16, 8), np.nan, np.float32)
    padded[:, :29] = Ks[0]
    kc2[tables[0, :nb]] = padded.reshape(1, nb, 16, 8).transpose(1, 0, 2, 3)
    got = oracle.paged_attention_decode(q, kc2, vc, tables, lens, 1.3, 16)
    for h in range(2):
        _close(got[0, h], Vs[0][0].astype(np.float64).mean(axis=0))


def test_one_overwhelming_key_selects_its_value():
    rng = np.random.default_rng(5)
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 1, 1, 1, 4, 16, [50])
    q[:] = 0
    q[0, 0, 0] = 1.0
    star = 33
    blk, off = tables[0, star // 16], star % 16
    kc[blk, 0, off, 0] = 1.0e4  # score gap ~1e4: every other weight is exp(-1e4) = 0
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 1.0, 16)
    assert np.array_equal(got[0, 0], Vs[0][0, star].astype(np.float64))


def test_physical_block_ids_do_not_matter():
    rng = np.random.default_rng(6)
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 4, 8, 2, 32, 16, [16, 1, 77, 130], "bf16")
    base = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.2, 16)
    pi = rng.permutation(kc.shape[0]).astype(np.int32)  # block b moves to pi[b]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    got = oracle.paged_attention_decode(q, kc2, vc2, pi[tables], lens, 0.2, 16)
    assert np.array_equal(got, base)
    # a contiguous layout (identity table over the same data) gives the same bits
    nbs = (lens + 15) // 16
    order = np.concatenate([tables[s, :nbs[s]] for s in range(4)])
    kc3 = kc[order]
    vc3 = vc[order]
    t3 = np.zeros_like(tables)
    c = 0
    for s in range(4):
        t3[s, :nbs[s]] = np.arange(c, c + nbs[s])
        c += nbs[s]
    got3 = oracle.paged_attention_decode(q, kc3, vc3, t3, lens, 0.2, 16)
    assert np.array_equal(got3, base)


def test_poisoned_free_blocks_and_tails_do_not_reach_output():
    rng = np.random.default_rng(7)
    q, Ks, Vs, kc, vc, tables, lens, free = _make(rng, 3, 4, 2, 16, 16, [5, 33, 48],
                                                 poison=False)
    clean = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.25, 16)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[free] = np.nan
    vc2[free] = np.inf
    for s in range(3):
        n = int(lens[s])
        if n % 16:
            kc2[tables[s, (n - 1) // 16], :, n % 16:] = np.nan
            vc2[tables[s, (n - 1) // 16], :, n % 16:] = np.nan
    got = oracle.paged_attention_decode(q, kc2, vc2, tables, lens, 0.25, 16)
    assert np.array_equal(got, clean)


def test_token_order_is_a_set_for_attention():
    # no positional term in decode: permuting whole (K, V) token rows together
    # must not change the result beyond rounding
    rng = np.random.default_rng(8)
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 1, 2, 1, 16, 16, [45])
    base = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.5, 16)
    p = rng.permutation(45)
    Ks2 = [Ks[0][:, p]]
    Vs2 = [Vs[0][:, p]]
    kc2, vc2 = kc.copy(), vc.copy()
    for src, dst in ((Ks2[0], kc2), (Vs2[0], vc2)):
        padded = np.full((1, 48, 16), np.nan, np.float32)
        padded[:, :45] = src
        dst[tables[0, :3]] = padded.reshape(1, 3, 16, 16).transpose(1, 0, 2, 3)
    got = oracle.paged_attention_decode(q, kc2, vc2, tables, lens, 0.5, 16)
    _close(got, base)
    # and swapping only V rows must change it (K and V stay paired by position)
    vc3 = vc.copy()
    padded = np.full((1, 48, 16), np.nan, np.float32)
    padded[:, :45] = Vs[0][:, p]
    vc3[tables[0, :3]] = padded.reshape(1, 3, 16, 16).transpose(1, 0, 2, 3)
    got3 = oracle.paged_attention_decode(q, kc, vc3, tables, lens, 0.5, 16)
    assert not np.allclose(got3, base)


def test_row_mask_computes_the_same_rows():
    rng = np.random.default_rng(9)
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 3, 4, 2, 8, 16, [20, 3, 50])
    full = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.4, 16)
    mask = np.zeros((3, 4), bool)
    mask[1, 2] = mask[2, 0] = True
    part = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.4, 16, row_mask=mask)
    assert np.array_equal(part[mask], full[mask])
    assert np.all(np.isnan(part[~mask]))


def test_e4m3_cache_matches_library_attention_on_decoded_values():
    rng = np.random.default_rng(10)
    S, Hkv, G, D, bs = 3, 2, 4, 32, 16
    lens = np.array([1, 31, 70], np.int32)
    nbs = (lens + bs - 1) // bs
    NB = int(nbs.sum()) + 2
    perm = rng.permutation(NB).astype(np.int32)
    tables = np.zeros((S, nbs.max()), np.int32)
    c = 0
    for s in range(S):
        tables[s, :nbs[s]] = perm[c:c + nbs[s]]
        c += nbs[s]
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    kc = rng.choice(finite, size=(NB, Hkv, bs, D)).astype(np.uint8)
    vc = rng.choice(finite, size=(NB, Hkv, bs, D)).astype(np.uint8)
    q = bf16_bits_from_f32(rng.standard_normal((S, Hkv * G, D)).astype(np.float32) * 0.05)
    ks, vs = 0.0123, 0.731
    got = oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.17, bs, k_scale=ks, v_scale=vs)
    # library decode of the codes (torch float8_e4m3fn), then contiguous attention
    dec = lambda a: torch.from_numpy(a).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    Ks, Vs = [], []
    for s in range(S):
        blocks_k = dec(kc[tables[s, :nbs[s]]]) * np.float64(np.float32(ks))
        blocks_v = dec(vc[tables[s, :nbs[s]]]) * np.float64(np.float32(vs))
        Ks.append(blocks_k.transpose(1, 0, 2, 3).reshape(Hkv, -1, D)[:, :lens[s]])
        Vs.append(blocks_v.transpose(1, 0, 2, 3).reshape(Hkv, -1, D)[:, :lens[s]])
    _close(got, _sdpa(q, Ks, Vs, float(np.float32(0.17))))


def test_out_of_pool_block_id_is_rejected():
    rng = np.random.default_rng(11)
    q, Ks, Vs, kc, vc, tables, lens, _ = _make(rng, 1, 2, 1, 8, 16, [20])
    tables[0, 1] = kc.shape[0]
    with pytest.raises(ValueError):
        oracle.paged_attention_decode(q, kc, vc, tables, lens, 0.4, 16)
