"""A seeded multi-step decode loop driven by the host BlockPool, on the GPU and
in the oracle side by side, each from its own pool.

Every step: some sequences are admitted (prompts sharing leading tokens, so the
prefix cache matches blocks; the matched part is not written again), forked,
finished, swapped out (blocks gathered to device staging) or swapped back in
(scattered into fresh blocks); then every live sequence gets one new token, its
copy-on-write pairs are copied with paged_kv_copy_blocks, and the write and
the attention run as one paged_attention_decode_append call.  A token's K/V
rows are a fixed function of its id and position, so a cached block holds
exactly what the new prompt would have written.  After every step the decode
output matches the oracle's on the oracle's pool, and both pools agree bit for
bit (blocks recycled from finished sequences still hold their old rows: stale
data never reaches an output)."""
import math

import numpy as np
import pytest

import oracle
import workloads
from paged_kv_cache_135_amd.block_pool import BlockPool, OutOfBlocks
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
torch = gu.torch
import paged_kv_cache_135_amd as pkv  # noqa: E402

H, G, D, BS, NB = 2, 4, 128, 16, 160
SCALE = 1.0 / math.sqrt(D)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


def _rows(token_ids, positions, which):
    """bf16 K (which=0) or V (which=1) rows [n, H, D] of tokens with these ids at
    these positions: a fixed function of (id, position)."""
    out = np.empty((len(token_ids), H, D), np.uint16)
    for i, (t, p) in enumerate(zip(token_ids, positions)):
        workloads.fill_normal(out[i:i + 1], 0.5, 1_000_003 * int(t) + int(p), 40 + which)
    return out


@pytest.mark.parametrize("seed", range(4))
def test_serving_loop(seed):
    rng = np.random.default_rng([seed, 8181])
    pool = BlockPool(NB, BS, enable_prefix_caching=True)
    kc = np.full((NB, H, BS, D), workloads.BF16_NAN, np.uint16)
    vc = kc.copy()
    gk, gv = gu.dev(kc), gu.dev(vc)
    tokens, swapped = {}, {}
    next_id = [0]
    base_prompt = [int(x) for x in rng.integers(0, 50, size=90)]

    def write(toks, positions, slots):
        k, v = _rows(toks, positions, 0), _rows(toks, positions, 1)
        s = np.asarray(slots, np.int32)
        pkv.paged_kv_write(gu.dev(k), gu.dev(v), gu.dev(s), gk, gv)
        oracle.paged_kv_write(k, v, s, kc, vc)

    def admit():
        share = int(rng.integers(0, 91))
        n = share + int(rng.integers(1, 60))
        toks = base_prompt[:share] + [int(x) for x in rng.integers(0, 50, size=n - share)]
        name = f"s{next_id[0]}"
        next_id[0] += 1
        try:
            slots = pool.allocate(name, n, token_ids=toks)
        except OutOfBlocks:
            return
        c = pool.cached_tokens(name)
        write(toks[c:], range(c, n), slots[c:])
        tokens[name] = toks

    for _ in range(3):
        admit()
    n_cow = 0
    # the first steps fork, swap out, swap back in, finish and admit in turn;
    # then the step's action is drawn
    script = [0.35, 0.55, 0.65, 0.45, 0.0]
    for step in range(14):
        r = script[step] if step < len(script) else rng.random()
        live = sorted(tokens)
        if r < 0.3 or not live:
            admit()
        elif r < 0.4:
            src = live[int(rng.integers(0, len(live)))]
            name = f"s{next_id[0]}"
            next_id[0] += 1
            pool.fork(src, name)
            tokens[name] = list(tokens[src])
        elif r < 0.5 and len(live) > 1:
            name = live[int(rng.integers(0, len(live)))]
            pool.free(name)
            del tokens[name]
        elif r < 0.6 and len(live) > 1:
            name = live[int(rng.integers(0, len(live)))]
            ids = pool.swap_out(name)
            sk = torch.empty((len(ids), H, BS, D), dtype=torch.bfloat16, device="cuda")
            sv = torch.empty_like(sk)
            pkv.paged_kv_gather_blocks(gk, gv, gu.dev(ids), sk, sv)
            swapped[name] = (tokens.pop(name), sk, sv, oracle.gather_blocks(kc, ids),
                             oracle.gather_blocks(vc, ids))
        elif r < 0.7 and swapped:
            name = sorted(swapped)[0]
            try:
                ids = pool.swap_in(name)
            except OutOfBlocks:
                continue
            toks, sk, sv, ok, ov = swapped.pop(name)
            pkv.paged_kv_scatter_blocks(sk, sv, gu.dev(ids), gk, gv)
            oracle.scatter_blocks(ok, ids, kc)
            oracle.scatter_blocks(ov, ids, vc)
            tokens[name] = toks
        # one new token for every live sequence: copy-on-write first, then the
        # write and the attention in one call
        seqs = sorted(tokens)
        new_tok, slots, pairs = [], [], []
        try:
            for name in seqs:
                t = int(rng.integers(0, 50))
                sl, cow = pool.append(name, 1, token_ids=[t])
                new_tok.append(t)
                slots.append(int(sl[0]))
                pairs += cow
                tokens[name].append(t)
        except OutOfBlocks:
            pytest.skip("pool exhausted by this seed's admissions")
        n_cow += len(pairs)
        if pairs:
            pr = np.array(pairs, np.int32)
            pkv.validate_block_pairs(pr, NB)
            pkv.paged_kv_copy_blocks(gk, gv, gu.dev(pr))
            oracle.copy_blocks(kc, vc, pr)
        tables = pool.block_tables(seqs)
        lens = pool.context_lens(seqs)
        pos = [int(n) - 1 for n in lens]
        nk, nv = _rows(new_tok, pos, 0), _rows(new_tok, pos, 1)
        q = np.empty((len(seqs), H * G, D), np.uint16)
        workloads.fill_normal(q, 0.5, 7000 + step, seed)
        sl = np.asarray(slots, np.int32)
        pkv.validate_append_slots(sl, tables, lens, NB, BS)
        out = torch.empty_like(gu.dev(q))
        pkv.paged_attention_decode_append(out, gu.dev(q), gu.dev(nk), gu.dev(nv), gu.dev(sl), gk, gv,
                                          gu.dev(tables), gu.dev(lens), SCALE, BS)
        oracle.paged_kv_write(nk, nv, sl, kc, vc)
        ref = oracle.paged_attention_decode(q, kc, vc, tables, lens, SCALE, BS)
        gu.assert_close(gu.host(out), ref, "bf16", f"seed {seed} step {step}")
        assert np.array_equal(gu.host(gk), kc) and np.array_equal(gu.host(gv), vc), f"step {step}"
        # every live sequence's tokens are where its table says
        for name in seqs:
            toks = tokens[name]
            p = len(toks) - 1
            assert pool.slot(name, p) == slots[seqs.index(name)]
    assert pool.stats()["max_waste"] <= BS - 1
    # the run went through the prefix cache and copy-on-write
    assert pool.stats()["prefix_hit_blocks"] > 0 and n_cow > 0
