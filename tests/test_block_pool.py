"""Host allocator checks (CPU), against the facts the pages print
(golden/allocation_examples.txt and golden/block_size_example.txt)."""
import numpy as np
import pytest

from paged_kv_cache_135_amd import BlockPool, OutOfBlocks, block_bytes, blocks_for_memory
from tests._golden import load

A = load("allocation_examples.txt")
B = load("block_size_example.txt")


def test_block_bytes_and_pool_size_worked_example():
    bb = block_bytes(B["num_layers"], B["num_kv_heads"], B["head_dim"], B["block_tokens"],
                     B["elem_bytes"])
    assert bb == B["block_bytes"]
    n = blocks_for_memory(int(B["kv_gb"] * 1e9), bb)
    assert abs(n - B["approx_blocks"]) / B["approx_blocks"] < 0.01
    assert abs(n * B["block_tokens"] - B["approx_tokens"]) / B["approx_tokens"] < 0.01


def test_forty_tokens_hold_three_blocks():
    pool = BlockPool(64, 16)
    pool.allocate("a", 1)
    for _ in range(39):
        pool.append("a")
    assert len(pool.table("a")) == A["tokens_40_blocks_bs16"]


def test_prompt_gets_just_enough_then_one_block_per_block_size_tokens():
    pool = BlockPool(64, 16)
    pool.allocate("a", 33)
    assert len(pool.table("a")) == 3
    grown = []
    for _ in range(40):
        pool.append("a")
        grown.append(len(pool.table("a")))
    # a new block exactly when the previous one is full: at token 49, 65
    assert grown[:15] == [3] * 15 and grown[15] == 4 and grown[31] == 5


def test_waste_never_exceeds_block_size_minus_one():
    rng = np.random.default_rng(0)
    pool = BlockPool(4096, 16)
    for i, n in enumerate(rng.integers(1, 700, size=60)):
        pool.allocate(i, int(n))
    st = pool.stats()
    assert st["max_waste"] <= A["max_waste_per_seq_bs16"]
    assert all(w == (-int(pool.num_tokens(q))) % 16 for q, w in st["waste_per_seq"].items())
    assert st["live_fraction"] > 0.96


def test_contiguous_reservation_waste_examples():
    # prior art the pages contrast with paging: one slab of max length per request
    assert 4096 - (100 + 50) == A["reserved_4096_used_150_empty"]
    # 98.5%, printed as "~98%"
    assert int(100 * (4096 - 60) / 4096) == A["reserved_4096_emitted_60_untouched_pct"]
    pool = BlockPool(512, 16)
    pool.allocate("x", 150)
    assert pool.stats()["waste_per_seq"]["x"] == 10  # paging: 10 slots, not 3,946


def test_prefix_sharing_is_block_granular():
    pool = BlockPool(256, 32)
    pool.allocate("p", 1000)
    full = 1000 // 32
    pool.allocate("q", 1000, prefix_of="p", prefix_blocks=full)
    shared = sum(1 for a, b in zip(pool.table("p"), pool.table("q")) if a == b)
    assert shared * 32 == A["prefix_1000_reused_bs32"]
    with pytest.raises(ValueError):  # the partly filled 32nd block cannot be shared
        pool.allocate("r", 1000, prefix_of="p", prefix_blocks=full + 1)


def test_forks_count_references_and_copy_on_write():
    pool = BlockPool(64, 16)
    pool.allocate("prompt", 40)  # 2 full blocks + 8 tokens in the third
    for i in range(4):
        pool.fork("prompt", f"f{i}")
    t = pool.table("prompt")
    assert [pool.refcount(b) for b in t] == [A["forks_5_refcount"]] * 3
    slots, cow = pool.append("f0")
    # the shared, partly filled last block is copied before f0 writes into it
    assert len(cow) == 1 and cow[0][0] == t[2]
    new = cow[0][1]
    assert pool.table("f0")[:2] == t[:2] and pool.table("f0")[2] == new
    assert pool.refcount(t[2]) == 4 and pool.refcount(new) == 1
    assert slots[0] == new * 16 + 8
    # a branch writing into a fresh block needs no copy
    for _ in range(7):
        pool.append("f0")
    s, cow2 = pool.append("f0")
    assert cow2 == [] and len(pool.table("f0")) == 4


def test_free_returns_blocks_for_reuse():
    pool = BlockPool(8, 16)
    pool.allocate("a", 16 * 5)
    assert pool.num_free == 3
    with pytest.raises(OutOfBlocks):
        pool.allocate("b", 16 * 4)
    pool.free("a")
    assert pool.num_free == 8
    slots = pool.allocate("b", 16 * 8)
    assert sorted(set(slots // 16)) == list(range(8))


def test_shared_blocks_survive_until_last_reference():
    pool = BlockPool(16, 16)
    pool.allocate("a", 32)
    pool.fork("a", "b")
    pool.free("a")
    assert pool.num_free == 14 and all(pool.refcount(b) == 1 for b in pool.table("b"))
    pool.free("b")
    assert pool.num_free == 16


def test_pool_too_small_for_one_max_length_sequence_is_refused():
    with pytest.raises(OutOfBlocks):
        BlockPool(10, 16, max_model_len=161)
    BlockPool(10, 16, max_model_len=160)


def test_exhaustion_on_append_raises_and_leaves_state_unchanged():
    pool = BlockPool(2, 16)
    pool.allocate("a", 32)
    with pytest.raises(OutOfBlocks):
        pool.append("a")
    assert pool.num_tokens("a") == 32 and len(pool.table("a")) == 2


def test_tables_and_slots_agree():
    rng = np.random.default_rng(3)
    pool = BlockPool(128, 16)
    lens = [5, 16, 17, 100]
    for i, n in enumerate(lens):
        pool.allocate(i, n)
    tables = pool.block_tables(range(4), pad=0)
    assert tables.dtype == np.int32 and tables.shape == (4, 7)
    assert list(pool.context_lens(range(4))) == lens
    for i, n in enumerate(lens):
        for p in rng.integers(0, n, size=5):
            p = int(p)
            assert pool.slot(i, p) == tables[i, p // 16] * 16 + p % 16


# ------------------------------------------------------------ prefix caching
def test_block_granular_prefix_reuse_matches_the_pages_example():
    """[foundry] "Failure modes": with block_size 32 a shared 1,000-token
    prefix reuses at most 992 tokens."""
    pool = BlockPool(200, 32, enable_prefix_caching=True)
    rng = np.random.default_rng(0)
    prefix = list(rng.integers(0, 50000, 1000))
    a = prefix + list(rng.integers(0, 50000, 300))
    b = prefix + list(rng.integers(0, 50000, 17))
    pool.allocate("a", len(a), token_ids=a)
    assert pool.cached_tokens("a") == 0
    pool.allocate("b", len(b), token_ids=b)
    assert pool.cached_tokens("b") == 992
    assert pool.table("b")[:31] == pool.table("a")[:31]
    assert pool.table("b")[31] != pool.table("a")[31]
    assert all(pool.refcount(x) == 2 for x in pool.table("a")[:31])


def test_divergence_inside_a_block_loses_that_block():
    pool = BlockPool(100, 32, enable_prefix_caching=True)
    base = list(range(1000))
    other = list(base)
    other[500] = -7  # inside block 15 (tokens 480..511)
    pool.allocate("a", 1000, token_ids=base)
    pool.allocate("b", 1000, token_ids=other)
    assert pool.cached_tokens("b") == 15 * 32
    assert pool.table("b")[:15] == pool.table("a")[:15]


def test_freed_blocks_stay_matchable_until_reused_for_other_tokens():
    pool = BlockPool(12, 16, enable_prefix_caching=True)
    t = list(range(100, 164))  # 4 full blocks
    pool.allocate("a", 64, token_ids=t)
    first = pool.table("a")
    pool.free("a")
    pool.allocate("b", 64, token_ids=t)
    # the block holding the prompt's last token is never reused
    assert pool.cached_tokens("b") == 48 and pool.table("b")[:3] == first[:3]
    assert pool.table("b")[3] != first[3]
    pool.free("b")
    # 8 blocks never used come off the free list first (least recently freed) ...
    pool.allocate("c", 8 * 16, token_ids=list(range(5000, 5128)))
    pool.allocate("d", 64, token_ids=t)
    assert pool.cached_tokens("d") == 48
    pool.free("d")
    pool.free("c")
    # ... then the cached ones are overwritten by new tokens and stop matching
    pool.allocate("e", 12 * 16, token_ids=list(range(9000, 9192)))
    pool.free("e")
    pool.allocate("f", 64, token_ids=t)
    assert pool.cached_tokens("f") == 0


def test_appended_tokens_fill_blocks_that_join_the_cache():
    pool = BlockPool(20, 16, enable_prefix_caching=True)
    prompt = list(range(20))
    pool.allocate("a", 20, token_ids=prompt)
    gen = list(range(1000, 1030))
    for tok in gen:
        pool.append("a", 1, token_ids=[tok])
    full = prompt + gen  # 50 tokens: 3 full blocks
    pool.allocate("b", 48, token_ids=full[:48])
    assert pool.cached_tokens("b") == 32
    assert pool.table("b")[:2] == pool.table("a")[:2]
    pool.allocate("c", 49, token_ids=full[:49])
    assert pool.cached_tokens("c") == 48
    assert pool.table("c")[:3] == pool.table("a")[:3]


def test_a_full_hit_still_leaves_the_last_prompt_token_to_compute():
    """Every block of the prompt is cached: reuse stops one block short, so the
    step that produces the first output token has a token to compute and
    writes only into a block of its own."""
    pool = BlockPool(20, 16, enable_prefix_caching=True)
    t = list(range(64))
    pool.allocate("a", 64, token_ids=t)
    pool.allocate("b", 64, token_ids=t)
    assert pool.cached_tokens("b") == 48
    last = pool.table("b")[3]
    assert pool.refcount(last) == 1 and last != pool.table("a")[3]
    for n in (1, 15, 16, 17):
        pool.allocate(("s", n), n, token_ids=t[:n])
        assert pool.cached_tokens(("s", n)) == ((n - 1) // 16) * 16 < n


def test_prefix_caching_off_shares_nothing():
    pool = BlockPool(20, 16)
    pool.allocate("a", 40, token_ids=list(range(40)))
    pool.allocate("b", 40, token_ids=list(range(40)))
    assert pool.cached_tokens("b") == 0
    assert not set(pool.table("a")) & set(pool.table("b"))


# ------------------------------------------------------------------- swapping
def test_swap_out_releases_and_swap_in_takes_fresh_blocks():
    pool = BlockPool(10, 16)
    pool.allocate("a", 40)
    pool.allocate("b", 16)
    ids = pool.swap_out("a")
    assert list(ids) == [0, 1, 2] and pool.num_free == 9 and pool.is_swapped("a")
    pool.allocate("c", 48)  # reuses the released blocks
    back = pool.swap_in("a")
    assert len(back) == 3
    assert not set(back) & (set(pool.table("c")) | set(pool.table("b")))
    assert pool.num_tokens("a") == 40 and pool.slot("a", 39) == back[2] * 16 + 7
    pool.swap_out("b")
    pool.swap_out("c")
    pool.allocate("d", pool.num_free * 16)  # takes every free block
    with pytest.raises(OutOfBlocks):
        pool.swap_in("b")
    assert pool.is_swapped("b")


def test_shares_blocks_tells_when_a_decode_may_stream_the_pool():
    pool = BlockPool(64, 16)
    pool.allocate("a", 40)
    pool.allocate("b", 17)
    assert not pool.shares_blocks(["a", "b"])
    pool.fork("a", "c")  # c lists a's three blocks
    assert pool.shares_blocks(["a", "c"]) and pool.shares_blocks(["b", "c", "a"])
    assert not pool.shares_blocks(["b", "c"])  # a's blocks are shared, but not inside this batch
    for _ in range(30):
        pool.append("c")  # copy-on-write of the partly filled block, then fresh ones
    assert pool.shares_blocks(["a", "c"])  # the two full prompt blocks stay shared
    pool.free("a")
    assert not pool.shares_blocks(["b", "c"])


def test_tables_share_blocks_reads_only_the_used_columns():
    from paged_kv_cache_135_amd import tables_share_blocks
    t = np.array([[3, 4, 9], [5, 4, 0]], np.int32)
    assert tables_share_blocks(t, [40, 17], 16)        # block 4 in both sequences
    assert not tables_share_blocks(t, [40, 16], 16)    # sequence 1 uses only block 5
    assert not tables_share_blocks(t, [40, 17], 16, skip_blocks=2)  # past the prefix: 9 alone
    assert not tables_share_blocks(t[:0], [], 16)
