"""The oracle on the small named workload (4 sequences, f32): every token
placed by the oracle's write, then decode, against torch's float64 attention on
the same tokens kept contiguous."""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads


def test_c1_write_then_decode_matches_library_attention():
    case = workloads.c1_tiny_f32()
    assert case.block_tables.shape == (4, 7)
    kc, vc = case.key_cache.copy(), case.value_cache.copy()
    oracle.paged_kv_write(case.fill_k, case.fill_v, case.fill_slots, kc, vc)
    got = oracle.paged_attention_decode(case.q, kc, vc, case.block_tables, case.context_lens,
                                        case.scale, case.block_size)
    o = 0
    for s, n in enumerate(case.context_lens):
        n = int(n)
        k = torch.from_numpy(case.fill_k[o:o + n].astype(np.float64)).permute(1, 0, 2)[None]
        v = torch.from_numpy(case.fill_v[o:o + n].astype(np.float64)).permute(1, 0, 2)[None]
        q = torch.from_numpy(case.q[s].astype(np.float64))[None, :, None, :]
        ref = F.scaled_dot_product_attention(q, k, v, scale=case.scale, enable_gqa=True)
        np.testing.assert_allclose(got[s], ref[0, :, 0, :].numpy(), rtol=1e-11, atol=1e-12)
        o += n
    # 13 of the 64 pool blocks are in use; the rest still hold the poison
    used = np.unique(np.concatenate([case.block_tables[s, :(int(n) + 15) // 16]
                                     for s, n in enumerate(case.context_lens)]))
    assert used.size == 13
    free = np.setdiff1d(np.arange(64), used)
    assert np.all(np.isnan(kc[free])) and np.all(np.isnan(vc[free]))


def test_waste_is_below_one_block_per_sequence():
    # "PagedAttention, clearly explained": waste is at most the unfilled tail of
    # one block; the small workload's tails are 15, 15, 8 and 12 slots
    case = workloads.c1_tiny_f32()
    bs = case.block_size
    waste = [(-int(n)) % bs for n in case.context_lens]
    assert waste == [15, 15, 8, 12]
    assert max(waste) <= bs - 1


def test_step_writes_into_a_shared_block_come_from_one_sequence():
    # "PagedAttention Memory Management", "Complex Topologies and Memory
    # Sharing": a block listed by several tables is copied before one of them
    # writes into it.  Sequences whose context ends inside the shared prefix
    # would all write its last slot; the generator lets the first of them write
    # and skips the others (slot -1), so no two writes of one step collide.
    case = workloads.build_case("ends_in_prefix", seed=5, context_lens=[64, 64, 70, 64, 90],
                                num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=32,
                                cache_dtype="bf16", std=0.5, scale=0.125, shared_prefix_blocks=2)
    slots = case.slot_mapping
    assert slots.size == 5
    live = slots[slots >= 0]
    assert np.unique(live).size == live.size
    last_prefix_slot = int(case.block_tables[0, 1]) * 32 + 31
    assert slots[0] == last_prefix_slot and slots[1] == -1 and slots[3] == -1
    assert slots[2] >= 0 and slots[4] >= 0
