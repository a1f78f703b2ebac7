"""Pins for the oracle's block sizing against the pages' worked example.

"PagedAttention Memory Management" (apxml), section "Calculating Physical
Block Sizes": the block-size formula, its Qwen2.5-7B / FP16 / 16-token value
and the pool sizing that follows it (fixture: golden/block_size_example.txt).
"""
import oracle
from tests._golden import load


def test_block_bytes_worked_example():
    g = load("block_size_example.txt")
    got = oracle.block_bytes(g["num_layers"], g["num_kv_heads"], g["head_dim"],
                             g["block_tokens"], g["elem_bytes"])
    assert got == g["block_bytes"]


def test_block_bytes_terms():
    # each factor enters linearly; FP8 halves an FP16 block (P_bytes 1 vs 2)
    base = oracle.block_bytes(28, 4, 128, 16, 2)
    assert oracle.block_bytes(28, 4, 128, 16, 1) * 2 == base
    assert oracle.block_bytes(28, 4, 128, 32, 2) == 2 * base
    assert oracle.block_bytes(1, 1, 1, 1, 1) == 2


def test_pool_capacity_worked_example():
    g = load("block_size_example.txt")
    assert abs(g["device_gb"] - g["weights_gb"] - g["reserve_gb"] - g["kv_gb"]) < 1e-9
    blocks, tokens = oracle.pool_capacity(g["device_gb"] * 1e9, g["weights_gb"] * 1e9,
                                          g["reserve_gb"] * 1e9, g["block_bytes"],
                                          g["block_tokens"])
    assert abs(blocks - g["approx_blocks"]) / g["approx_blocks"] < 0.01
    assert abs(tokens - g["approx_tokens"]) / g["approx_tokens"] < 0.01
