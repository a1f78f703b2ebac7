"""Seeded synthetic inputs for the paged KV cache hot path.

This module is shared by the oracle's tests, the GPU parity tests and the
benchmark.  It only draws numbers and lays out tables: it performs none of the
computations under test (no KV write, no gather, no attention, no FP8 coding),
so neither side can lean on the other through it.

Workload shapes follow the pages:
  * block size 16 by default, 16 or 32 allowed ("PagedAttention Memory
    Management", section "Internal and External Fragmentation Constraints";
    "pipe-paged-block-allocation-kv-cache", section "The knobs");
  * Qwen2.5-7B-like layer: 4 KV heads, head dim 128 ("PagedAttention Memory
    Management", section "Calculating Physical Block Sizes", worked example),
    with 28 query heads;
  * physical block ids scattered over one pool, shared blocks listed by many
    tables ("What problem does PagedAttention solve", sections "The paging
    idea" and "Sharing, the second dividend").

Random streams: numpy PCG64 seeded from (seed, stream, chunk) so that tables
and data use separate streams and large arrays fill in parallel chunks with a
result that does not depend on the number of threads.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)
F32_NAN_BITS = np.uint32(0x7FC00000)

_STREAM_TABLES, _STREAM_Q, _STREAM_K, _STREAM_V, _STREAM_NEWK, _STREAM_NEWV, _STREAM_CHUNK, \
    _STREAM_PREFILL = range(8)
_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); finite input."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & 1
    return ((u + np.uint32(0x7FFF) + r) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _amax(x: np.ndarray) -> np.float32:
    """Largest magnitude of finite float32 or bfloat16-bits data.  For bf16 the
    order of non-negative values is the order of their bit patterns, so the
    sign-cleared bits are compared instead of converting every element."""
    if x.dtype == np.uint16:
        top = np.bitwise_and(x, np.uint16(0x7FFF)).max(initial=0)
        return np.float32(bf16_to_f32(np.array([top], np.uint16))[0])
    return np.float32(np.abs(x).max(initial=0.0))


def fill_normal(out: np.ndarray, std: float, seed: int, stream: int) -> np.ndarray:
    """Fill ``out`` (float32, or uint16 = bfloat16 bits) with N(0,1)*std draws."""
    flat = out.reshape(-1)
    n = flat.size
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def one(c: int):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        rng = np.random.default_rng([seed, stream, c])
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        x *= np.float32(std)
        if flat.dtype == np.float32:
            flat[lo:hi] = x
        else:
            flat[lo:hi] = bf16_bits_from_f32(x)

    if nchunks <= 1:
        for c in range(nchunks):
            one(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(nchunks)))
    return out


def _poison_value(elem: str):
    return {"f32": np.float32(np.nan), "bf16": BF16_NAN, "fp8_e4m3": FP8_NAN}[elem]


def _np_dtype(elem: str):
    return {"f32": np.float32, "bf16": np.uint16, "fp8_e4m3": np.uint8}[elem]


@dataclass
class PagedCase:
    """One decode step's inputs, as host arrays.

    Element types: float32 = f32, uint16 = bfloat16 bits, uint8 = E4M3 codes.

    ``key_cache``/``value_cache`` hold the pool before this step's writes.
    ``fill_k``/``fill_v``/``fill_slots`` (possibly empty) are writes that
    bring the pool to its pre-step state (the cache is then a poisoned pool and
    these tokens land through the KV write).  ``k_new``/``v_new``/
    ``slot_mapping`` are this step's writes; decode runs after all writes.
    """

    name: str
    cache_dtype: str          # "f32" | "bf16" | "fp8_e4m3"
    q: np.ndarray             # [S, Hq, D]
    key_cache: np.ndarray     # [NB, Hkv, bs, D]
    value_cache: np.ndarray
    block_tables: np.ndarray  # int32 [S, max_blocks]
    context_lens: np.ndarray  # int32 [S]
    block_size: int
    scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    fill_k: np.ndarray | None = None
    fill_v: np.ndarray | None = None
    fill_slots: np.ndarray | None = None
    k_new: np.ndarray | None = None
    v_new: np.ndarray | None = None
    slot_mapping: np.ndarray | None = None
    free_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))
    shared_blocks: int = 0
    query_start: np.ndarray | None = None  # prefill: int32 [S+1] row offsets of q's sequences
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.key_cache.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    @property
    def num_blocks(self) -> int:
        return int(self.key_cache.shape[0])

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes one decode call reads: every attended token's
        K and V row for every KV head (block-tail padding not counted)."""
        elem = self.key_cache.dtype.itemsize
        return int(self.context_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * \
            self.head_dim * elem

    def prefill_flops(self) -> int:
        """Algorithmic flops of one chunked-prefill call: q.K and P.V (2 flops
        per multiply-add each) for every query head and every key a query
        sees (keys up to and including its own position)."""
        qs = self.query_start.astype(np.int64)
        ctx = self.context_lens.astype(np.int64)
        nq = qs[1:] - qs[:-1]
        # queries sit at positions ctx-nq .. ctx-1 and see pos + 1 keys each
        keys = (nq * (ctx - nq) + nq * (nq + 1) // 2).sum()
        return int(keys) * self.num_q_heads * self.head_dim * 4

    def prefill_kv_bytes(self) -> int:
        """K/V bytes a chunked-prefill call must read at least once: every
        context token of every sequence with queries, each KV head."""
        qs = self.query_start.astype(np.int64)
        live = (qs[1:] - qs[:-1]) > 0
        elem = self.key_cache.dtype.itemsize
        return int(self.context_lens.astype(np.int64)[live].sum()) * 2 * self.num_kv_heads * \
            self.head_dim * elem

    def unique_kv_bytes(self) -> int:
        """KV bytes counting each shared physical block once."""
        elem = self.key_cache.dtype.itemsize
        tok = int(self.context_lens.astype(np.int64).sum()) - \
            (self.num_seqs - 1) * self.shared_blocks * self.block_size if self.shared_blocks else \
            int(self.context_lens.astype(np.int64).sum())
        return tok * 2 * self.num_kv_heads * self.head_dim * elem


def slots_of(block_tables: np.ndarray, seq: int, positions: np.ndarray, block_size: int) -> np.ndarray:
    """Cache slot (physical block * block_size + offset) of logical positions of one sequence."""
    pos = np.asarray(positions, dtype=np.int64)
    return (block_tables[seq, pos // block_size].astype(np.int64) * block_size +
            pos % block_size).astype(np.int32)


def build_case(name: str, *, seed: int, context_lens, num_q_heads: int, num_kv_heads: int,
               head_dim: int, block_size: int, cache_dtype: str, std: float, scale: float,
               shared_prefix_blocks: int = 0, spare_fraction: float = 0.1,
               num_blocks: int | None = None, poison: bool = True, fill_via_write: bool = False,
               new_token_step: bool = True, prefill_chunk: int = 0) -> PagedCase:
    """Lay out one pool, its block tables and data.

    Tables: the pool holds ``ceil((1 + spare_fraction) * needed)`` blocks
    (shared prefix blocks counted once); physical ids come from one seeded
    shuffle, the shared prefix first, then each sequence's private blocks.
    Entries past a sequence's last block name a poisoned free block.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    S = ctx.size
    bs = block_size
    nb = (ctx + bs - 1) // bs
    if shared_prefix_blocks:
        if np.any(ctx < shared_prefix_blocks * bs):
            raise ValueError("every sequence must cover the shared prefix")
    private = nb - shared_prefix_blocks
    needed = shared_prefix_blocks + int(private.sum())
    NB = num_blocks if num_blocks is not None else int(math.ceil((1.0 + spare_fraction) * needed))
    if NB < needed:
        raise ValueError("pool too small")
    rng_t = np.random.default_rng([seed, _STREAM_TABLES])
    perm = rng_t.permutation(NB).astype(np.int32)
    shared_ids = perm[:shared_prefix_blocks]
    cursor = shared_prefix_blocks
    max_blocks = max(1, int(nb.max()) if S else 1)
    free = perm[needed:]
    pad = int(free[0]) if free.size else 0
    tables = np.full((S, max_blocks), pad, dtype=np.int32)
    for s in range(S):
        tables[s, :shared_prefix_blocks] = shared_ids
        k = int(private[s])
        tables[s, shared_prefix_blocks:shared_prefix_blocks + k] = perm[cursor:cursor + k]
        cursor += k

    elem = cache_dtype
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    in_elem = "f32" if cache_dtype == "f32" else "bf16"
    q = np.empty((S, Hq, D), dtype=_np_dtype(in_elem))
    fill_normal(q, std, seed, _STREAM_Q)

    kc = np.empty((NB, Hkv, bs, D), dtype=_np_dtype(elem))
    vc = np.empty_like(kc)
    case = PagedCase(name=name, cache_dtype=cache_dtype, q=q, key_cache=kc, value_cache=vc,
                     block_tables=tables, context_lens=ctx.astype(np.int32), block_size=bs,
                     scale=float(np.float32(scale)), free_blocks=free.copy(),
                     shared_blocks=shared_prefix_blocks)

    if fill_via_write or cache_dtype == "fp8_e4m3":
        # poisoned pool; every attended token arrives through the KV write
        kc.fill(_poison_value(elem))
        vc.fill(_poison_value(elem))
        T = int(ctx.sum())
        fk = np.empty((T, Hkv, D), dtype=_np_dtype(in_elem))
        fv = np.empty_like(fk)
        fill_normal(fk, std, seed, _STREAM_K)
        fill_normal(fv, std, seed, _STREAM_V)
        slots = np.empty(T, dtype=np.int32)
        o = 0
        for s in range(S):
            n = int(ctx[s])
            slots[o:o + n] = slots_of(tables, s, np.arange(n), bs)
            o += n
        if shared_prefix_blocks:
            # shared blocks are written once, by the first sequence
            keep = np.ones(T, dtype=bool)
            o = 0
            for s in range(S):
                if s > 0:
                    keep[o:o + shared_prefix_blocks * bs] = False
                o += int(ctx[s])
            fk, fv, slots = fk[keep], fv[keep], slots[keep]
        case.fill_k, case.fill_v, case.fill_slots = fk, fv, slots
        if cache_dtype == "fp8_e4m3":
            # per-tensor scales: amax / 448, fixed when the cache is created
            case.k_scale = float(_amax(fk) / np.float32(448.0))
            case.v_scale = float(_amax(fv) / np.float32(448.0))
    else:
        fill_normal(kc, std, seed, _STREAM_K)
        fill_normal(vc, std, seed, _STREAM_V)
        if poison:
            pv = _poison_value(elem)
            if free.size:
                kc[free] = pv
                vc[free] = pv
            for s in range(S):
                n = int(ctx[s])
                if n % bs:
                    last = tables[s, (n - 1) // bs]
                    kc[last, :, n % bs:, :] = pv
                    vc[last, :, n % bs:, :] = pv

    if new_token_step and S:
        # this step's token: position ctx-1 of every sequence with ctx > 0
        live = np.nonzero(ctx > 0)[0]
        slots = np.array([slots_of(tables, int(s), [int(ctx[s]) - 1], bs)[0] for s in live],
                         dtype=np.int32)
        # a slot in a block several tables share (a sequence whose context
        # ends inside the shared prefix) is written by the first of them only:
        # the others would first need a copy-on-write of that block
        _, first = np.unique(slots, return_index=True)
        dup = np.ones(slots.size, dtype=bool)
        dup[first] = False
        slots[dup] = -1
        kn = np.empty((live.size, Hkv, D), dtype=_np_dtype(in_elem))
        vn = np.empty_like(kn)
        fill_normal(kn, std, seed, _STREAM_NEWK)
        fill_normal(vn, std, seed, _STREAM_NEWV)
        case.k_new, case.v_new, case.slot_mapping = kn, vn, slots
    if prefill_chunk:
        # a prefill chunk written into distinct random slots of free blocks
        rng_c = np.random.default_rng([seed, _STREAM_CHUNK])
        free_slots = (free.astype(np.int64)[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
        if free_slots.size < prefill_chunk:
            raise ValueError("not enough free slots for the prefill chunk")
        pick = rng_c.choice(free_slots.size, size=prefill_chunk, replace=False)
        slots = free_slots[pick].astype(np.int32)
        kn = np.empty((prefill_chunk, Hkv, D), dtype=_np_dtype(in_elem))
        vn = np.empty_like(kn)
        fill_normal(kn, std, seed + 7919, _STREAM_NEWK)
        fill_normal(vn, std, seed + 7919, _STREAM_NEWV)
        case.k_new, case.v_new, case.slot_mapping = kn, vn, slots
    case.meta = dict(seed=seed, needed_blocks=needed)
    return case


def build_prefill_case(name: str, *, seed: int, prefix_lens, chunk_lens, num_q_heads: int,
                       num_kv_heads: int, head_dim: int, block_size: int, cache_dtype: str,
                       std: float, scale: float, **kw) -> PagedCase:
    """A chunked-prefill batch: sequence s already holds ``prefix_lens[s]``
    tokens and gets ``chunk_lens[s]`` new ones.  The pool (built as in
    ``build_case``) holds all ``prefix + chunk`` tokens, the chunk's K/V
    included (they are written before the attention runs).  ``q`` is the packed
    [sum(chunk), Hq, D] block of the chunks' queries; ``query_start`` [S+1]
    gives each sequence's first row."""
    pre = np.asarray(prefix_lens, dtype=np.int64)
    chk = np.asarray(chunk_lens, dtype=np.int64)
    if pre.shape != chk.shape or np.any(pre < 0) or np.any(chk < 0):
        raise ValueError("prefix and chunk lengths must be non-negative and of equal count")
    case = build_case(name, seed=seed, context_lens=pre + chk, num_q_heads=num_q_heads,
                      num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
                      cache_dtype=cache_dtype, std=std, scale=scale, new_token_step=False, **kw)
    qs = np.zeros(chk.size + 1, dtype=np.int32)
    qs[1:] = np.cumsum(chk)
    in_elem = "f32" if cache_dtype == "f32" else "bf16"
    q = np.empty((int(qs[-1]), num_q_heads, head_dim), dtype=_np_dtype(in_elem))
    fill_normal(q, std, seed, _STREAM_PREFILL)
    case.q = q
    case.query_start = qs
    return case


# ----------------------------------------------------------- named workloads
def c1_tiny_f32() -> PagedCase:
    """4 sequences (lengths 1, 17, 40, 100), 4 q / 2 KV heads, head dim 64,
    block size 16, pool of 64 blocks, f32, q/K/V ~ N(0,1); every token placed
    by the KV write."""
    return build_case("c1_tiny_f32", seed=1000, context_lens=[1, 17, 40, 100], num_q_heads=4,
                      num_kv_heads=2, head_dim=64, block_size=16, cache_dtype="f32", std=1.0,
                      scale=1.0 / 8.0, num_blocks=64, fill_via_write=True, new_token_step=False)


def c2_qwen_decode(seed: int = 1001, num_seqs: int = 64, block_size: int = 16,
                   num_q_heads: int = 28) -> PagedCase:
    """Qwen2.5-7B-shaped decode layer, bf16: 28 q / 4 KV heads, head dim 128,
    lengths uniform in [128, 4096], pool sized to fit plus 10% free.
    num_q_heads: another multiple of 4 gives the same K/V with another group
    size (named c2_qwen_decode_hq<N>)."""
    rng = np.random.default_rng([seed, 99])
    ctx = rng.integers(128, 4097, size=num_seqs)
    name = "c2_qwen_decode" if num_q_heads == 28 else f"c2_qwen_decode_hq{num_q_heads}"
    return build_case(name, seed=seed, context_lens=ctx, num_q_heads=num_q_heads,
                      num_kv_heads=4, head_dim=128, block_size=block_size, cache_dtype="bf16",
                      std=0.5, scale=1.0 / math.sqrt(128))


def c3_shared_prefix(seed: int = 1002, num_seqs: int = 256) -> PagedCase:
    """Chat batch with a shared 1024-token system prompt (64 shared blocks),
    then private tails of log-normal length (median 300, sigma 1, cap 8192);
    32 q / 8 KV heads, head dim 128, bf16."""
    rng = np.random.default_rng([seed, 99])
    tail = np.clip(np.rint(np.exp(rng.normal(math.log(300.0), 1.0, size=num_seqs))), 1, 8192)
    ctx = 1024 + tail.astype(np.int64)
    return build_case("c3_shared_prefix", seed=seed, context_lens=ctx, num_q_heads=32,
                      num_kv_heads=8, head_dim=128, block_size=16, cache_dtype="bf16", std=0.5,
                      scale=1.0 / math.sqrt(128), shared_prefix_blocks=64)


def c4_long_context(block_size: int = 16, seed: int = 1003, num_seqs: int = 8,
                    context_len: int = 131072) -> PagedCase:
    """8 sequences of 131072 tokens, 28 q / 4 KV heads, head dim 128, bf16."""
    return build_case(f"c4_long_bs{block_size}", seed=seed, context_lens=[context_len] * num_seqs,
                      num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=block_size,
                      cache_dtype="bf16", std=0.5, scale=1.0 / math.sqrt(128))


def c5_fp8(seed: int = 1004, num_seqs: int = 512, prefill_chunk: int = 4096) -> PagedCase:
    """E4M3 cache with per-tensor scales: lengths uniform in [16, 2048], 32 q /
    8 KV heads, head dim 128, plus a 4096-token bf16 prefill chunk written into
    random free slots."""
    rng = np.random.default_rng([seed, 99])
    ctx = rng.integers(16, 2049, size=num_seqs)
    return build_case("c5_fp8", seed=seed, context_lens=ctx, num_q_heads=32, num_kv_heads=8,
                      head_dim=128, block_size=16, cache_dtype="fp8_e4m3", std=0.5,
                      scale=1.0 / math.sqrt(128), new_token_step=False,
                      prefill_chunk=prefill_chunk)


WORKLOADS = {
    "c1": c1_tiny_f32,
    "c2": c2_qwen_decode,
    "c3": c3_shared_prefix,
    "c4": c4_long_context,
    "c5": c5_fp8,
}


def p1_chunked_prefill(seed: int = 1005, num_seqs: int = 8, chunk: int = 512,
                       max_prefix: int = 3584) -> PagedCase:
    """Chunked prefill in the Qwen2.5-7B shape (28 q / 4 KV heads, head dim
    128, bf16, block size 16): 8 sequences, each with a cached prefix of
    U[0, 3584] tokens read through its block table and a 512-token chunk of
    new queries, 4,096 query tokens in all."""
    rng = np.random.default_rng([seed, _STREAM_TABLES + 100])
    prefix = rng.integers(0, max_prefix + 1, size=num_seqs)
    return build_prefill_case("p1_chunked_prefill", seed=seed, prefix_lens=prefix,
                              chunk_lens=[chunk] * num_seqs, num_q_heads=28, num_kv_heads=4,
                              head_dim=128, block_size=16, cache_dtype="bf16", std=0.5,
                              scale=1.0 / math.sqrt(128))
