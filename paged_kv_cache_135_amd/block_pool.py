"""Host-side block allocator for the paged KV cache (bookkeeping only, no GPU).

What it keeps, by page and section:
  * a pool of fixed-size physical blocks carved once, handed out from a free
    list ("pipe-paged-block-allocation-kv-cache", section "In and out": the
    free-block pool holds physical indices into one pre-allocated tensor per
    layer); it is kept as a queue so that, with prefix caching, the least
    recently freed block is the first one overwritten;
  * a block table per sequence mapping logical block j (tokens j*bs ..
    j*bs+bs-1) to a physical id ("PagedAttention, clearly explained"; foundry
    section "Concept": a page table by another name);
  * on-demand growth: a sequence starts with just enough blocks for its prompt
    and gains one block each time the last one fills ("What problem does
    PagedAttention solve...", section "The paging idea");
  * release on finish: blocks return to the pool when no table lists them;
  * reference counts and copy-on-write: forks list the same physical blocks,
    and a shared block is copied before one branch writes into it
    ("PagedAttention Memory Management", section "Complex Topologies and
    Memory Sharing"; katajob section "Sharing, the second dividend");
  * pool sizing from the memory left after weights and a reserve, with the
    per-block byte formula ("PagedAttention Memory Management", section
    "Calculating Physical Block Sizes");
  * prefix caching ("pipe-paged-block-allocation-kv-cache", section "The
    knobs": every filled block is hashed so unrelated requests with the same
    tokens share physical blocks; hashes are per block, so a shared prefix is
    reused only in whole blocks and a divergence inside a block loses that
    block, section "Failure modes"); a freed block keeps its hash and can be
    matched again until it is handed out for other tokens, least recently
    freed first;
  * swap-out / swap-in of a preempted sequence (katajob, section "Operational
    consequences"): its blocks are released after the caller gathers them to
    a staging buffer, and fresh blocks are taken when it comes back.

Slots handed to the KV write are ``physical_block * block_size + offset``.
Copy-on-write returns (source, destination) physical block pairs; copying the
block contents on the device is the caller's job before the write lands.
"""
from __future__ import annotations

import hashlib
from collections import deque
from dataclasses import dataclass, field

import numpy as np


class OutOfBlocks(MemoryError):
    """The free list cannot satisfy a request (the point where a scheduler
    would preempt a sequence)."""


def block_bytes(num_layers: int, num_kv_heads: int, head_dim: int, block_size: int,
                elem_bytes: int) -> int:
    """Bytes of one physical block over all layers, K and V."""
    return 2 * num_layers * num_kv_heads * head_dim * block_size * elem_bytes


def blocks_for_memory(free_bytes: int, one_block_bytes: int) -> int:
    """Whole blocks that fit in ``free_bytes``."""
    if one_block_bytes <= 0:
        raise ValueError("block bytes must be positive")
    return max(0, int(free_bytes) // int(one_block_bytes))


@dataclass
class _Seq:
    table: list = field(default_factory=list)
    num_tokens: int = 0
    hashes: list = field(default_factory=list)   # chain hash of each full block (prefix caching)
    tail: list = field(default_factory=list)     # token ids of the partly filled last block
    cached: int = 0                              # prompt tokens found in the prefix cache


def block_hash(parent: bytes, tokens) -> bytes:
    """Chain hash of one full block: its token ids and the hash of the block
    before it, so equal hashes mean equal prefixes up to this block."""
    h = hashlib.blake2b(parent, digest_size=16)
    h.update(np.asarray(tokens, dtype=np.int64).tobytes())
    return h.digest()


class BlockPool:
    """Free list + per-sequence block tables + reference counts (+ prefix cache)."""

    def __init__(self, num_blocks: int, block_size: int, max_model_len: int | None = None,
                 enable_prefix_caching: bool = False):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        if max_model_len is not None and num_blocks * block_size < max_model_len:
            # a pool that cannot hold one sequence of the maximum length is refused
            raise OutOfBlocks(
                f"pool of {num_blocks} x {block_size} slots cannot hold one sequence of "
                f"{max_model_len} tokens")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.prefix_caching = bool(enable_prefix_caching)
        # free queue: blocks are taken from the left, released ones go to the
        # right, so the least recently freed (cached) block is reused first
        self._free = deque(range(self.num_blocks))
        self._ref = np.zeros(self.num_blocks, dtype=np.int64)
        self._seqs: dict = {}
        self._hash_of: dict = {}    # block -> chain hash of its content
        self._block_of: dict = {}   # chain hash -> block
        self._swapped: dict = {}    # sequence -> its _Seq while swapped out
        self.prefix_hit_blocks = 0

    # ------------------------------------------------------------ queries
    @property
    def num_free(self) -> int:
        return len(self._free)

    def refcount(self, block: int) -> int:
        return int(self._ref[block])

    def table(self, seq) -> list:
        return list(self._seqs[seq].table)

    def num_tokens(self, seq) -> int:
        return self._seqs[seq].num_tokens

    def shares_blocks(self, seqs) -> bool:
        """True if some physical block sits in the tables of two of these
        sequences (a prefix or a fork).  A decode over them then reads that
        block more than once and should keep it cached; otherwise every block
        is read once and the call may stream the pool (stream_kv=True)."""
        ids = [b for s in seqs for b in self._seqs[s].table]
        return len(ids) != len(set(ids))

    def blocks_needed(self, n_tokens: int) -> int:
        return -(-int(n_tokens) // self.block_size)

    def slot(self, seq, position: int) -> int:
        s = self._seqs[seq]
        if not 0 <= position < s.num_tokens:
            raise IndexError("position outside the sequence")
        return s.table[position // self.block_size] * self.block_size + position % self.block_size

    # -------------------------------------------------------------- edits
    def _pop(self) -> int:
        if not self._free:
            raise OutOfBlocks("no free block")
        b = self._free.popleft()
        self._ref[b] = 1
        h = self._hash_of.pop(b, None)  # its cached content is overwritten from now on
        if h is not None and self._block_of.get(h) == b:
            del self._block_of[h]
        return b

    def _register(self, b: int, h: bytes) -> None:
        if h not in self._block_of:
            self._block_of[h] = b
            self._hash_of[b] = h

    def _chain(self, token_ids, n_full: int, parent: bytes = b"") -> list:
        bs = self.block_size
        out = []
        for j in range(n_full):
            parent = block_hash(parent, token_ids[j * bs:(j + 1) * bs])
            out.append(parent)
        return out

    def _release(self, b: int) -> None:
        self._ref[b] -= 1
        if self._ref[b] == 0:
            self._free.append(b)
        elif self._ref[b] < 0:  # pragma: no cover - bookkeeping bug
            raise AssertionError("negative reference count")

    def allocate(self, seq, n_tokens: int, prefix_of=None, prefix_blocks: int = 0,
                 token_ids=None) -> np.ndarray:
        """Admit a sequence with ``n_tokens`` prompt tokens; returns their slots.

        ``prefix_of``/``prefix_blocks``: the first ``prefix_blocks`` logical
        blocks are the ones another sequence already lists (a shared prompt
        prefix); only the rest are taken from the pool.

        ``token_ids`` (with prefix caching on): the prompt's token ids.  The
        longest run of leading full blocks whose chain hashes are cached is
        reused, short of the block holding the prompt's last token;
        ``cached_tokens(seq)`` then tells how many prompt tokens need no
        prefill (always fewer than ``n_tokens``)."""
        if seq in self._seqs or seq in self._swapped:
            raise KeyError(f"sequence {seq!r} exists")
        n_tokens = int(n_tokens)
        bs = self.block_size
        need = self.blocks_needed(n_tokens)
        shared = []
        hashes = []
        if token_ids is not None:
            token_ids = list(token_ids)
            if len(token_ids) != n_tokens:
                raise ValueError("token_ids must hold n_tokens ids")
            if self.prefix_caching:
                hashes = self._chain(token_ids, n_tokens // bs)
        if prefix_of is not None:
            src = self._seqs[prefix_of]
            if prefix_blocks > len(src.table) or prefix_blocks * bs > n_tokens:
                raise ValueError("prefix longer than the source or the new sequence")
            if prefix_blocks * bs > src.num_tokens:
                raise ValueError("only filled blocks can be shared")
            shared = src.table[:prefix_blocks]
        elif hashes:
            # reuse stops short of the prompt's last token: a full hit would
            # leave the step that produces the first output token nothing to
            # compute, and recomputing that token would write into a shared
            # block.  The final block is then taken fresh (block-granular).
            for h in hashes[:(n_tokens - 1) // bs]:
                b = self._block_of.get(h)
                if b is None:
                    break
                shared.append(b)
        fresh = need - len(shared)
        revive = sum(1 for b in shared if self._ref[b] == 0)
        if fresh + revive > len(self._free):
            raise OutOfBlocks(f"need {fresh} blocks, {len(self._free) - revive} free")
        for b in shared:
            if self._ref[b] == 0:
                self._free.remove(b)  # a cached block comes back into use
            self._ref[b] += 1
        if prefix_of is None:
            self.prefix_hit_blocks += len(shared)
        s = _Seq(table=list(shared) + [self._pop() for _ in range(fresh)], num_tokens=n_tokens)
        s.cached = len(shared) * bs if prefix_of is None else 0
        if token_ids is not None and self.prefix_caching:
            for j, h in enumerate(hashes):
                self._register(s.table[j], h)
            s.hashes = hashes
            s.tail = token_ids[len(hashes) * bs:]
        self._seqs[seq] = s
        return self._slots(s, 0, n_tokens)

    def cached_tokens(self, seq) -> int:
        """Prompt tokens of ``seq`` found in the prefix cache at admission."""
        return self._seqs[seq].cached

    def append(self, seq, n: int = 1, token_ids=None):
        """Grow a sequence by ``n`` tokens.  Returns (slots, cow_pairs): the new
        tokens' slots and the (source, destination) physical blocks to copy
        before writing (copy-on-write of a shared, partly filled last block).
        With prefix caching, ``token_ids`` of the new tokens let every block
        they fill join the cache."""
        s = self._seqs[seq]
        bs = self.block_size
        cow = []
        n = int(n)
        if token_ids is not None and len(token_ids) != n:
            raise ValueError("token_ids must hold n ids")
        if n <= 0:
            return np.zeros(0, np.int32), cow
        new_total = s.num_tokens + n
        extra = self.blocks_needed(new_total) - len(s.table)
        partial_shared = s.num_tokens % bs != 0 and self._ref[s.table[-1]] > 1
        if extra + (1 if partial_shared else 0) > len(self._free):
            raise OutOfBlocks(f"need {extra + partial_shared} blocks, {len(self._free)} free")
        if partial_shared:
            old = s.table[-1]
            new = self._pop()
            self._ref[old] -= 1
            s.table[-1] = new
            cow.append((old, new))
        for _ in range(extra):
            s.table.append(self._pop())
        first = s.num_tokens
        s.num_tokens = new_total
        if self.prefix_caching and token_ids is not None and len(s.hashes) * bs + len(s.tail) == first:
            s.tail = list(s.tail) + list(token_ids)
            while len(s.tail) >= bs:
                parent = s.hashes[-1] if s.hashes else b""
                h = block_hash(parent, s.tail[:bs])
                self._register(s.table[len(s.hashes)], h)
                s.hashes.append(h)
                s.tail = s.tail[bs:]
        return self._slots(s, first, new_total), cow

    def fork(self, seq, new_seq) -> None:
        """New sequence listing the same blocks (parallel sampling, beam search)."""
        if new_seq in self._seqs:
            raise KeyError(f"sequence {new_seq!r} exists")
        s = self._seqs[seq]
        for b in s.table:
            self._ref[b] += 1
        self._seqs[new_seq] = _Seq(table=list(s.table), num_tokens=s.num_tokens)

    def free(self, seq) -> None:
        """Finish a sequence: its blocks go back to the pool once unreferenced
        (with prefix caching, still matchable until handed out again)."""
        s = self._seqs.pop(seq, None)
        if s is None:
            self._swapped.pop(seq)
            return
        for b in reversed(s.table):
            self._release(b)

    def swap_out(self, seq) -> np.ndarray:
        """Preempt ``seq``: returns its physical blocks in logical order (the
        caller gathers them to a staging buffer before anything else is
        written to the pool) and releases them."""
        s = self._seqs.pop(seq)
        ids = np.asarray(s.table, dtype=np.int32)
        for b in reversed(s.table):
            self._release(b)
        s.table = []
        self._swapped[seq] = s
        return ids

    def swap_in(self, seq) -> np.ndarray:
        """Bring ``seq`` back: takes fresh blocks and returns them in logical
        order (the caller scatters the staged blocks into them)."""
        s = self._swapped[seq]
        need = self.blocks_needed(s.num_tokens)
        if need > len(self._free):
            raise OutOfBlocks(f"need {need} blocks, {len(self._free)} free")
        del self._swapped[seq]
        s.table = [self._pop() for _ in range(need)]
        for j, h in enumerate(s.hashes):
            self._register(s.table[j], h)
        self._seqs[seq] = s
        return np.asarray(s.table, dtype=np.int32)

    def is_swapped(self, seq) -> bool:
        return seq in self._swapped

    # ---------------------------------------------------- kernel inputs
    def _slots(self, s: _Seq, lo: int, hi: int) -> np.ndarray:
        pos = np.arange(lo, hi, dtype=np.int64)
        tab = np.asarray(s.table, dtype=np.int64)
        return (tab[pos // self.block_size] * self.block_size + pos % self.block_size).astype(np.int32)

    def block_tables(self, seqs, pad: int = 0) -> np.ndarray:
        """int32 [len(seqs), max blocks] tables, padded with ``pad``."""
        seqs = list(seqs)
        width = max([1] + [len(self._seqs[q].table) for q in seqs])
        out = np.full((len(seqs), width), pad, dtype=np.int32)
        for i, q in enumerate(seqs):
            t = self._seqs[q].table
            out[i, :len(t)] = t
        return out

    def context_lens(self, seqs) -> np.ndarray:
        return np.array([self._seqs[q].num_tokens for q in seqs], dtype=np.int32)

    def decode_order(self, seqs) -> np.ndarray:
        """Positions of ``seqs`` (as batched by block_tables / context_lens),
        longest context first, ties in batch order: the decode's seq_order
        (the same order as the library's pkv_decode_order)."""
        return np.argsort(-self.context_lens(seqs).astype(np.int64), kind="stable").astype(np.int32)

    def stats(self) -> dict:
        """Live-KV fraction (tokens held / slots of blocks in use, each physical
        block counted once) and per-sequence tail waste."""
        in_use = int((self._ref > 0).sum())
        bs = self.block_size
        live = set()
        for s in self._seqs.values():
            for j, b in enumerate(s.table):
                filled = min(bs, s.num_tokens - j * bs)
                live.add((b, filled))
        # a shared block counts its filled slots once (the largest fill seen)
        best = {}
        for b, f in live:
            best[b] = max(best.get(b, 0), f)
        held = sum(best.values())
        waste = {q: (-s.num_tokens) % bs if s.table else 0 for q, s in self._seqs.items()}
        return {
            "blocks_in_use": in_use,
            "blocks_free": len(self._free),
            "blocks_cached": len(self._hash_of),
            "prefix_hit_blocks": self.prefix_hit_blocks,
            "live_fraction": held / (in_use * bs) if in_use else 1.0,
            "waste_per_seq": waste,
            "max_waste": max(waste.values()) if waste else 0,
        }
