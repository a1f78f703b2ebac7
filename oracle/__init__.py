"""Plain fp64 CPU oracle for the paged KV cache hot path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``paged_kv_cache_135_amd`` and the HIP library behind ``include/pagedkv.h``)
never imports, links or runs anything here, and nothing here imports it.

The arithmetic lives in ``oracle.c`` (plain C loops in double precision); this
module only marshals numpy arrays.  Element types travel as numpy dtypes:
``float32`` is f32, ``uint16`` carries bfloat16 bit patterns and ``uint8``
carries OCP E4M3 codes.

Sources, by page and section:
  * block_bytes: "PagedAttention Memory Management" (apxml), section
    "Calculating Physical Block Sizes", the block-size formula.
  * pool_capacity: same section, the worked sizing of the pool from the memory
    left after weights and the runtime reserve.
  * paged_kv_write / paged_attention_decode / paged_attention_prefill /
    copy_blocks / the E4M3 codec: see oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
_ERRORS = {1: "bad argument", 2: "slot or block id outside the pool", 3: "out of memory"}

_lib = None


def build() -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
        "-fno-fast-math", "-o", _LIB_PATH + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.orc_e4m3_decode_n.argtypes = [P, i64, P]
    lib.orc_e4m3_decode_n.restype = None
    lib.orc_e4m3_encode_n.argtypes = [P, i64, P]
    lib.orc_e4m3_encode_n.restype = None
    lib.orc_paged_kv_write.argtypes = [P, P, ctypes.c_int, P, i64, i32, i32, P, P, ctypes.c_int,
                                       i64, i32, f32, f32]
    lib.orc_paged_kv_write.restype = ctypes.c_int
    lib.orc_paged_attention_decode.argtypes = [P, ctypes.c_int, P, P, ctypes.c_int, P, P, i32, i32,
                                               i32, i32, i64, i32, i32, f32, f32, f32, P, P]
    lib.orc_paged_attention_decode.restype = ctypes.c_int
    lib.orc_copy_blocks.argtypes = [P, P, i64, i64, P, i64]
    lib.orc_copy_blocks.restype = ctypes.c_int
    lib.orc_paged_attention_prefill.argtypes = [P, ctypes.c_int, P, P, ctypes.c_int, P, P, P, i32,
                                                i32, i32, i32, i64, i32, i32, f32, f32, f32, P]
    lib.orc_paged_attention_prefill.restype = ctypes.c_int
    lib.orc_move_blocks.argtypes = [P, i64, i64, P, P, i64, ctypes.c_int]
    lib.orc_move_blocks.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _tag(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8_E4M3
    raise TypeError(f"unsupported element type {a.dtype}")


def _check(status: int):
    if status != 0:
        raise ValueError(f"oracle: {_ERRORS.get(status, status)}")


# ----------------------------------------------------------------- sizing
def block_bytes(num_layers: int, num_kv_heads: int, head_dim: int, block_tokens: int,
                elem_bytes: int) -> int:
    """Bytes of one physical block across all layers: K and V (the factor 2)
    for every layer, KV head, head dimension and token slot of the block."""
    return 2 * num_layers * num_kv_heads * head_dim * block_tokens * elem_bytes


def pool_capacity(device_bytes: float, weight_bytes: float, reserve_bytes: float,
                  one_block_bytes: int, block_tokens: int) -> tuple[float, float]:
    """(blocks, tokens) that fit in the memory left after the weights and the
    runtime reserve, as unrounded ratios."""
    kv = device_bytes - weight_bytes - reserve_bytes
    blocks = kv / one_block_bytes
    return blocks, blocks * block_tokens


# -------------------------------------------------------------- E4M3 codec
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_e4m3_decode_n(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint8)
    _load().orc_e4m3_encode_n(_ptr(a), a.size, _ptr(out))
    return out


# ------------------------------------------------------------- hot path
def paged_kv_write(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray,
                   key_cache: np.ndarray, value_cache: np.ndarray,
                   k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Write tokens' K/V ([T, Hkv, D]) into the caches ([NB, Hkv, bs, D]) in place."""
    for a in (k, v, slot_mapping, key_cache, value_cache):
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    T, H, D = k.shape
    NB, Hc, bs, Dc = key_cache.shape
    if v.shape != k.shape or value_cache.shape != key_cache.shape or (Hc, Dc) != (H, D):
        raise ValueError("shape mismatch")
    if slot_mapping.dtype != np.int32 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int32 [T]")
    if key_cache.dtype != value_cache.dtype or k.dtype != v.dtype:
        raise ValueError("dtype mismatch")
    _check(_load().orc_paged_kv_write(
        _ptr(k), _ptr(v), _tag(k), _ptr(slot_mapping), T, H, D, _ptr(key_cache),
        _ptr(value_cache), _tag(key_cache), NB, bs, float(k_scale), float(v_scale)))


def paged_attention_decode(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                           block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                           block_size: int, k_scale: float = 1.0, v_scale: float = 1.0,
                           row_mask: np.ndarray | None = None) -> np.ndarray:
    """fp64 decode attention; returns [S, Hq, D] float64.  Rows excluded by
    row_mask ([S, Hq] bool) are returned as NaN."""
    for a in (q, key_cache, value_cache, block_tables, context_lens):
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    S, Hq, D = q.shape
    NB, Hkv, bs, Dc = key_cache.shape
    if bs != block_size or Dc != D or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if block_tables.dtype != np.int32 or context_lens.dtype != np.int32:
        raise ValueError("tables and lengths must be int32")
    if block_tables.ndim != 2 or block_tables.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("tables must be [S, max_blocks], lengths [S]")
    out = np.full((S, Hq, D), np.nan, dtype=np.float64)
    mask_arg = None
    if row_mask is not None:
        m = np.ascontiguousarray(row_mask, dtype=np.uint8)
        if m.shape != (S, Hq):
            raise ValueError("row_mask must be [S, Hq]")
        mask_arg = _ptr(m)
    _check(_load().orc_paged_attention_decode(
        _ptr(q), _tag(q), _ptr(key_cache), _ptr(value_cache), _tag(key_cache),
        _ptr(block_tables), _ptr(context_lens), S, Hq, Hkv, D, NB, bs,
        block_tables.shape[1], float(scale), float(k_scale), float(v_scale), mask_arg, _ptr(out)))
    return out


def copy_blocks(key_cache: np.ndarray, value_cache: np.ndarray, pairs: np.ndarray) -> None:
    """Copy-on-write block copies in place: for each (src, dst) row of the int32
    [P, 2] array, block dst of both pools becomes a copy of block src."""
    if key_cache.shape != value_cache.shape or key_cache.dtype != value_cache.dtype:
        raise ValueError("pools differ")
    for a in (key_cache, value_cache, pairs):
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    pr = np.ascontiguousarray(pairs, dtype=np.int32)
    if pr.ndim != 2 or pr.shape[1] != 2:
        raise ValueError("pairs must be [P, 2]")
    nb = key_cache.shape[0]
    bb = key_cache[0].nbytes if nb else 0
    _check(_load().orc_copy_blocks(_ptr(key_cache), _ptr(value_cache), nb, bb, _ptr(pr),
                                   pr.shape[0]))


def paged_attention_prefill(q: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                            block_tables: np.ndarray, context_lens: np.ndarray,
                            query_start: np.ndarray, scale: float, block_size: int,
                            k_scale: float = 1.0, v_scale: float = 1.0) -> np.ndarray:
    """fp64 chunked-prefill attention; q is [T, Hq, D] with sequence s's queries
    in rows query_start[s] .. query_start[s+1]-1, at the last positions of its
    context.  Returns [T, Hq, D] float64."""
    for a in (q, key_cache, value_cache, block_tables, context_lens, query_start):
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    T, Hq, D = q.shape
    NB, Hkv, bs, Dc = key_cache.shape
    S = context_lens.shape[0]
    if bs != block_size or Dc != D or value_cache.shape != key_cache.shape:
        raise ValueError("shape mismatch")
    if (block_tables.dtype != np.int32 or context_lens.dtype != np.int32
            or query_start.dtype != np.int32):
        raise ValueError("tables, lengths and query starts must be int32")
    if block_tables.shape[0] != S or query_start.shape != (S + 1,) or query_start[-1] != T:
        raise ValueError("tables must be [S, max_blocks], query_start [S+1] ending at T")
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    _check(_load().orc_paged_attention_prefill(
        _ptr(q), _tag(q), _ptr(key_cache), _ptr(value_cache), _tag(key_cache),
        _ptr(block_tables), _ptr(context_lens), _ptr(query_start), S, Hq, Hkv, D, NB, bs,
        block_tables.shape[1], float(scale), float(k_scale), float(v_scale), _ptr(out)))
    return out


def gather_blocks(pool: np.ndarray, block_ids: np.ndarray) -> np.ndarray:
    """Swap-out: staging slot i = pool block ids[i] (slots of negative ids stay 0)."""
    if not pool.flags.c_contiguous:
        raise ValueError("oracle arrays must be C-contiguous")
    ids = np.ascontiguousarray(block_ids, dtype=np.int32)
    out = np.zeros((ids.size,) + pool.shape[1:], dtype=pool.dtype)
    bb = pool[0].nbytes if pool.shape[0] else 0
    _check(_load().orc_move_blocks(_ptr(pool), pool.shape[0], bb, _ptr(out), _ptr(ids), ids.size, 1))
    return out


def scatter_blocks(stage: np.ndarray, block_ids: np.ndarray, pool: np.ndarray) -> None:
    """Swap-in, in place: pool block ids[i] = staging slot i (negative ids skipped)."""
    if not pool.flags.c_contiguous or not stage.flags.c_contiguous:
        raise ValueError("oracle arrays must be C-contiguous")
    ids = np.ascontiguousarray(block_ids, dtype=np.int32)
    if stage.shape != (ids.size,) + pool.shape[1:] or stage.dtype != pool.dtype:
        raise ValueError("staging buffer must be [n] + one block")
    bb = pool[0].nbytes if pool.shape[0] else 0
    _check(_load().orc_move_blocks(_ptr(pool), pool.shape[0], bb, _ptr(stage), _ptr(ids), ids.size, 0))
