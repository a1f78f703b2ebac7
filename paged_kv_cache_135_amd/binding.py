"""ctypes binding of libpagedkv.so (include/pagedkv.h).

Argument marshalling only: torch tensors are described to the C ABI (pointer,
dtype, shape, strides) and the work is queued on torch's current HIP stream.
Every step of the hot path runs in the library's HIP kernels; if the library
is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_F32, PKV_BF16, PKV_FP8_E4M3, PKV_I32 = 0, 1, 2, 3
STATUS_NAMES = {
    0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_DTYPE", 3: "PKV_ERR_SHAPE", 4: "PKV_ERR_LAYOUT",
    5: "PKV_ERR_UNSUPPORTED", 6: "PKV_ERR_WORKSPACE", 7: "PKV_ERR_HIP", 8: "PKV_ERR_RANGE",
}
EXPORTED = (
    "pkv_abi_version", "pkv_last_error", "paged_kv_write", "paged_attention_decode",
    "paged_attention_decode_merge", "paged_attention_decode_append", "paged_attention_prefill",
    "paged_attention_decode_workspace_bytes", "paged_kv_copy_blocks", "pkv_validate_slots",
    "pkv_validate_decode_inputs", "pkv_validate_append_slots", "pkv_validate_prefill_inputs",
    "pkv_validate_block_pairs", "paged_kv_gather_blocks", "paged_kv_scatter_blocks",
    "pkv_validate_block_ids", "paged_attention_decode_shared_prefix",
    "paged_attention_decode_shared_prefix_workspace_bytes", "pkv_validate_shared_prefix",
    "pkv_read_probe_blocks", "pkv_read_probe", "paged_attention_decode_shared_prefix_append",
    "paged_attention_decode_noalloc", "pkv_noalloc_scratch_bytes", "pkv_decode_order",
    "pkv_validate_seq_order", "pkv_tile_gather_probe",
)
ABI_VERSION = 10
DECODE_DEFER_MERGE = 1
DECODE_STREAM_KV = 2


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class PkvTensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
        ("scale", ctypes.c_float),
    ]


class PkvDecodeOpts(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("partition_size", ctypes.c_int32),
        ("waves_per_group", ctypes.c_int32),
        ("num_workers", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("flags", ctypes.c_int32),
        ("seq_order", ctypes.c_void_p),
    ]


class PkvPrefillOpts(ctypes.Structure):
    _fields_ = [("rows_per_wave", ctypes.c_int32)]


DECODE_MODES = {"single": 0, "partitioned": 1, "balanced": 2, "auto": 3}


def decode_opts(mode: str | None = None, partition_size: int = 0, waves_per_group: int = 0,
                num_workers: int = 0, defer_merge: bool = False,
                stream_kv: bool = False, seq_order=None) -> PkvDecodeOpts:
    """Options struct; mode None means "partitioned" if partition_size > 0, else "auto".

    stream_kv: the batch shares no block between sequences (every refcount 1,
    see BlockPool.shares_blocks), so the pool reads may stream past the caches
    (PKV_DECODE_STREAM_KV); results are bit-identical either way.
    seq_order: None, or a contiguous int32 GPU tensor [S], a permutation of
    the sequences giving the order in which the single pass starts them
    (decode_order: longest first); results are bit-identical either way."""
    if mode is None:
        mode = "partitioned" if partition_size > 0 else "auto"
    o = PkvDecodeOpts()
    o.mode = DECODE_MODES[mode]
    o.partition_size = int(partition_size)
    o.waves_per_group = int(waves_per_group)
    o.num_workers = int(num_workers)
    o.flags = (DECODE_DEFER_MERGE if defer_merge else 0) | (DECODE_STREAM_KV if stream_kv else 0)
    if seq_order is not None:
        if (seq_order.device.type != "cuda" or seq_order.dim() != 1 or not seq_order.is_contiguous()
                or str(seq_order.dtype) != "torch.int32"):
            raise ValueError("seq_order must be a contiguous int32 GPU tensor [num_seqs]")
        o.seq_order = seq_order.data_ptr() if seq_order.numel() else None
    return o


def decode_order(context_lens: np.ndarray) -> np.ndarray:
    """Longest-context-first order of a batch (host lengths) for seq_order:
    element i is the sequence with the i-th longest context, ties in index
    order (the library's pkv_decode_order)."""
    n = np.ascontiguousarray(context_lens, dtype=np.int32)
    order = np.empty(n.size, np.int32)
    _check(load().pkv_decode_order(n.ctypes.data_as(ctypes.c_void_p), n.size,
                                   order.ctypes.data_as(ctypes.c_void_p)))
    return order


def validate_seq_order(seq_order: np.ndarray, num_seqs: int) -> None:
    """Host check that seq_order is a permutation of 0..num_seqs-1; raises PagedKVError."""
    o = np.ascontiguousarray(seq_order, dtype=np.int32)
    if o.shape != (num_seqs,):
        raise ValueError(f"seq_order must have shape ({num_seqs},)")
    _check(load().pkv_validate_seq_order(o.ctypes.data_as(ctypes.c_void_p), num_seqs))


_lib = None


def load():
    """Load libpagedkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_135_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    T = ctypes.POINTER(PkvTensor)
    lib.pkv_abi_version.restype = ctypes.c_int32
    if lib.pkv_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {lib.pkv_abi_version()}, this binding "
                           f"expects {ABI_VERSION}: rebuild it")
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_read_probe_blocks.restype = ctypes.c_int32
    lib.pkv_read_probe.argtypes = [P, ctypes.c_size_t, P, P]
    lib.pkv_read_probe.restype = ctypes.c_int
    lib.paged_kv_write.argtypes = [T, T, T, T, T, P]
    lib.paged_kv_write.restype = ctypes.c_int
    lib.paged_attention_decode.argtypes = [T, T, T, T, T, T, ctypes.c_float, ctypes.c_int32,
                                           ctypes.POINTER(PkvDecodeOpts), P]
    lib.paged_attention_decode.restype = ctypes.c_int
    lib.paged_attention_decode_merge.argtypes = lib.paged_attention_decode.argtypes
    lib.paged_attention_decode_merge.restype = ctypes.c_int
    lib.paged_attention_decode_noalloc.argtypes = lib.paged_attention_decode.argtypes
    lib.paged_attention_decode_noalloc.restype = ctypes.c_int
    lib.pkv_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.paged_attention_decode_append.argtypes = [T, T, T, T, T, T, T, T, T, ctypes.c_float,
                                                  ctypes.c_int32, ctypes.POINTER(PkvDecodeOpts), P]
    lib.paged_attention_decode_append.restype = ctypes.c_int
    lib.pkv_validate_append_slots.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int64, ctypes.c_int32]
    lib.pkv_validate_append_slots.restype = ctypes.c_int
    lib.paged_attention_prefill.argtypes = [T, T, T, T, T, T, T, ctypes.c_int32, ctypes.c_float,
                                            ctypes.c_int32, ctypes.POINTER(PkvPrefillOpts), P]
    lib.paged_attention_prefill.restype = ctypes.c_int
    lib.pkv_validate_prefill_inputs.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_int32]
    lib.pkv_validate_prefill_inputs.restype = ctypes.c_int
    lib.paged_attention_decode_workspace_bytes.argtypes = [ctypes.c_int32] * 6 + [
        ctypes.POINTER(PkvDecodeOpts)]
    lib.paged_attention_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.pkv_validate_slots.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    lib.pkv_validate_slots.restype = ctypes.c_int
    lib.pkv_validate_decode_inputs.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int64, ctypes.c_int32]
    lib.pkv_validate_decode_inputs.restype = ctypes.c_int
    lib.paged_kv_copy_blocks.argtypes = [T, T, T, P]
    lib.paged_kv_copy_blocks.restype = ctypes.c_int
    lib.pkv_validate_block_pairs.argtypes = [P, ctypes.c_int64, ctypes.c_int64]
    lib.pkv_validate_block_pairs.restype = ctypes.c_int
    lib.paged_kv_gather_blocks.argtypes = [T, T, T, T, T, P]
    lib.paged_kv_gather_blocks.restype = ctypes.c_int
    lib.paged_kv_scatter_blocks.argtypes = [T, T, T, T, T, P]
    lib.paged_kv_scatter_blocks.restype = ctypes.c_int
    lib.pkv_validate_block_ids.argtypes = [P, ctypes.c_int64, ctypes.c_int64]
    lib.pkv_validate_block_ids.restype = ctypes.c_int
    lib.pkv_tile_gather_probe.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                          ctypes.c_int32, P, P]
    lib.pkv_tile_gather_probe.restype = ctypes.c_int
    lib.pkv_decode_order.argtypes = [P, ctypes.c_int32, P]
    lib.pkv_decode_order.restype = ctypes.c_int
    lib.pkv_validate_seq_order.argtypes = [P, ctypes.c_int32]
    lib.pkv_validate_seq_order.restype = ctypes.c_int
    lib.paged_attention_decode_shared_prefix.argtypes = [T, T, T, T, T, T, ctypes.c_int32,
                                                         ctypes.c_float, ctypes.c_int32,
                                                         ctypes.POINTER(PkvDecodeOpts), P]
    lib.paged_attention_decode_shared_prefix.restype = ctypes.c_int
    lib.paged_attention_decode_shared_prefix_append.argtypes = [T] * 9 + [
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.POINTER(PkvDecodeOpts), P]
    lib.paged_attention_decode_shared_prefix_append.restype = ctypes.c_int
    lib.paged_attention_decode_shared_prefix_workspace_bytes.argtypes = [ctypes.c_int32] * 7 + [
        ctypes.POINTER(PkvDecodeOpts)]
    lib.paged_attention_decode_shared_prefix_workspace_bytes.restype = ctypes.c_size_t
    lib.pkv_validate_shared_prefix.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    lib.pkv_validate_shared_prefix.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load().pkv_last_error()
        raise PagedKVError(status, msg.decode() if msg else "")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PKV_FP8_E4M3
    if t.dtype == torch.int32:
        return PKV_I32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def describe(t, scale: float = 1.0) -> PkvTensor:
    """pkv_tensor descriptor of a torch tensor (no copy)."""
    if t.dim() > 4:
        raise ValueError("at most 4 dims")
    d = PkvTensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    d.scale = float(scale)
    return d


def _stream(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _same_device(*ts):
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError("all tensors must live on the same GPU")


def paged_kv_write(k, v, slot_mapping, key_cache, value_cache, *, k_scale: float = 1.0,
                   v_scale: float = 1.0, stream=None) -> None:
    """Write tokens' K/V [T, Hkv, D] into the pools [NB, Hkv, bs, D] at their
    slots (see include/pagedkv.h).  k_scale/v_scale apply to E4M3 pools."""
    _same_device(k, v, slot_mapping, key_cache, value_cache)
    dk, dv, ds = describe(k), describe(v), describe(slot_mapping)
    dkc, dvc = describe(key_cache, k_scale), describe(value_cache, v_scale)
    _check(load().paged_kv_write(ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(ds),
                                 ctypes.byref(dkc), ctypes.byref(dvc), _stream(k, stream)))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_blocks_per_seq: int, block_size: int, mode: str | None = None,
                           partition_size: int = 0, num_workers: int = 0) -> int:
    o = decode_opts(mode, partition_size, 0, num_workers)
    return int(load().paged_attention_decode_workspace_bytes(
        num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq, block_size,
        ctypes.byref(o)))


def _workspace_for(opts: PkvDecodeOpts, q, key_cache, block_tables, block_size, workspace,
                   prefix_len: int = 0):
    import torch
    args = (q.shape[0], q.shape[1], key_cache.shape[1], q.shape[2], block_tables.shape[1],
            block_size)
    if prefix_len:
        need = int(load().paged_attention_decode_shared_prefix_workspace_bytes(
            *args, int(prefix_len), ctypes.byref(opts)))
    else:
        need = int(load().paged_attention_decode_workspace_bytes(*args, ctypes.byref(opts)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    return workspace


def paged_attention_decode(out, q, key_cache, value_cache, block_tables, context_lens,
                           scale: float, block_size: int, *, k_scale: float = 1.0,
                           v_scale: float = 1.0, mode: str | None = None, partition_size: int = 0,
                           waves_per_group: int = 0, num_workers: int = 0, workspace=None,
                           stream_kv: bool = False, seq_order=None, stream=None):
    """Decode attention over the paged pools into ``out`` [S, Hq, D].

    mode: "single", "partitioned" (needs partition_size), "balanced" or "auto";
    None picks "partitioned" when partition_size > 0, else "auto".  The split
    modes need a workspace (a uint8 device tensor of at least
    decode_workspace_bytes(...)); it is allocated here when not given.
    stream_kv, seq_order: see decode_opts."""
    _same_device(out, q, key_cache, value_cache, block_tables, context_lens)
    opts = decode_opts(mode, partition_size, waves_per_group, num_workers, stream_kv=stream_kv,
                       seq_order=seq_order)
    ws = _workspace_for(opts, q, key_cache, block_tables, block_size, workspace)
    dout, dq = describe(out), describe(q)
    dkc, dvc = describe(key_cache, k_scale), describe(value_cache, v_scale)
    dt, dl = describe(block_tables), describe(context_lens)
    _check(load().paged_attention_decode(
        ctypes.byref(dout), ctypes.byref(dq), ctypes.byref(dkc), ctypes.byref(dvc),
        ctypes.byref(dt), ctypes.byref(dl), float(scale), int(block_size), ctypes.byref(opts),
        _stream(q, stream)))
    if ws is not None and workspace is None and stream is not None:
        ws.record_stream(stream)
    return out


def paged_attention_decode_noalloc(out, q, key_cache, value_cache, block_tables, context_lens,
                                   scale: float, block_size: int, *, k_scale: float = 1.0,
                                   v_scale: float = 1.0, mode: str | None = None,
                                   partition_size: int = 0, waves_per_group: int = 0,
                                   num_workers: int = 0, stream_kv: bool = False, seq_order=None,
                                   stream=None):
    """paged_attention_decode with the library's fixed device scratch as the
    split workspace: allocates nothing (see include/pagedkv.h; calls that
    overlap on one GPU race)."""
    _same_device(out, q, key_cache, value_cache, block_tables, context_lens)
    opts = decode_opts(mode, partition_size, waves_per_group, num_workers, stream_kv=stream_kv,
                       seq_order=seq_order)
    dout, dq = describe(out), describe(q)
    dkc, dvc = describe(key_cache, k_scale), describe(value_cache, v_scale)
    dt, dl = describe(block_tables), describe(context_lens)
    _check(load().paged_attention_decode_noalloc(
        ctypes.byref(dout), ctypes.byref(dq), ctypes.byref(dkc), ctypes.byref(dvc),
        ctypes.byref(dt), ctypes.byref(dl), float(scale), int(block_size), ctypes.byref(opts),
        _stream(q, stream)))
    return out


def noalloc_scratch_bytes() -> int:
    """Bytes of device scratch behind paged_attention_decode_noalloc (per GPU)."""
    return int(load().pkv_noalloc_scratch_bytes())


def paged_attention_decode_append(out, q, k, v, slot_mapping, key_cache, value_cache,
                                  block_tables, context_lens, scale: float, block_size: int, *,
                                  k_scale: float = 1.0, v_scale: float = 1.0,
                                  mode: str | None = None, partition_size: int = 0,
                                  waves_per_group: int = 0, num_workers: int = 0, workspace=None,
                                  stream_kv: bool = False, seq_order=None, stream=None):
    """One decode step in one call: write each sequence's new token (k, v
    [S, Hkv, D] at slot_mapping [S]) and attend (see include/pagedkv.h).
    Equal to paged_kv_write followed by paged_attention_decode when every
    slot is position context_lens[s]-1 of its own sequence."""
    _same_device(out, q, k, v, slot_mapping, key_cache, value_cache, block_tables, context_lens)
    opts = decode_opts(mode, partition_size, waves_per_group, num_workers, stream_kv=stream_kv,
                       seq_order=seq_order)
    ws = _workspace_for(opts, q, key_cache, block_tables, block_size, workspace)
    d = [describe(out), describe(q), describe(k), describe(v), describe(slot_mapping),
         describe(key_cache, k_scale), describe(value_cache, v_scale), describe(block_tables),
         describe(context_lens)]
    _check(load().paged_attention_decode_append(*[ctypes.byref(x) for x in d], float(scale),
                                                int(block_size), ctypes.byref(opts),
                                                _stream(q, stream)))
    if ws is not None and workspace is None and stream is not None:
        ws.record_stream(stream)
    return out


def paged_attention_prefill(out, q, key_cache, value_cache, block_tables, context_lens,
                            query_start_loc, max_query_len: int, scale: float, block_size: int, *,
                            k_scale: float = 1.0, v_scale: float = 1.0, rows_per_wave: int = 0,
                            stream=None):
    """Chunked-prefill attention into ``out`` [T, Hq, D]: sequence s's queries
    are rows query_start_loc[s] .. query_start_loc[s+1]-1 of q, at the last
    positions of its context, attending causally (see include/pagedkv.h)."""
    _same_device(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc)
    o = PkvPrefillOpts()
    o.rows_per_wave = int(rows_per_wave)
    d = [describe(out), describe(q), describe(key_cache, k_scale), describe(value_cache, v_scale),
         describe(block_tables), describe(context_lens), describe(query_start_loc)]
    _check(load().paged_attention_prefill(*[ctypes.byref(x) for x in d], int(max_query_len),
                                          float(scale), int(block_size), ctypes.byref(o),
                                          _stream(q, stream)))
    return out


def paged_attention_decode_shared_prefix(out, q, key_cache, value_cache, block_tables,
                                         context_lens, prefix_len: int, scale: float,
                                         block_size: int, *, k_scale: float = 1.0,
                                         v_scale: float = 1.0, num_workers: int = 0,
                                         workspace=None, stream_kv: bool = False, stream=None):
    """Decode for sequences whose first ``prefix_len`` tokens are the same shared
    blocks: the prefix part once for all sequences, the tails through the
    balanced split, merged (see include/pagedkv.h).  stream_kv (see
    decode_opts) applies to the tails' reads: the tails must share no block."""
    _same_device(out, q, key_cache, value_cache, block_tables, context_lens)
    opts = decode_opts("auto", 0, 0, num_workers, stream_kv=stream_kv)
    ws = _workspace_for(opts, q, key_cache, block_tables, block_size, workspace, prefix_len)
    d = [describe(out), describe(q), describe(key_cache, k_scale), describe(value_cache, v_scale),
         describe(block_tables), describe(context_lens)]
    _check(load().paged_attention_decode_shared_prefix(
        *[ctypes.byref(x) for x in d], int(prefix_len), float(scale), int(block_size),
        ctypes.byref(opts), _stream(q, stream)))
    if ws is not None and workspace is None and stream is not None:
        ws.record_stream(stream)
    return out


def paged_attention_decode_shared_prefix_append(out, q, k, v, slot_mapping, key_cache,
                                                value_cache, block_tables, context_lens,
                                                prefix_len: int, scale: float, block_size: int, *,
                                                k_scale: float = 1.0, v_scale: float = 1.0,
                                                num_workers: int = 0, workspace=None,
                                                stream_kv: bool = False, stream=None):
    """One shared-prefix decode step in one call: write each sequence's new
    token (k, v [S, Hkv, D] at slot_mapping [S], inside its own tail) and
    attend as paged_attention_decode_shared_prefix (see include/pagedkv.h).
    Every context_lens[s] must exceed prefix_len."""
    _same_device(out, q, k, v, slot_mapping, key_cache, value_cache, block_tables, context_lens)
    opts = decode_opts("auto", 0, 0, num_workers, stream_kv=stream_kv)
    ws = _workspace_for(opts, q, key_cache, block_tables, block_size, workspace, prefix_len)
    d = [describe(out), describe(q), describe(k), describe(v), describe(slot_mapping),
         describe(key_cache, k_scale), describe(value_cache, v_scale), describe(block_tables),
         describe(context_lens)]
    _check(load().paged_attention_decode_shared_prefix_append(
        *[ctypes.byref(x) for x in d], int(prefix_len), float(scale), int(block_size),
        ctypes.byref(opts), _stream(q, stream)))
    if ws is not None and workspace is None and stream is not None:
        ws.record_stream(stream)
    return out


def tables_share_blocks(block_tables: np.ndarray, context_lens: np.ndarray, block_size: int,
                        skip_blocks: int = 0) -> bool:
    """True if a physical block is listed by two of the sequences (host tables),
    counting each sequence's blocks from column skip_blocks up to its length.
    False means a decode reads every block once and may pass stream_kv=True."""
    t = np.asarray(block_tables)
    n = -(-np.asarray(context_lens, dtype=np.int64) // int(block_size))
    ids = np.concatenate([t[s, skip_blocks:max(skip_blocks, int(n[s]))] for s in range(t.shape[0])]
                         + [np.zeros(0, t.dtype)])
    return np.unique(ids).size != ids.size


def validate_shared_prefix(block_tables: np.ndarray, context_lens: np.ndarray, num_blocks: int,
                           block_size: int, prefix_len: int) -> None:
    """Host check of a shared-prefix decode's tables; raises PagedKVError."""
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    n = np.ascontiguousarray(context_lens, dtype=np.int32)
    if t.ndim != 2 or n.shape != (t.shape[0],):
        raise ValueError("block_tables must be [S, max_blocks], context_lens [S]")
    _check(load().pkv_validate_shared_prefix(t.ctypes.data_as(ctypes.c_void_p),
                                             n.ctypes.data_as(ctypes.c_void_p), t.shape[0],
                                             t.shape[1], num_blocks, block_size, prefix_len))


def paged_kv_copy_blocks(key_cache, value_cache, block_pairs, *, stream=None) -> None:
    """Copy-on-write: for each int32 row (src, dst) of ``block_pairs`` [P, 2],
    block dst of both pools becomes a copy of block src (see include/pagedkv.h)."""
    _same_device(key_cache, value_cache, block_pairs)
    dk, dv, dp = describe(key_cache), describe(value_cache), describe(block_pairs)
    _check(load().paged_kv_copy_blocks(ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(dp),
                                       _stream(key_cache, stream)))


def _stream_of(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device if t.device.type == "cuda" else None)
    return ctypes.c_void_p(stream.cuda_stream)


def paged_kv_gather_blocks(key_cache, value_cache, block_ids, out_k, out_v, *,
                           stream=None) -> None:
    """Swap-out: staging slot i of out_k/out_v ([n, Hkv, bs, D], device memory)
    receives block block_ids[i] of the pools."""
    _same_device(key_cache, value_cache, block_ids, out_k, out_v)
    d = [describe(key_cache), describe(value_cache), describe(block_ids), describe(out_k),
         describe(out_v)]
    _check(load().paged_kv_gather_blocks(*[ctypes.byref(x) for x in d],
                                         _stream_of(key_cache, stream)))


def paged_kv_scatter_blocks(in_k, in_v, block_ids, key_cache, value_cache, *,
                            stream=None) -> None:
    """Swap-in: block block_ids[i] of the pools receives staging slot i of
    in_k/in_v ([n, Hkv, bs, D], device memory)."""
    _same_device(key_cache, value_cache, block_ids, in_k, in_v)
    d = [describe(in_k), describe(in_v), describe(block_ids), describe(key_cache),
         describe(value_cache)]
    _check(load().paged_kv_scatter_blocks(*[ctypes.byref(x) for x in d],
                                          _stream_of(key_cache, stream)))


def read_probe(buf, sink=None, *, stream=None):
    """Measurement support: one streaming pass over the device tensor ``buf``
    (the attainable read rate the decode byte rates are set against).  Returns
    the sink, a uint32 device tensor whose XOR is the XOR of buf's 32-bit words."""
    import torch
    lib = load()
    if sink is None:
        sink = torch.empty(lib.pkv_read_probe_blocks(), dtype=torch.int32, device=buf.device)
    s = stream if stream is not None else torch.cuda.current_stream(buf.device)
    _check(lib.pkv_read_probe(ctypes.c_void_p(buf.data_ptr()),
                              buf.numel() * buf.element_size(),
                              ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(s.cuda_stream)))
    return sink


def tile_gather_probe(key_cache, value_cache, tile_rows, workers: int, mode: int, sink=None, *,
                      stream=None):
    """Measurement support: the decode's tile gather alone over a bf16,
    head-dim-128 pool (see include/pagedkv.h, pkv_tile_gather_probe): mode 0
    loads the MFMA operands straight to registers, mode 1 stages each tile
    through LDS first.  tile_rows: int32 GPU tensor of first pool rows.
    Returns the sink (int32 device tensor, one word per workgroup)."""
    import torch
    if key_cache.dtype != torch.bfloat16 or key_cache.shape[-1] != 128:
        raise ValueError("the gather probe reads bf16 pools of head dim 128")
    if sink is None:
        sink = torch.empty((workers + 3) // 4, dtype=torch.int32, device=key_cache.device)
    num_rows = key_cache.numel() // 128
    s = stream if stream is not None else torch.cuda.current_stream(key_cache.device)
    _check(load().pkv_tile_gather_probe(
        ctypes.c_void_p(key_cache.data_ptr()), ctypes.c_void_p(value_cache.data_ptr()),
        ctypes.c_void_p(tile_rows.data_ptr()), tile_rows.numel(), num_rows, int(workers), int(mode),
        ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(s.cuda_stream)))
    return sink


def swap_out_to_host(key_cache, value_cache, block_ids, host_k, host_v, *, staging=None,
                     stream=None):
    """Swap-out to host memory: gather the blocks into a device staging buffer
    (the kernel), then copy it to host_k/host_v (pinned CPU tensors,
    [n, Hkv, bs, D]) with the copy engine.  Returns the staging pair, which
    must stay alive until the copies are done."""
    import torch
    n = block_ids.shape[0]
    shape = (n,) + tuple(key_cache.shape[1:])
    if staging is None:
        staging = (torch.empty(shape, dtype=key_cache.dtype, device=key_cache.device),
                   torch.empty(shape, dtype=key_cache.dtype, device=key_cache.device))
    paged_kv_gather_blocks(key_cache, value_cache, block_ids, staging[0], staging[1], stream=stream)
    s = stream if stream is not None else torch.cuda.current_stream(key_cache.device)
    with torch.cuda.stream(s):
        host_k.copy_(staging[0], non_blocking=True)
        host_v.copy_(staging[1], non_blocking=True)
    return staging


def swap_in_from_host(host_k, host_v, block_ids, key_cache, value_cache, *, staging=None,
                      stream=None):
    """Swap-in from host memory: copy host_k/host_v into a device staging buffer
    with the copy engine, then scatter it into the pools' blocks (the kernel)."""
    import torch
    if staging is None:
        staging = (torch.empty(host_k.shape, dtype=key_cache.dtype, device=key_cache.device),
                   torch.empty(host_v.shape, dtype=key_cache.dtype, device=key_cache.device))
    s = stream if stream is not None else torch.cuda.current_stream(key_cache.device)
    with torch.cuda.stream(s):
        staging[0].copy_(host_k, non_blocking=True)
        staging[1].copy_(host_v, non_blocking=True)
    paged_kv_scatter_blocks(staging[0], staging[1], block_ids, key_cache, value_cache, stream=stream)
    return staging


def validate_block_ids(block_ids: np.ndarray, num_blocks: int) -> None:
    """Host check of swap block ids (range, no repeats); raises PagedKVError."""
    b = np.ascontiguousarray(block_ids, dtype=np.int32)
    _check(load().pkv_validate_block_ids(b.ctypes.data_as(ctypes.c_void_p), b.size, num_blocks))


def validate_block_pairs(pairs: np.ndarray, num_blocks: int) -> None:
    """Host check of copy-on-write pairs (range, distinct destinations, no
    destination used as a source); raises PagedKVError."""
    p = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    _check(load().pkv_validate_block_pairs(p.ctypes.data_as(ctypes.c_void_p), p.shape[0],
                                           num_blocks))


def validate_slots(slots: np.ndarray, num_blocks: int, block_size: int) -> None:
    """Host check of a slot mapping (range, no repeats); raises PagedKVError."""
    s = np.ascontiguousarray(slots, dtype=np.int32)
    _check(load().pkv_validate_slots(s.ctypes.data_as(ctypes.c_void_p), s.size, num_blocks,
                                     block_size))


def validate_decode_inputs(block_tables: np.ndarray, context_lens: np.ndarray, num_blocks: int,
                           block_size: int) -> None:
    """Host check of tables and lengths against the pool; raises PagedKVError."""
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    n = np.ascontiguousarray(context_lens, dtype=np.int32)
    if t.ndim != 2 or n.shape != (t.shape[0],):
        raise ValueError("block_tables must be [S, max_blocks], context_lens [S]")
    _check(load().pkv_validate_decode_inputs(t.ctypes.data_as(ctypes.c_void_p),
                                             n.ctypes.data_as(ctypes.c_void_p), t.shape[0],
                                             t.shape[1], num_blocks, block_size))


def validate_append_slots(slots: np.ndarray, block_tables: np.ndarray, context_lens: np.ndarray,
                          num_blocks: int, block_size: int) -> None:
    """Host check of an append call's slots: each is -1 or position len-1 of its
    own sequence, in a block no other sequence reads; raises PagedKVError."""
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    n = np.ascontiguousarray(context_lens, dtype=np.int32)
    if t.ndim != 2 or n.shape != (t.shape[0],) or sl.shape != (t.shape[0],):
        raise ValueError("block_tables must be [S, max_blocks], context_lens and slots [S]")
    _check(load().pkv_validate_append_slots(sl.ctypes.data_as(ctypes.c_void_p),
                                            t.ctypes.data_as(ctypes.c_void_p),
                                            n.ctypes.data_as(ctypes.c_void_p), t.shape[0],
                                            t.shape[1], num_blocks, block_size))


def validate_prefill_inputs(query_start_loc: np.ndarray, block_tables: np.ndarray,
                            context_lens: np.ndarray, num_blocks: int, block_size: int,
                            num_query_rows: int, max_query_len: int) -> None:
    """Host check of a chunked-prefill call's query layout, tables and lengths;
    raises PagedKVError."""
    qs = np.ascontiguousarray(query_start_loc, dtype=np.int32)
    t = np.ascontiguousarray(block_tables, dtype=np.int32)
    n = np.ascontiguousarray(context_lens, dtype=np.int32)
    if t.ndim != 2 or n.shape != (t.shape[0],) or qs.shape != (t.shape[0] + 1,):
        raise ValueError("block_tables must be [S, max_blocks], context_lens [S], "
                         "query_start_loc [S + 1]")
    _check(load().pkv_validate_prefill_inputs(qs.ctypes.data_as(ctypes.c_void_p),
                                              t.ctypes.data_as(ctypes.c_void_p),
                                              n.ctypes.data_as(ctypes.c_void_p), t.shape[0],
                                              t.shape[1], num_blocks, block_size, num_query_rows,
                                              max_query_len))


class PrefillLaunch:
    """A chunked-prefill call with its descriptors built once."""

    def __init__(self, out, q, key_cache, value_cache, block_tables, context_lens,
                 query_start_loc, max_query_len: int, scale: float, block_size: int, *,
                 k_scale: float = 1.0, v_scale: float = 1.0, rows_per_wave: int = 0):
        _same_device(out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc)
        self._keep = (out, q, key_cache, value_cache, block_tables, context_lens, query_start_loc)
        self._d = [describe(out), describe(q), describe(key_cache, k_scale),
                   describe(value_cache, v_scale), describe(block_tables), describe(context_lens),
                   describe(query_start_loc)]
        self._refs = [ctypes.byref(d) for d in self._d]
        self._opts = PkvPrefillOpts()
        self._opts.rows_per_wave = int(rows_per_wave)
        self._mql, self._scale, self._bs = int(max_query_len), float(scale), int(block_size)
        self._lib = load()
        self._device = q.device

    def __call__(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self._device)
        _check(self._lib.paged_attention_prefill(*self._refs, self._mql, self._scale, self._bs,
                                                 ctypes.byref(self._opts),
                                                 ctypes.c_void_p(s.cuda_stream)))


class WriteLaunch:
    """A KV write with its descriptors built once (for tight loops and graph
    capture).  Holds references to the tensors; call to launch on the current
    stream (or ``stream``)."""

    def __init__(self, k, v, slot_mapping, key_cache, value_cache, *, k_scale: float = 1.0,
                 v_scale: float = 1.0):
        _same_device(k, v, slot_mapping, key_cache, value_cache)
        self._keep = (k, v, slot_mapping, key_cache, value_cache)
        self._d = [describe(k), describe(v), describe(slot_mapping), describe(key_cache, k_scale),
                   describe(value_cache, v_scale)]
        self._refs = [ctypes.byref(d) for d in self._d]
        self._lib = load()
        self._device = k.device

    def __call__(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self._device)
        _check(self._lib.paged_kv_write(*self._refs, ctypes.c_void_p(s.cuda_stream)))


class DecodeLaunch:
    """A decode call with descriptors, options and workspace prepared once.

    append=(k, v, slot_mapping) makes it the one-call decode step
    (paged_attention_decode_append; with prefix_len,
    paged_attention_decode_shared_prefix_append).  defer_merge=True launches only the
    streaming kernel; call merge() next on the same stream.  stream_kv: see
    decode_opts."""

    def __init__(self, out, q, key_cache, value_cache, block_tables, context_lens, scale: float,
                 block_size: int, *, k_scale: float = 1.0, v_scale: float = 1.0,
                 mode: str | None = None, partition_size: int = 0, waves_per_group: int = 0,
                 num_workers: int = 0, workspace=None, append=None, defer_merge: bool = False,
                 prefix_len: int = 0, stream_kv: bool = False, seq_order=None):
        _same_device(out, q, key_cache, value_cache, block_tables, context_lens)
        if prefix_len and defer_merge:
            raise ValueError("a shared-prefix decode takes no deferred merge")
        if prefix_len and mode is None:
            mode = "auto"
        self._opts = decode_opts(mode, partition_size, waves_per_group, num_workers, defer_merge,
                                 stream_kv, seq_order)
        self._merge_opts = decode_opts(mode, partition_size, waves_per_group, num_workers)
        self.workspace = _workspace_for(self._opts, q, key_cache, block_tables, block_size,
                                        workspace, prefix_len)
        _workspace_for(self._merge_opts, q, key_cache, block_tables, block_size, self.workspace,
                       prefix_len)
        self._prefix = int(prefix_len)
        self._keep = (out, q, key_cache, value_cache, block_tables, context_lens, append, seq_order)
        self._d = [describe(out), describe(q), describe(key_cache, k_scale),
                   describe(value_cache, v_scale), describe(block_tables), describe(context_lens)]
        self._refs = [ctypes.byref(d) for d in self._d]
        self._app_refs = None
        if append is not None:
            k, v, slots = append
            _same_device(q, k, v, slots)
            self._da = [describe(k), describe(v), describe(slots)]
            r = self._refs
            self._app_refs = [r[0], r[1]] + [ctypes.byref(d) for d in self._da] + r[2:]
        self._scale = float(scale)
        self._bs = int(block_size)
        self._lib = load()
        self._device = q.device

    def _s(self, stream):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream(self._device)
        return ctypes.c_void_p(s.cuda_stream)

    def __call__(self, stream=None):
        if self._prefix and self._app_refs is not None:
            _check(self._lib.paged_attention_decode_shared_prefix_append(
                *self._app_refs, self._prefix, self._scale, self._bs, ctypes.byref(self._opts),
                self._s(stream)))
        elif self._prefix:
            _check(self._lib.paged_attention_decode_shared_prefix(
                *self._refs, self._prefix, self._scale, self._bs, ctypes.byref(self._opts),
                self._s(stream)))
        elif self._app_refs is not None:
            _check(self._lib.paged_attention_decode_append(*self._app_refs, self._scale, self._bs,
                                                           ctypes.byref(self._opts),
                                                           self._s(stream)))
        else:
            _check(self._lib.paged_attention_decode(*self._refs, self._scale, self._bs,
                                                    ctypes.byref(self._opts), self._s(stream)))

    def merge(self, stream=None):
        """Second half of a deferred-merge call (no-op for modes without a merge)."""
        _check(self._lib.paged_attention_decode_merge(*self._refs, self._scale, self._bs,
                                                      ctypes.byref(self._merge_opts),
                                                      self._s(stream)))
