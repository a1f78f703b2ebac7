"""Shared helpers for the GPU parity tests: move seeded host inputs to the GPU,
run the HIP path through the binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import paged_kv_cache_135_amd as pkv  # noqa: E402
from workloads import PagedCase, bf16_to_f32  # noqa: E402

# Tolerances |gpu - ref| <= ATOL + RTOL * |ref|, ref = fp64 oracle on the stored cache.
# bf16 and E4M3 caches: the stated bar.  f32: derived from fp32 arithmetic: a 64-term fp32
# dot product with sum |q_d k_d| ~ 40 carries ~sqrt(64) * 2^-24 * 40 ~ 2e-5 absolute error,
# which reaches the output as a relative error of the softmax weights.
TOL = {
    "bf16": (2e-3, 1e-2),
    "fp8_e4m3": (2e-3, 5e-2),
    "f32": (2e-5, 2e-4),
}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkv.load()  # raises if the HIP library is missing: never fall back


def dev(a: np.ndarray, device="cuda"):
    """Host array -> device tensor (uint16 carries bf16 bits, uint8 E4M3 codes)."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host(t) -> np.ndarray:
    """Device tensor -> host array with the same bit conventions."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return bf16_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


class GpuCase:
    """A PagedCase resident on the GPU."""

    def __init__(self, case: PagedCase):
        self.case = case
        self.q = dev(case.q)
        self.kc = dev(case.key_cache)
        self.vc = dev(case.value_cache)
        self.tables = dev(case.block_tables)
        self.lens = dev(case.context_lens)
        self.out = torch.empty_like(self.q)

    def write(self, k: np.ndarray, v: np.ndarray, slots: np.ndarray):
        c = self.case
        pkv.paged_kv_write(dev(k), dev(v), dev(slots), self.kc, self.vc, k_scale=c.k_scale,
                           v_scale=c.v_scale)

    def fill_and_step_writes(self):
        c = self.case
        if c.fill_k is not None:
            self.write(c.fill_k, c.fill_v, c.fill_slots)
        if c.k_new is not None:
            self.write(c.k_new, c.v_new, c.slot_mapping)

    def decode(self, partition_size=0, waves=0, out=None, mode=None, workers=0, stream_kv=False,
               seq_order=None):
        """seq_order: None, or a host int32 permutation (copied to the GPU)."""
        c = self.case
        out = self.out if out is None else out
        order = None if seq_order is None else dev(np.ascontiguousarray(seq_order, np.int32))
        pkv.paged_attention_decode(out, self.q, self.kc, self.vc, self.tables, self.lens, c.scale,
                                   c.block_size, k_scale=c.k_scale, v_scale=c.v_scale, mode=mode,
                                   partition_size=partition_size, waves_per_group=waves,
                                   num_workers=workers, stream_kv=stream_kv, seq_order=order)
        return out

    def decode_mode(self, m, stream_kv=False, seq_order=None):
        """m = (mode, partition_size, waves_per_group, num_workers)."""
        mode, part, waves, workers = m
        return self.decode(partition_size=part, waves=waves, mode=mode, workers=workers,
                           stream_kv=stream_kv, seq_order=seq_order)


def oracle_caches(case: PagedCase, tokens_mask=None):
    """The oracle's own pool after this case's writes (never the GPU's)."""
    import oracle
    kc, vc = case.key_cache.copy(), case.value_cache.copy()
    if case.fill_k is not None:
        fk, fv, fs = case.fill_k, case.fill_v, case.fill_slots
        if tokens_mask is not None:
            fk, fv, fs = fk[tokens_mask], fv[tokens_mask], fs[tokens_mask]
        oracle.paged_kv_write(np.ascontiguousarray(fk), np.ascontiguousarray(fv),
                              np.ascontiguousarray(fs), kc, vc, case.k_scale, case.v_scale)
    if case.k_new is not None:
        oracle.paged_kv_write(case.k_new, case.v_new, case.slot_mapping, kc, vc, case.k_scale,
                              case.v_scale)
    return kc, vc


def oracle_decode(case: PagedCase, kc, vc, row_mask=None):
    import oracle
    return oracle.paged_attention_decode(case.q, kc, vc, case.block_tables, case.context_lens,
                                         case.scale, case.block_size, case.k_scale, case.v_scale,
                                         row_mask=row_mask)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", mask=None):
    atol, rtol = TOL[dtype]
    g = as_f64(got)
    if mask is not None:
        g, ref = g[mask], ref[mask]
    err = np.abs(g - ref)
    bound = atol + rtol * np.abs(ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside |err| <= {atol} + {rtol}|ref|; "
            f"first at {tuple(idx)}: got {g[tuple(idx)]!r} ref {ref[tuple(idx)]!r}; "
            f"max err {float(err.max()):.3g}")
    return float(err.max()) if err.size else 0.0
