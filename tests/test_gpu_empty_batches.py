"""Empty batches through every attention and write entry point: no sequences
at all, and sequences that all have empty contexts.

Empty tensors are made both from numpy arrays and by torch directly: their
reported strides differ (torch gives stride 0 for some), and an empty tensor
has no layout to check.  Nothing may be written to the pools, and every output
row of an empty context is zero."""
import numpy as np
import pytest

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
torch = gu.torch
import paged_kv_cache_135_amd as pkv  # noqa: E402

H, G, D, BS, NB = 2, 4, 128, 16, 8
MODES = [None, "single", "partitioned", "balanced"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


def _pools():
    rng = np.random.default_rng(77)
    kc = rng.integers(0, 2**16, size=(NB, H, BS, D), dtype=np.uint16)
    vc = rng.integers(0, 2**16, size=(NB, H, BS, D), dtype=np.uint16)
    return kc, vc, gu.dev(kc), gu.dev(vc)


def _empty(make, shape, npdt):
    if make == "numpy":
        return gu.dev(np.empty(shape, npdt))
    tdt = {np.uint16: torch.bfloat16, np.int32: torch.int32}[npdt]
    return torch.empty(shape, dtype=tdt, device="cuda")


def _unchanged(gk, gv, kc, vc):
    assert np.array_equal(gu.host(gk), kc) and np.array_equal(gu.host(gv), vc)


@pytest.mark.parametrize("make", ["numpy", "torch"])
def test_no_sequences(make):
    kc, vc, gk, gv = _pools()
    q = _empty(make, (0, H * G, D), np.uint16)
    out = _empty(make, (0, H * G, D), np.uint16)
    tables = _empty(make, (0, 3), np.int32)
    lens = _empty(make, (0,), np.int32)
    rows = _empty(make, (0, H, D), np.uint16)
    slots = _empty(make, (0,), np.int32)
    for mode in MODES:
        kw = dict(partition_size=64) if mode == "partitioned" else {}
        pkv.paged_attention_decode(out, q, gk, gv, tables, lens, 0.1, BS, mode=mode, **kw)
        pkv.paged_attention_decode_append(out, q, rows, rows, slots, gk, gv, tables, lens, 0.1, BS,
                                          mode=mode, **kw)
    pkv.paged_attention_decode_noalloc(out, q, gk, gv, tables, lens, 0.1, BS)
    pkv.paged_kv_write(rows, rows, slots, gk, gv)
    qsl = gu.dev(np.zeros(1, np.int32))
    pkv.paged_attention_prefill(out, q, gk, gv, tables, lens, qsl, 0, 0.1, BS)
    torch.cuda.synchronize()
    _unchanged(gk, gv, kc, vc)


@pytest.mark.parametrize("make", ["numpy", "torch"])
def test_every_context_empty(make):
    """Three sequences, none with a token: zero rows in every mode, the pools
    untouched (the append's slots are all -1), and a prefill with no query
    tokens writes nothing."""
    kc, vc, gk, gv = _pools()
    S = 3
    q = gu.dev(np.full((S, H * G, D), 0x3F80, np.uint16))   # ones
    tables = gu.dev(np.arange(S, dtype=np.int32).reshape(S, 1))
    lens = gu.dev(np.zeros(S, np.int32))
    rows = gu.dev(np.full((S, H, D), 0x3F80, np.uint16))
    slots = gu.dev(np.full(S, -1, np.int32))
    pkv.validate_append_slots(np.full(S, -1, np.int32), np.arange(S, dtype=np.int32).reshape(S, 1),
                              np.zeros(S, np.int32), NB, BS)
    for mode in MODES:
        kw = dict(partition_size=64) if mode == "partitioned" else {}
        for append in (False, True):
            out = torch.full_like(q, float("nan"))
            if append:
                pkv.paged_attention_decode_append(out, q, rows, rows, slots, gk, gv, tables, lens,
                                                  0.1, BS, mode=mode, **kw)
            else:
                pkv.paged_attention_decode(out, q, gk, gv, tables, lens, 0.1, BS, mode=mode, **kw)
            torch.cuda.synchronize()
            assert np.all(gu.as_f64(gu.host(out)) == 0.0), (mode, append)
    out = torch.full_like(q, float("nan"))
    pkv.paged_attention_decode_noalloc(out, q, gk, gv, tables, lens, 0.1, BS)
    torch.cuda.synchronize()
    assert np.all(gu.as_f64(gu.host(out)) == 0.0)
    # no query tokens in any sequence
    qsl = gu.dev(np.zeros(S + 1, np.int32))
    empty_q = _empty(make, (0, H * G, D), np.uint16)
    pkv.paged_attention_prefill(_empty(make, (0, H * G, D), np.uint16), empty_q, gk, gv, tables,
                                lens, qsl, 0, 0.1, BS)
    torch.cuda.synchronize()
    _unchanged(gk, gv, kc, vc)
