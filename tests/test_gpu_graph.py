"""Calls replayed from a captured HIP graph give, on every replay, the same bits
as the eager call on the same inputs (the library queues only kernels on the
given stream: no allocation, no memset, no synchronisation): the decode step in
each mode, the shared-prefix call (with and without the step's write folded in)
and chunked prefill."""
import math

import numpy as np
import pytest

import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
torch = gu.torch
import paged_kv_cache_135_amd as pkv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


@pytest.mark.parametrize("mode", ["balanced", "partitioned", "single"])
def test_graph_replays_match_eager(mode):
    case = workloads.build_case("graph", seed=61, context_lens=[5, 300, 1000, 77, 2048, 16],
                                num_q_heads=28, num_kv_heads=4, head_dim=128, block_size=16,
                                cache_dtype="bf16", std=0.5, scale=1.0 / math.sqrt(128))
    g = gu.GpuCase(case)
    kn, vn, sl = gu.dev(case.k_new), gu.dev(case.v_new), gu.dev(case.slot_mapping)
    out = torch.empty_like(g.q)
    kw = dict(mode=mode, partition_size=256 if mode == "partitioned" else 0)
    launch = pkv.DecodeLaunch(out, g.q, g.kc, g.vc, g.tables, g.lens, case.scale, case.block_size,
                              append=(kn, vn, sl), **kw)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        launch()  # warm up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        launch()
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for rep in range(4):
        qn = workloads.bf16_bits_from_f32(rng.standard_normal(case.q.shape).astype(np.float32) * 0.5)
        g.q.copy_(gu.dev(qn))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = gu.host(out).copy()
        launch()  # eager, same inputs
        torch.cuda.synchronize()
        assert np.array_equal(got, gu.host(out)), f"replay {rep}"


def _replays_match(stream, launch, refresh, out):
    """Capture `launch` on `stream`, then replay it 4 times; before each replay
    `refresh` writes new inputs eagerly, and the replay's output must equal the
    eager call's on the same inputs bit for bit."""
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        launch()  # warm up on the capture stream
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        launch()
    torch.cuda.synchronize()
    for rep in range(4):
        refresh(rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = gu.host(out).copy()
        launch()
        torch.cuda.synchronize()
        assert np.array_equal(got, gu.host(out)), f"replay {rep}"


@pytest.mark.parametrize("append", [False, True])
def test_shared_prefix_graph_replays_match_eager(append):
    """The shared-prefix call's three kernels (prefix, tails, merge) in one graph."""
    case = workloads.build_case("graph_prefix", seed=62, context_lens=[70, 300, 65, 129, 1000],
                                num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                                cache_dtype="bf16", std=0.5, scale=1.0 / math.sqrt(128),
                                shared_prefix_blocks=4)
    g = gu.GpuCase(case)
    g.fill_and_step_writes()
    out = torch.empty_like(g.q)
    app = (gu.dev(case.k_new), gu.dev(case.v_new), gu.dev(case.slot_mapping)) if append else None
    launch = pkv.DecodeLaunch(out, g.q, g.kc, g.vc, g.tables, g.lens, case.scale, case.block_size,
                              prefix_len=4 * case.block_size, append=app)
    rng = np.random.default_rng(6)

    def refresh(rep):
        qn = workloads.bf16_bits_from_f32(rng.standard_normal(case.q.shape).astype(np.float32) * 0.5)
        g.q.copy_(gu.dev(qn))

    _replays_match(torch.cuda.Stream(), launch, refresh, out)


def test_prefill_graph_replays_match_eager():
    case = workloads.build_prefill_case("graph_prefill", seed=63, prefix_lens=[0, 100, 37],
                                        chunk_lens=[40, 77, 200], num_q_heads=28, num_kv_heads=4,
                                        head_dim=128, block_size=16, cache_dtype="bf16", std=0.5,
                                        scale=1.0 / math.sqrt(128))
    g = gu.GpuCase(case)
    g.fill_and_step_writes()
    qs = gu.dev(case.query_start)
    mql = int(np.diff(case.query_start).max())
    out = torch.empty_like(g.q)

    def launch():
        pkv.paged_attention_prefill(out, g.q, g.kc, g.vc, g.tables, g.lens, qs, mql, case.scale,
                                    case.block_size)

    rng = np.random.default_rng(7)

    def refresh(rep):
        qn = workloads.bf16_bits_from_f32(rng.standard_normal(case.q.shape).astype(np.float32) * 0.5)
        g.q.copy_(gu.dev(qn))

    _replays_match(torch.cuda.Stream(), launch, refresh, out)
