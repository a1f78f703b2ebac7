#!/usr/bin/env python3
"""Benchmark of the paged KV cache hot path on one MI355X.

One step = one decode step of one attention layer over one batch: the
slot-mapped KV write of every sequence's new token, then paged decode
attention over the whole context (by default the balanced split: equal runs
of tiles per wavefront, each split (sequence, KV head) pair merged by its last
piece in the same launch).
When the step's writes are one new token per sequence at position len-1, the
step is one call (paged_attention_decode_append, the write folded into the
decode launch); otherwise (a prefill chunk into free slots) it is the KV write
followed by the decode.  Inputs are seeded synthetic data resident in HBM
before timing starts.  Steps rotate over several layer pools (each its own K/V
tensors) so a pool is not still resident in the 256 MB last-level cache when
it is read again.

Prints ONE JSON line:
  value  = KV bytes read per step / wall time per step (GB/s, decimal)
  roofline = KV bytes / the streaming decode kernel's duration per launch
             (HIP events around back-to-back launches of it alone) vs 8 TB/s
  call_roofline = the same bytes / the whole call (streaming kernel + merge)
  cpu_baseline = the fp64 oracle timed on this host on the same workload
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MALL_BYTES = 256 * 2 ** 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=400)
    p.add_argument("--workload", default="c2",
                   choices=["c1", "c2", "c3", "c4", "c4bs32", "c5", "c5write", "cow", "p1", "swap"],
                   help="c5write: the E4M3 workload's 4,096-token bf16 chunk quantized into its "
                        "slots, alone; cow: copy-on-write block copies of the Qwen-shaped pool; "
                        "p1: chunked prefill of 8 x 512 tokens over cached prefixes; swap: "
                        "swap-out gather and swap-in scatter of 4,096 blocks (each its own metric)")
    p.add_argument("--shared-prefix", action="store_true",
                   help="c3: decode with paged_attention_decode_shared_prefix (the shared "
                        "prefix computed once for all sequences)")
    p.add_argument("--prefill-rows", type=int, default=0,
                   help="p1: (query, head) rows per wavefront (0 = library default)")
    p.add_argument("--mode", default="auto", choices=["single", "partitioned", "balanced", "auto"])
    p.add_argument("--q-heads", type=int, default=0,
                   help="Qwen-shaped batch with this many query heads over its 4 KV heads "
                        "(same K/V bytes, another group size; 0 = 28)")
    p.add_argument("--seq-order", default="lpt", choices=["lpt", "given"],
                   help="start order of the single pass / partitioned sequences: longest first "
                        "(the library's pkv_decode_order) or the batch's own")
    p.add_argument("--partition", type=int, default=512, help="tokens per partition (partitioned)")
    p.add_argument("--waves", type=int, default=0, help="wavefronts per workgroup (0 = default)")
    p.add_argument("--workers", type=int, default=0, help="balanced workers (0 = default)")
    p.add_argument("--layers", type=int, default=0, help="layer pools to rotate (0 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--graph", action="store_true", help="replay the steps from a HIP graph")
    p.add_argument("--kv-hint", default="auto", choices=["auto", "stream", "cached"],
                   help="pool reads: stream (PKV_DECODE_STREAM_KV, for batches whose tables share "
                        "no block), cached, or auto = stream exactly when the tables share none")
    p.add_argument("--step", default="auto", choices=["auto", "append", "split"],
                   help="append: one call per step; split: KV write then decode; auto: append "
                        "when the step writes one token per sequence at position len-1 "
                        "(split with --shared-prefix)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="run one plain device copy of this many MiB first (scales PMC byte counters)")
    return p.parse_args()


def build_workload(name, q_heads: int = 0):
    import workloads
    if name == "c1":
        return workloads.c1_tiny_f32()
    if name == "c2":
        return workloads.c2_qwen_decode(num_q_heads=q_heads or 28)
    if name == "c3":
        return workloads.c3_shared_prefix()
    if name == "c4":
        return workloads.c4_long_context(block_size=16)
    if name == "c4bs32":
        return workloads.c4_long_context(block_size=32)
    return workloads.c5_fp8()


def measured_traffic(workload: str, root: str | None = None,
                     sources: tuple = ("decode.hip", "tile.h")):
    """HBM bytes per launch of the measured kernel(s) from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summary whose title names exactly this
    workload key ("<case>" or "<case>+cascade"), or None when the kernel
    sources (the files in `sources`, hashed together) changed since the
    counters were taken.  root: the directory with profiles/ (default: this
    file's)."""
    import glob
    import hashlib
    here = root or os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_cache_135_amd", "csrc")
    h = hashlib.sha256()
    for name in sources:
        h.update(open(os.path.join(csrc, name), "rb").read())
    sha = h.hexdigest()
    field = "+".join(sources) + " sha256"
    for path in sorted(glob.glob(os.path.join(here, "profiles", "*_pmc_traffic.md"))):
        fields = {}
        with open(path) as f:
            first = f.readline()
            for line in f:
                if ":" in line:
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        key = first.split(":", 1)[-1].strip()
        key = key[:-len(" decode step")] if key.endswith(" decode step") else key
        if key == workload and fields.get(field) == sha:
            return int(fields["traffic_bytes_per_launch"]), fields.get("kernel", "")
    return None, None


def read_ceiling(stream, gib: int = 2, reps: int = 20) -> dict:
    """The box's attainable streaming-read rate: the library's read probe over a
    fresh device buffer (larger than L2 and the MALL), back to back between
    two events, after two untimed passes."""
    import torch

    import paged_kv_cache_135_amd as pkv
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = pkv.read_probe(buf, stream=stream)
    pkv.read_probe(buf, sink, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        pkv.read_probe(buf, sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / reps
    del buf
    return {"value": round((gib << 30) / s / 1e9, 1), "unit": "GB/s", "bytes": gib << 30,
            "kernel": "read_probe_kernel (one pass, 16-byte non-temporal loads)"}


def read_ceiling_same_size(stream, nbytes: int, regions: int = 4, reps: int = 20) -> dict:
    """The read probe over as many bytes as the measured kernel reads per
    launch, rotating over `regions` buffers of that size (as the bench rotates
    layer pools) so that no pass finds its data in the last-level cache: the
    streaming-read rate a launch of that size can reach, start-up and drain
    included."""
    import torch

    import paged_kv_cache_135_amd as pkv
    n = (int(nbytes) + 15) // 16 * 16
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(regions)]
    sink = pkv.read_probe(bufs[0], stream=stream)
    for b in bufs:
        pkv.read_probe(b, sink, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        pkv.read_probe(bufs[i % regions], sink, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / reps
    del bufs
    return {"value": round(n / s / 1e9, 1), "unit": "GB/s", "bytes": n, "regions": regions,
            "us_per_pass": round(s * 1e6, 2)}


def gather_ceiling(case, pools, stream, workers: int = 0, reps: int = 20) -> dict:
    """The decode's tile gather alone (pkv_tile_gather_probe) over this batch's
    tiles in the balanced split's order, the same worker count, rotating over
    the layer pools: mode 0 loads the MFMA operands straight to registers (the
    decode's way), mode 1 stages every tile through LDS first.  Both read the
    same words, so their sinks must agree."""
    import numpy as np
    import torch

    import paged_kv_cache_135_amd as pkv
    H, bs = case.num_kv_heads, case.block_size
    rows = []
    for s, n in enumerate(case.context_lens):
        for h in range(H):
            for j in range((int(n) + 15) // 16):
                tok = 16 * j
                rows.append((int(case.block_tables[s, tok // bs]) * H + h) * bs + tok % bs)
    tile_rows = torch.tensor(rows, dtype=torch.int32, device="cuda")
    W = workers or 4 * torch.cuda.get_device_properties(0).multi_processor_count
    out = {"workers": W, "tiles": len(rows), "bytes": len(rows) * 8192}
    sinks = {}
    for mode, name in ((0, "direct"), (1, "lds_staged")):
        sink = pkv.tile_gather_probe(pools[0][0], pools[0][1], tile_rows, W, mode, stream=stream)
        for kc, vc in pools:
            pkv.tile_gather_probe(kc, vc, tile_rows, W, mode, sink, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(reps):
            kc, vc = pools[i % len(pools)]
            pkv.tile_gather_probe(kc, vc, tile_rows, W, mode, sink, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        pkv.tile_gather_probe(pools[0][0], pools[0][1], tile_rows, W, mode, sink, stream=stream)
        torch.cuda.synchronize()
        x = 0
        for w in sink.cpu().numpy().view(np.uint32):
            x ^= int(w)
        sinks[name] = x
        out[name + "_us"] = round(us, 2)
        out[name + "_gbps"] = round(out["bytes"] / us / 1e3, 1)
    out["same_words"] = sinks["direct"] == sinks["lds_staged"]
    return out


def _oracle_steps(case, seconds):
    """Repeat the oracle's whole step (write + decode) for about `seconds`."""
    import oracle
    kc, vc = case.key_cache.copy(), case.value_cache.copy()
    reps = 0
    t0 = time.perf_counter()
    while True:
        if case.k_new is not None:
            oracle.paged_kv_write(case.k_new, case.v_new, case.slot_mapping, kc, vc,
                                  case.k_scale, case.v_scale)
        oracle.paged_attention_decode(case.q, kc, vc, case.block_tables, case.context_lens,
                                      case.scale, case.block_size, case.k_scale, case.v_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return reps, el


def cpu_baseline(case, seconds):
    """The fp64 oracle (write + decode of one step) on this host's cores, and
    a shorter sample of it on one thread (OpenMP's thread count set through
    libgomp, then restored)."""
    import ctypes
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    reps, el = _oracle_steps(case, seconds)
    single = None
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        r1, e1 = _oracle_steps(case, seconds / 2)
        gomp.omp_set_num_threads(threads)
        single = {"value": case.kv_bytes() * r1 / e1 / 1e9, "unit": "GB/s", "cores": 1,
                  "tokens_per_s_per_layer": case.num_seqs * r1 / e1,
                  "sample": f"the same step, {r1} times in {e1:.1f} s"}
    except OSError:
        pass
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": case.kv_bytes() * reps / el / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole {case.name} step (write + fp64 decode of all {case.num_seqs} "
                  f"sequences), repeated {reps} times in {el:.1f} s",
        "tokens_per_s_per_layer": case.num_seqs * reps / el,
        "cpu_model": model,
        "single_thread": single,
    }


def copy_calibration(mib: int) -> None:
    """One device copy of `mib` MiB, for scaling the byte counters of a
    rocprofv3 --pmc run (a copy of known size read and written once)."""
    if not mib:
        return
    import torch
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def copy_ceiling(nbytes: int, reps: int = 200) -> dict:
    """A plain device copy moving the same bytes (nbytes / 2 read, nbytes / 2
    written), back to back between two events: what a simple streaming kernel
    reaches at this size."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    return {"kind": "torch device copy of the same bytes moved", "bytes": 2 * src.numel(),
            "us": round(us, 3), "value": round(2 * src.numel() / us / 1e3, 1), "unit": "GB/s"}


def bench_chunk_write(args):
    """The E4M3 workload's KV write on its own: 4,096 bf16 tokens (8 KV heads x
    128) quantized into distinct random slots of the E4M3 pool.  Algorithmic
    bytes per call: the bf16 rows read plus the E4M3 codes written (K and V)."""
    import numpy as np
    import torch

    import paged_kv_cache_135_amd as pkv
    import workloads

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    print("[bench] building workload c5 (chunk write)", file=sys.stderr, flush=True)
    case = workloads.c5_fp8()
    kc, vc = dev(case.key_cache), dev(case.value_cache)
    kn, vn, slots = dev(case.k_new), dev(case.v_new), dev(case.slot_mapping)
    T, H, D = case.k_new.shape
    moved = 2 * T * H * D * (2 + 1)
    w = pkv.WriteLaunch(kn, vn, slots, kc, vc, k_scale=case.k_scale, v_scale=case.v_scale)
    copy_calibration(args.copy_calibration_mib)
    for _ in range(args.warmup):
        w()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        w()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    eager = e0.elapsed_time(e1) / 1e3 / args.steps
    # The launch from Python takes about as long as the kernel, so back-to-back
    # eager launches leave the GPU idle between them; the kernel's own duration
    # comes from the same launches replayed from a graph (50 per replay).
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        w()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    per_graph = 50
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            w()
    g.replay()
    torch.cuda.synchronize()
    replays = max(1, args.steps // per_graph)
    e0.record(stream)
    for _ in range(replays):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) / 1e3 / (replays * per_graph)
    gbps = moved / per / 1e9
    print(f"[bench] chunk write: {per*1e6:.2f} us per launch replayed from a graph, {gbps:.1f} GB/s "
          f"({eager*1e6:.2f} us per eager launch back to back)", file=sys.stderr, flush=True)
    res = {
        "metric": "KV write of a 4,096-token bf16 chunk into an E4M3 cache: GB/s moved (read + write)",
        "value": round(moved / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16->fp8_e4m3", "data": "synthetic",
        "config": {"workload": "c5_fp8_chunk_write", "tokens": int(T), "num_kv_heads": int(H),
                   "head_dim": int(D), "block_size": case.block_size},
        "bytes_per_call": moved, "write_kernel_us": round(per * 1e6, 3),
        "eager_launch_us": round(eager * 1e6, 3),
        "ceiling": copy_ceiling(moved),
        "roofline": {"kernel": "kv_write_kernel (bf16 -> E4M3)", "bound": "hbm",
                     "achieved": round(gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("c5_fp8_chunk_write", sources=("kv_write.hip", "e4m3.h"))[0]},
    }
    if not args.no_cpu_baseline:
        import ctypes

        import oracle
        kh, vh = case.key_cache.copy(), case.value_cache.copy()
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))

        def writes(seconds):
            reps, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < seconds:
                oracle.paged_kv_write(case.k_new, case.v_new, case.slot_mapping, kh, vh,
                                      case.k_scale, case.v_scale)
                reps += 1
            return reps, time.perf_counter() - t0

        reps, el = writes(min(args.cpu_seconds, 10.0))
        res["cpu_baseline"] = {"value": round(moved * reps / el / 1e9, 3), "unit": "GB/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"the same 4,096-token write, {reps} times in {el:.1f} s"}
        try:
            gomp = ctypes.CDLL("libgomp.so.1")
            gomp.omp_set_num_threads(1)
            r1, e1 = writes(min(args.cpu_seconds, 10.0) / 2)
            gomp.omp_set_num_threads(threads)
            res["cpu_baseline"]["single_thread"] = {
                "value": round(moved * r1 / e1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                "sample": f"the same write, {r1} times in {e1:.1f} s"}
        except OSError:
            pass
    print(json.dumps(res), flush=True)
    return 0


def bench_copy_blocks(args):
    """Copy-on-write block copies: 4096 (src, dst) pairs over the Qwen-shaped
    bf16 pool (4 KV heads x 16 slots x 128 dims: 16 KiB per block per pool).
    Algorithmic bytes per call: pairs x 2 pools x block bytes, read and written."""
    import numpy as np
    import torch

    import paged_kv_cache_135_amd as pkv
    import workloads
    NB, H, bs, D, P = 20000, 4, 16, 128, 4096
    rng = np.random.default_rng(1005)
    kc = torch.empty((NB, H, bs, D), dtype=torch.bfloat16, device="cuda").normal_()
    vc = torch.empty_like(kc).normal_()
    perm = rng.permutation(NB).astype(np.int32)
    pairs_np = np.stack([perm[:P], perm[P:2 * P]], axis=1)
    pairs = torch.from_numpy(pairs_np).cuda()
    pkv.validate_block_pairs(pairs_np, NB)
    block_bytes = H * bs * D * 2
    moved = P * 2 * block_bytes * 2
    copy_calibration(args.copy_calibration_mib)
    for _ in range(args.warmup):
        pkv.paged_kv_copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        pkv.paged_kv_copy_blocks(kc, vc, pairs)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    res = {
        "metric": "copy-on-write block copy: GB/s moved (read + write)",
        "value": round(moved / (us / 1e6) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "cow_block_copy", "pairs": P, "block_bytes_per_pool": block_bytes,
                   "num_blocks": NB},
        "roofline": {"kernel": "copy_blocks_kernel", "bound": "hbm",
                     "achieved": round(moved / (us / 1e6) / 1e9, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(moved / (us / 1e6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("cow_block_copy", sources=("copy_blocks.hip",))[0]},
    }
    if not args.no_cpu_baseline:
        import oracle
        kh = kc.view(torch.int16).cpu().numpy().view(np.uint16)
        vh = vc.view(torch.int16).cpu().numpy().view(np.uint16)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            oracle.copy_blocks(kh, vh, pairs_np)
            reps += 1
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(moved * reps / el / 1e9, 3), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"the same {P} pair copies, {reps} times in {el:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def bench_swap(args):
    """Swap-out / swap-in of 4,096 blocks (16 KiB per block and pool, K and V:
    128 MiB) of the Qwen-shaped pool: gather into a device staging buffer and
    scatter back (HBM-bound: every byte read and written once), and the same
    with a copy-engine transfer to / from pinned host memory (host-link-bound)."""
    import numpy as np
    import torch

    import paged_kv_cache_135_amd as pkv
    import workloads

    print("[bench] building swap workload", file=sys.stderr, flush=True)
    case = workloads.c2_qwen_decode()
    kc = torch.from_numpy(case.key_cache.view(np.int16)).cuda().view(torch.bfloat16)
    vc = torch.from_numpy(case.value_cache.view(np.int16)).cuda().view(torch.bfloat16)
    rng = np.random.default_rng(77)
    n = 4096
    ids = torch.from_numpy(rng.choice(kc.shape[0], size=n, replace=False).astype(np.int32)).cuda()
    per_block = kc[0].numel() * kc.element_size()
    moved = 2 * n * per_block  # K and V bytes per direction
    res_all = {}
    shape = (n,) + tuple(kc.shape[1:])
    sk = torch.empty(shape, dtype=kc.dtype, device="cuda")
    sv = torch.empty_like(sk)
    hk = torch.empty(shape, dtype=kc.dtype, pin_memory=True)
    hv = torch.empty_like(hk)
    for where in ("device", "pinned"):
        if where == "device":
            gather = lambda: pkv.paged_kv_gather_blocks(kc, vc, ids, sk, sv)
            scatter = lambda: pkv.paged_kv_scatter_blocks(sk, sv, ids, kc, vc)
        else:  # device staging + copy-engine transfer to / from pinned host memory
            gather = lambda: pkv.swap_out_to_host(kc, vc, ids, hk, hv, staging=(sk, sv))
            scatter = lambda: pkv.swap_in_from_host(hk, hv, ids, kc, vc, staging=(sk, sv))
        for _ in range(args.warmup):
            gather()
            scatter()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        K = args.steps if where == "device" else max(1, args.steps // 10)
        t = {}
        for name, fn in (("gather", gather), ("scatter", scatter)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(K):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t[name] = e0.elapsed_time(e1) / 1e3 / K
        res_all[where] = t
        print(f"[bench] swap via {where}: gather {t['gather']*1e6:.1f} us "
              f"({moved / t['gather'] / 1e9:.1f} GB/s out), scatter {t['scatter']*1e6:.1f} us",
              file=sys.stderr, flush=True)
    dev_g = res_all["device"]["gather"]
    res = {
        "metric": "swap-out gather of whole blocks to a device staging buffer: GB/s moved (read + write)",
        "value": round(2 * moved / dev_g / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dev_g * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "swap_4096_blocks", "blocks": n, "block_bytes_per_pool": per_block},
        "device_staging": {k: round(v * 1e6, 2) for k, v in res_all["device"].items()},
        "pinned_host_staging_us": {k: round(v * 1e6, 2) for k, v in res_all["pinned"].items()},
        "pinned_host_gbps": {k: round(moved / v / 1e9, 2) for k, v in res_all["pinned"].items()},
        "roofline": {"kernel": "copy_blocks_kernel (gather)", "bound": "hbm",
                     "achieved": round(2 * moved / dev_g / 1e9, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(2 * moved / dev_g / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle
        ids_h = ids.cpu().numpy()
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            oracle.gather_blocks(case.key_cache, ids_h)
            oracle.gather_blocks(case.value_cache, ids_h)
            reps += 1
        el = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(2 * moved * reps / el / 1e9, 3), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"oracle gather of the same 4,096 blocks, {reps} times"}
    print(json.dumps(res), flush=True)
    return 0


def bench_prefill(args):
    """Chunked prefill (p1): one call attends 4,096 new query tokens (8 sequences
    x 512) causally over their cached prefixes and chunks.  It is a dense
    contraction, so it is measured in TFLOP/s against the bf16 MFMA peak."""
    import numpy as np
    import torch

    import paged_kv_cache_135_amd as pkv
    import workloads

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    print("[bench] building workload p1", file=sys.stderr, flush=True)
    case = workloads.p1_chunked_prefill()
    flops = case.prefill_flops()
    kvb = case.prefill_kv_bytes()
    q, tables, lens, qs = dev(case.q), dev(case.block_tables), dev(case.context_lens), dev(case.query_start)
    layers = 2
    pools = [(dev(case.key_cache), dev(case.value_cache))]
    pools += [(pools[0][0].clone(), pools[0][1].clone()) for _ in range(layers - 1)]
    out = torch.empty_like(q)
    mql = int(np.diff(case.query_start).max())
    calls = [pkv.PrefillLaunch(out, q, kc, vc, tables, lens, qs, mql, case.scale, case.block_size,
                               rows_per_wave=args.prefill_rows) for kc, vc in pools]
    for i in range(args.warmup):
        calls[i % layers]()
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for i in range(K):
        calls[i % layers]()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / K
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        calls[i % layers]()
    e1.record(stream)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) / 1e3 / K
    achieved = flops / per / 1e12
    print(f"[bench] prefill: {per*1e6:.1f} us per launch, {achieved:.1f} TFLOP/s, "
          f"wall {wall*1e6:.1f} us", file=sys.stderr, flush=True)
    res = {
        "metric": "chunked prefill paged attention: TFLOP/s (causal, algorithmic flops)",
        "value": round(flops / wall / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": case.name, "num_seqs": case.num_seqs, "query_tokens": int(q.shape[0]),
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "block_size": case.block_size,
                   "context_tokens": int(case.context_lens.astype(np.int64).sum()),
                   "rows_per_wave": args.prefill_rows or None, "layer_pools": layers},
        "flops_per_step": flops, "kv_bytes_per_step": kvb,
        "kv_gbps": round(kvb / per / 1e9, 2), "prefill_kernel_us": round(per * 1e6, 2),
        "roofline": {"kernel": "prefill_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle
        # bounded sample: the oracle on whole sequences (shortest first) for ~cpu-seconds
        order = np.argsort(case.context_lens)
        done_flops, el, used = 0, 0.0, []
        for s_ in order:
            a, b = int(case.query_start[s_]), int(case.query_start[s_ + 1])
            t1 = time.perf_counter()
            oracle.paged_attention_prefill(
                np.ascontiguousarray(case.q[a:b]), case.key_cache, case.value_cache,
                np.ascontiguousarray(case.block_tables[s_:s_ + 1]),
                np.ascontiguousarray(case.context_lens[s_:s_ + 1]), np.array([0, b - a], np.int32),
                case.scale, case.block_size)
            el += time.perf_counter() - t1
            n, c = int(case.context_lens[s_]), b - a
            done_flops += (c * (n - c) + c * (c + 1) // 2) * case.num_q_heads * case.head_dim * 4
            used.append(int(s_))
            if el >= args.cpu_seconds:
                break
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        # the oracle splits (sequence, KV head) pairs over threads: one sequence
        # at a time keeps at most num_kv_heads of them busy
        res["cpu_baseline"] = {"value": round(done_flops / el / 1e12, 6), "unit": "TFLOP/s",
                               "cores": min(threads, case.num_kv_heads), "kind": "oracle",
                               "sample": f"fp64 oracle on sequences {used} of the batch "
                                         f"({len(used)} of {case.num_seqs}), {el:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(decode shards by sequence or by KV head with no cross-GPU exchange)",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import paged_kv_cache_135_amd as pkv

    def dev(a):
        # host arrays carry bf16 as uint16 bits and E4M3 as uint8 codes
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    pkv.load()
    if args.workload == "cow":
        return bench_copy_blocks(args)
    if args.workload == "c5write":
        return bench_chunk_write(args)
    if args.workload == "p1":
        return bench_prefill(args)
    if args.workload == "swap":
        return bench_swap(args)
    print(f"[bench] building workload {args.workload}", file=sys.stderr, flush=True)
    if args.q_heads and args.workload != "c2":
        print("--q-heads applies to the Qwen-shaped workload (c2) only", file=sys.stderr)
        return 2
    case = build_workload(args.workload, args.q_heads)
    pool_bytes = case.key_cache.nbytes * 2
    layers = args.layers or max(2, math.ceil(4 * MALL_BYTES / pool_bytes))
    layers = min(layers, 16)

    q = dev(case.q)
    tables, lens = dev(case.block_tables), dev(case.context_lens)
    kc0, vc0 = dev(case.key_cache), dev(case.value_cache)
    if case.fill_k is not None:  # pools that start empty are filled through the write
        pkv.paged_kv_write(dev(case.fill_k), dev(case.fill_v), dev(case.fill_slots), kc0, vc0,
                           k_scale=case.k_scale, v_scale=case.v_scale)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(layers - 1)]
    # the step's own write (none for the tiny f32 workload, whose tokens all
    # arrive through the fill)
    has_write = case.k_new is not None
    knew, vnew, slots = ((dev(case.k_new), dev(case.v_new), dev(case.slot_mapping)) if has_write
                         else (None, None, None))
    out = torch.empty_like(q)
    nbytes = pkv.decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                        case.head_dim, case.block_tables.shape[1],
                                        case.block_size, args.mode, args.partition, args.workers)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    step = args.step
    prefix_len = 0
    if args.shared_prefix:
        if not case.shared_blocks:
            print("--shared-prefix needs a workload with shared prefix blocks (c3)", file=sys.stderr)
            return 2
        prefix_len = case.shared_blocks * case.block_size
    if step == "auto":
        step = "split"
        # one call per step when every new token is its sequence's last position.
        # Not for a shared prefix: there the tails' launch with the write folded
        # in is as much slower as the write launch it saves (115.2 vs 114.8 us
        # per step on the 256-sequence batch); --step append selects it.
        if has_write and case.slot_mapping.shape[0] == case.num_seqs and not prefix_len:
            try:
                pkv.validate_append_slots(case.slot_mapping, case.block_tables, case.context_lens,
                                          case.key_cache.shape[0], case.block_size)
                step = "append"
            except pkv.PagedKVError:
                pass
    if not has_write:
        step = "split"
    append = step == "append"
    # the streaming hint is for calls that read every block once: decided from
    # the tables (past the shared prefix when it is computed apart)
    shared = pkv.tables_share_blocks(case.block_tables, case.context_lens, case.block_size,
                                     skip_blocks=prefix_len // case.block_size)
    stream_kv = args.kv_hint == "stream" or (args.kv_hint == "auto" and not shared)
    # the single pass starts the sequences longest first: the order comes from
    # the host's lengths (once per step, shared by every layer), made before
    # the timed region like the tables themselves
    order = None
    if args.seq_order == "lpt":
        order = torch.from_numpy(pkv.decode_order(case.context_lens)).to(q.device)
    dkw = dict(k_scale=case.k_scale, v_scale=case.v_scale, mode=args.mode,
               partition_size=args.partition, waves_per_group=args.waves,
               num_workers=args.workers, workspace=ws, stream_kv=stream_kv, seq_order=order)

    if prefix_len:
        dkw["mode"] = "auto"
        dkw["workspace"] = None

    def decode_launch(kc, vc, defer):
        if prefix_len:  # its kernels launch together: time the whole call
            return pkv.DecodeLaunch(out, q, kc, vc, tables, lens, case.scale, case.block_size,
                                    append=(knew, vnew, slots) if append else None,
                                    prefix_len=prefix_len, **dkw)
        return pkv.DecodeLaunch(out, q, kc, vc, tables, lens, case.scale, case.block_size,
                                append=(knew, vnew, slots) if append else None,
                                defer_merge=defer, **dkw)

    writes = [pkv.WriteLaunch(knew, vnew, slots, kc, vc, k_scale=case.k_scale,
                              v_scale=case.v_scale) if has_write else (lambda: None)
              for kc, vc in pools]
    decodes = [decode_launch(kc, vc, False) for kc, vc in pools]
    split_decodes = [decode_launch(kc, vc, True) for kc, vc in pools]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def run_steps(n, ev=None):
        # ev[i]: events before the write, before the decode call and after it
        for i in range(n):
            li = i % layers
            if ev is not None:
                ev[i][0].record(stream)
            if not append:
                writes[li]()
            if ev is not None:
                ev[i][1].record(stream)
            decodes[li]()
            if ev is not None:
                ev[i][2].record(stream)

    copy_calibration(args.copy_calibration_mib)
    print(f"[bench] warmup {args.warmup} steps, {layers} layer pools", file=sys.stderr, flush=True)
    run_steps(args.warmup)
    torch.cuda.synchronize()

    # timed region 1: wall clock over K steps (no per-step events)
    K = args.steps
    if args.graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_steps(layers)
        torch.cuda.synchronize()
        reps = max(1, K // layers)
        K = reps * layers
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_steps(K)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / K

    # timed region 2: HIP events around each step's write and decode call
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    run_steps(K, ev)
    torch.cuda.synchronize()
    wr_ms = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)])
    call_ms = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])

    def back_to_back(launches, n):
        # n launches between one pair of events on the launch stream (an event
        # pair around each launch also counts its dispatch latency)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            launches[i % len(launches)]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    # timed region 3: the whole decode call (every kernel it launches: the
    # streaming kernel and, for split pairs or partitions, its merge or reduce
    # kernel) K times back to back
    call_s = back_to_back(decodes, K)
    # hot cache, reported beside the cold figure: every call reads the same
    # layer's pool (above, the pools rotate so each call reads from HBM)
    hot_s = back_to_back(decodes[:1], K)
    # timed region 4: the dominant kernel alone, the streaming kernel (the
    # call made with its merge deferred, K launches back to back); its merge
    # kernel is what the whole call adds (nothing for the single pass).  A
    # shared-prefix call launches its kernels together: there the whole call.
    if prefix_len:
        kern_s, merge_s = call_s, 0.0
    else:
        kern_s = back_to_back(split_decodes, K)
        merge_s = max(0.0, call_s - kern_s)

    kv = case.kv_bytes()
    # counters are keyed by workload and, outside auto mode, by the mode
    key = case.name + ("+cascade" if prefix_len else "")
    if args.mode != "auto" and not prefix_len:
        key += f"+{args.mode}" + (str(args.partition) if args.mode == "partitioned" else "")
    traffic, traffic_kernel = measured_traffic(key)
    ceiling = read_ceiling(stream)
    value = kv / (ms_per_step / 1e3) / 1e9
    # HBM roofline: bytes that must come from memory; a shared prefix counts once
    roof_bytes = case.unique_kv_bytes() if case.shared_blocks else kv
    achieved = roof_bytes / kern_s / 1e9
    call_achieved = roof_bytes / call_s / 1e9
    same = read_ceiling_same_size(stream, roof_bytes)
    ceiling["same_size"] = dict(same, frac_of_ceiling=round(achieved / same["value"], 4))
    if case.cache_dtype == "bf16" and case.head_dim == 128 and not prefix_len:
        ceiling["tile_gather"] = gather_ceiling(case, pools, stream, args.workers or 0)
    print(f"[bench] step {step}: decode call {call_s*1e6:.1f} us back to back "
          f"({call_ms.mean()*1e3:.1f} us between events around each, p10 "
          f"{np.percentile(call_ms,10)*1e3:.1f}, p90 {np.percentile(call_ms,90)*1e3:.1f}): "
          f"streaming kernel {kern_s*1e6:.1f} + merge {merge_s*1e6:.1f} us; "
          f"write {wr_ms.mean()*1e3:.1f} us, wall step {ms_per_step*1e3:.1f} us",
          file=sys.stderr, flush=True)

    res = {
        "metric": "paged decode attn: KV GB/s read (% of MI355X HBM peak) + decode tokens/s per layer",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8_e4m3": "fp8_e4m3/bf16", "f32": "f32"}[case.cache_dtype],
        "data": "synthetic",
        "config": {
            "workload": case.name,
            "num_seqs": case.num_seqs,
            "num_q_heads": case.num_q_heads,
            "num_kv_heads": case.num_kv_heads,
            "head_dim": case.head_dim,
            "block_size": case.block_size,
            "context_tokens": int(case.context_lens.astype(np.int64).sum()),
            "decode_mode": args.mode,
            "partition_size": args.partition if args.mode == "partitioned" else None,
            "waves_per_group": args.waves or None,
            "num_workers": args.workers or None,
            "layer_pools": layers,
            "graph": bool(args.graph),
            "step": step,
            "shared_prefix_tokens": prefix_len or None,
            "tables_share_blocks": bool(shared),
            "kv_stream_hint": bool(stream_kv),
            "seq_order": args.seq_order,
        },
        "kv_bytes_per_step": kv,
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_tokens_per_s_per_layer": round(case.num_seqs / (ms_per_step / 1e3), 1),
        "decode_call_us": round(call_s * 1e6, 2),
        "decode_call_event_pair_us": round(float(call_ms.mean()) * 1e3, 2),
        "decode_call_event_pair_percentiles_us": {
            f"p{p}": round(float(np.percentile(call_ms, p)) * 1e3, 2) for p in (10, 50, 90)},
        "decode_call_hot_cache_us": round(hot_s * 1e6, 2),
        "streaming_kernel_us": round(kern_s * 1e6, 2),
        "merge_us": round(merge_s * 1e6, 2),
        "write_us": round(float(wr_ms.mean()) * 1e3, 2) if not append else 0.0,
        "roofline": {
            "kernel": "shared-prefix decode call (prefix, tail and merge kernels)" if prefix_len
            else "streaming decode kernel (" + ("append, " if append else "") + {
                "single": "single pass", "partitioned": "partitions",
                "balanced": "balanced split", "auto": "auto mode"}[args.mode] + ")",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
        },
        # the whole decode call: every kernel it launches (streaming kernel and,
        # for split pairs, the merge), back to back
        "call_roofline": {
            "achieved": round(call_achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(call_achieved / HBM_PEAK_GBPS, 4), "us_per_call": round(call_s * 1e6, 2)},
        # the same kernel's rate against what one plain streaming pass reaches on this machine
        "read_ceiling": dict(ceiling, frac_of_ceiling=round(achieved / ceiling["value"], 4)),
    }
    if case.cache_dtype != "bf16" or case.shared_blocks:
        res["unique_kv_bytes_per_step"] = case.unique_kv_bytes()
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline ({args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
