#!/usr/bin/env python3
"""Benchmark of the sink-attention hot path on one MI355X.

One step = one split-KV decode of the decode workload (sinkattn_decode_split then
sinkattn_decode_merge): 8 sequences x 8192 cached tokens, 64 query heads over 8 KV heads,
head_dim 64, bf16, 8 chunks of 1024 keys. The single-launch form (sinkattn_decode: chunk states
and their merge in one kernel) is timed beside it. ``value`` is algorithmic KV bytes per second (the K and V rows actually
read plus q, out and sinks), with inputs resident in HBM. Decode inputs rotate over enough copies
(> 512 MB in all) that the 256 MB Infinity Cache cannot serve a step from the previous one.

The same JSON line also carries:
* ``roofline`` for the dominant kernel (the split kernel), timed alone with events on the stream
  it runs on, against the 8 TB/s HBM peak; ``traffic`` from the committed rocprofv3 FETCH_SIZE /
  WRITE_SIZE summary when it was taken on the current kernel source, else null;
* ``prefill``: causal prefill of one 8192-token sequence (64/8 heads, bf16), TFLOP/s over the
  allowed causal pairs (4 * D per pair) against the 2.5 PFLOP/s dense bf16 MFMA peak;
* ``prefill_append``: 512 new tokens against a 32768-key cache, unsplit and split 4 ways along the
  KV length (sinkattn_prefill_split + sinkattn_decode_merge);
* ``decode_multi``: the decode workload with T = 2, 4, 8 new tokens per sequence (the last T of the
  8192 keys), split + merge and single-launch, in KV GB/s;
* ``decode_long`` and ``mixed``: the long-decode workload (32 sequences of 16K-32K keys, 16 chunks,
  outlier keys) and the mixed one (128 decode sequences of 1-8192 keys; 16 prefill sequences of
  512-4096 tokens), each against its time target;
* ``moe_route``: MoE routing weights (top-4 of 128 experts, softmax over the chosen four) for 65,536
  tokens of bf16 logits, in GB/s of logits read plus ids and weights written;
* ``linear``: the linear layer with the bias in the accumulators, M = N = K = 4096, bf16 and FP8 with
  128 x 128 block scaling, TFLOP/s against the dense MFMA peaks (torch's bf16 linear timed beside it
  as context);
* ``cpu_baseline``: the float64 CPU oracle on the same decode workload, over the host cores (one BLAS
  thread per worker thread).

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 5] [--no-cpu-baseline] [--no-prefill]
                      [--no-hot] [--no-multi] [--no-moe] [--no-linear] [--no-long]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP8_MFMA_PEAK_TFLOPS = 5000.0
METRIC = "decode KV GB/s (% of HBM peak) + prefill TFLOP/s (% of bf16 MFMA peak)"
ROTATE_BYTES = 512 * 2**20
CALIB_BYTES = 256 * 2**20
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_split_b8_len8192_pmc.txt")
# The split kernel's complete source: its traffic figure is only reused while these are unchanged.
SPLIT_SOURCES = [os.path.join(ROOT, "gqa_learned_softmax_amd", "csrc", f)
                 for f in ("decode_split.hip", "chunk_merge.h", "device_common.h", "launch.h", "plan.h")]


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _source_hash(paths):
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic_from_profile(kernel_hash):
    """(fetch + write) bytes per split launch from the committed PMC summary, if it matches."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    text = open(PMC_SUMMARY).read()
    m = re.search(r"kernel_source_sha256_16:\s*(\w+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != kernel_hash:
        return None
    return float(t.group(1))


def _capture(fn, calls, torch):
    """A HIP graph holding ``calls`` back-to-back calls ``fn(0) .. fn(calls - 1)``.

    Replaying it issues the kernels without Python or ctypes in between, so event timings see
    GPU time (plus the small inter-kernel dispatch gap) rather than host launch overhead.
    """
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(calls):
            fn(i)
    return graph


def _time_graph(graph, calls, torch, replays=20):
    """Median over ``replays`` replays of the ms per captured call, events on the replay stream
    around each replay (the first replay, which uploads the graph, is not timed)."""
    graph.replay()
    torch.cuda.synchronize()
    events = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    events[0].record()
    for r in range(replays):
        graph.replay()
        events[r + 1].record()
    torch.cuda.synchronize()
    per_call = sorted(events[r].elapsed_time(events[r + 1]) / calls for r in range(replays))
    mid = replays // 2
    return per_call[mid] if replays % 2 else 0.5 * (per_call[mid - 1] + per_call[mid])


# Instructions per wave and iteration of each sinkattn_ceiling_issue kind (include/sinkattn_ceilings.h).
ISSUE_KINDS = {"v_exp_f32": (0, 16), "v_mul_f32": (1, 16), "v_cvt_pk_bf16_f32": (2, 16), "v_fma_f32": (3, 16),
               "mfma_32x32x16_bf16": (4, 4), "mfma_16x16x32_bf16": (5, 4), "mfma32_plus_4_exp": (6, 4),
               "prefill_tile_mix_per_tile": (7, 0.25)}


def measure_issue_cycles(lib, torch, dev, sink, blocks=512, iters=20000):
    """SIMD cycles per instruction of the prefill's inner-loop instructions, two waves per SIMD (512
    work-groups of four waves on 256 CUs): kernel time x the clock the loop ran at (shader cycles
    over 100 MHz ticks, recorded in the kernel) / instructions per SIMD. 'mfma32_plus_4_exp' is per
    MFMA with its four exponentials; 'prefill_tile_mix_per_tile' is per 64 x 64 tile and wave (32 + 8
    MFMAs, 64 mul -> exp, 32 packs) with nothing else to wait for."""
    import ctypes
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    out = {}
    for name, (kind, per_iter) in ISSUE_KINDS.items():
        def launch(i, k=kind):
            rc = lib.sinkattn_ceiling_issue(k, blocks, iters, ctypes.c_void_p(clk.data_ptr()),
                                            ctypes.c_void_p(sink.data_ptr()),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if rc != 0:
                raise RuntimeError(f"issue-cost launch failed ({rc})")
        launch(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch(0)
        e1.record()
        torch.cuda.synchronize()
        t = clk.view(blocks, 2).double()
        ghz = float(t[:, 0].sum() / (t[:, 1].sum() / 100e6)) / 1e9
        waves_per_simd = blocks / 256
        cycles = e0.elapsed_time(e1) * 1e-3 * ghz * 1e9 / (iters * waves_per_simd)
        out[name] = round(cycles / per_iter, 2)
    return out


def measure_ceilings(torch, dev):
    """Measured ceilings (libsinkattn_ceilings, include/sinkattn_ceilings.h): the HBM streaming-read
    rate of a plain kernel, over 2 GiB and over decode-sized 128 MiB reads rotating through that
    buffer (more than the Infinity Cache, so every read comes from HBM); the bf16 MFMA rate of a loop
    of independent v_mfma_f32_32x32x16_bf16 at the clock the chip holds under it; and torch's bf16
    matmul at 8192^3 (hipBLASLt) as the practical library rate."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "gqa_learned_softmax_amd", "libsinkattn_ceilings.so"))
    lib.sinkattn_ceiling_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.sinkattn_ceiling_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sinkattn_ceiling_mfma_bf16_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.sinkattn_ceiling_mfma_bf16_flop.restype = ctypes.c_double
    lib.sinkattn_ceiling_issue.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.uint8, device=dev)
    big = 2 * 2**30
    buf = torch.empty(big, dtype=torch.uint8, device=dev).fill_(1)

    def stream(base, nbytes, blocks):
        stream_ptr = torch.cuda.current_stream().cuda_stream
        rc = lib.sinkattn_ceiling_stream_read(ctypes.c_void_p(base), nbytes, blocks, ctypes.c_void_p(sink.data_ptr()),
                                              ctypes.c_void_p(stream_ptr))
        if rc != 0:
            raise RuntimeError(f"stream-read ceiling launch failed ({rc})")

    res = {}
    best = (0.0, 0)
    for blocks in (1024, 2048, 4096, 8192, 16384):
        ms = _time_graph(_capture(lambda i, b=blocks: stream(buf.data_ptr(), big, b), 3, torch), 3, torch, replays=5)
        best = max(best, (big / (ms * 1e-3) / 1e9, blocks))
    res["stream_read_2GiB_gbs"] = round(best[0], 1)
    res["stream_read_2GiB_blocks"] = best[1]
    part = 128 * 2**20
    n_parts = big // part
    best = (0.0, 0)
    for blocks in (256, 512, 1024, 2048, 4096):
        ms = _time_graph(_capture(lambda i, b=blocks: stream(buf.data_ptr() + (i % n_parts) * part, part, b), 48,
                                  torch), 48, torch, replays=5)
        best = max(best, (part / (ms * 1e-3) / 1e9, blocks))
    res["stream_read_128MiB_gbs"] = round(best[0], 1)
    res["stream_read_128MiB_blocks"] = best[1]
    # The decode workload's own read pattern (8 sequences x 8 chunks of 1024 rows of 1 KB in K and in
    # V, 256-byte slices, 256 work-groups of 512 threads), rotating through the same buffer.
    lib.sinkattn_ceiling_stream_read_slices.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]

    def slices(base):
        stream_ptr = torch.cuda.current_stream().cuda_stream
        rc = lib.sinkattn_ceiling_stream_read_slices(ctypes.c_void_p(base), ctypes.c_void_p(base + part // 2), 8, 8,
                                                     1024, 1024, ctypes.c_void_p(sink.data_ptr()),
                                                     ctypes.c_void_p(stream_ptr))
        if rc != 0:
            raise RuntimeError(f"slice-read ceiling launch failed ({rc})")

    ms = _time_graph(_capture(lambda i: slices(buf.data_ptr() + (i % n_parts) * part), 48, torch), 48, torch,
                     replays=5)
    res["stream_read_decode_slices_gbs"] = round(part / (ms * 1e-3) / 1e9, 1)
    del buf

    def mfma(blocks, iters):
        stream_ptr = torch.cuda.current_stream().cuda_stream
        rc = lib.sinkattn_ceiling_mfma_bf16(blocks, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(stream_ptr))
        if rc != 0:
            raise RuntimeError(f"MFMA ceiling launch failed ({rc})")

    best = (0.0, 0)
    for blocks in (512, 1024):  # two and four waves per SIMD
        ms = _time_graph(_capture(lambda i, b=blocks: mfma(b, 4000), 3, torch), 3, torch, replays=5)
        best = max(best, (lib.sinkattn_ceiling_mfma_bf16_flop(blocks, 4000) / (ms * 1e-3) / 1e12, blocks))
    res["mfma_bf16_loop_tflops"] = round(best[0], 1)
    res["mfma_bf16_loop_blocks"] = best[1]
    lib.sinkattn_ceiling_mfma_bf16_random.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.sinkattn_ceiling_mfma_bf16_random_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.sinkattn_ceiling_mfma_bf16_random_flop.restype = ctypes.c_double

    def mfma_random(blocks, iters):
        stream_ptr = torch.cuda.current_stream().cuda_stream
        rc = lib.sinkattn_ceiling_mfma_bf16_random(blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                                   ctypes.c_void_p(stream_ptr))
        if rc != 0:
            raise RuntimeError(f"random-operand MFMA ceiling launch failed ({rc})")

    best = (0.0, 0)
    for blocks in (512, 1024):
        ms = _time_graph(_capture(lambda i, b=blocks: mfma_random(b, 2000), 3, torch), 3, torch, replays=5)
        best = max(best, (lib.sinkattn_ceiling_mfma_bf16_random_flop(blocks, 2000) / (ms * 1e-3) / 1e12, blocks))
    res["mfma_bf16_random_loop_tflops"] = round(best[0], 1)
    res["mfma_bf16_random_loop_blocks"] = best[1]
    res["issue_cycles"] = measure_issue_cycles(lib, torch, dev, sink)
    n = 8192
    gen = torch.Generator().manual_seed(1010)
    a = torch.randn((n, n), generator=gen).to(torch.bfloat16).to(dev)
    b = torch.randn((n, n), generator=gen).to(torch.bfloat16).to(dev)
    c = torch.empty((n, n), dtype=torch.bfloat16, device=dev)
    torch.matmul(a, b, out=c)
    ms = _time_graph(_capture(lambda i: torch.matmul(a, b, out=c), 3, torch), 3, torch, replays=5)
    res["torch_bf16_matmul_8192_tflops"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    del a, b, c
    return res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def _cpu_unit(task):
    """Oracle decode of one (sequence, KV head) unit, in a worker process (see cpu_baseline)."""
    import oracle
    b, g = task
    st = _CPU_STATE
    grp = st["q"].shape[1] // st["hkv"]
    heads = slice(g * grp, (g + 1) * grp)
    oracle.decode(st["q"][b:b + 1, heads], st["ks"][b][:, :, g:g + 1], st["vs"][b][:, :, g:g + 1],
                  st["sinks"][heads], [st["lens"][b]], st["scale"])


_CPU_STATE = {}


def cpu_baseline_worker(seconds=10.0):
    """The oracle, as it stands, on the decode workload (regenerated from its seed), over a pool of
    worker processes with one BLAS thread each; whole-workload passes repeat until >= ``seconds``.

    Runs in a child process of its own that never touches the GPU (bench.py starts it with
    ``--cpu-baseline-worker`` once the GPU work is done), so forking the pool is safe. Workers: the
    cores this process may use, at most 16 (the host CPUs a one-GPU machine gives its GPU)."""
    os.environ["OMP_NUM_THREADS"] = "1"
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    os.environ["MKL_NUM_THREADS"] = "1"
    import multiprocessing as mp

    import numpy as np
    from threadpoolctl import threadpool_limits

    import workloads

    case = workloads.make(2).decode
    kv_bytes = workloads.decode_kv_bytes(case)
    io_bytes = case.q.numel() * 2 + case.q.numel() * 2 + case.sinks.numel() * 4
    lens = [int(n) for n in case.seqlens_k.tolist()]
    _CPU_STATE.update(q=case.q.double().numpy(), sinks=case.sinks.double().numpy(), lens=lens,
                      ks=[case.k[b:b + 1, :n].float().numpy() for b, n in enumerate(lens)],
                      vs=[case.v[b:b + 1, :n].float().numpy() for b, n in enumerate(lens)],
                      hkv=case.k.shape[2], scale=case.scale)
    tasks = [(b, g) for b in range(len(lens)) for g in range(case.k.shape[2])]
    workers = max(1, min(len(os.sched_getaffinity(0)), 16, len(tasks)))
    with threadpool_limits(limits=1), mp.get_context("fork").Pool(workers) as pool:
        pool.map(_cpu_unit, tasks)  # untimed warm-up pass
        reps = 0
        t0 = time.perf_counter()
        while True:
            pool.map(_cpu_unit, tasks)
            reps += 1
            elapsed = time.perf_counter() - t0
            if elapsed >= seconds:
                break
    return {
        "value": round(reps * (kv_bytes + io_bytes) / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"whole decode workload ({len(lens)} seqs x {max(lens)} keys, {case.q.shape[1]}/{case.k.shape[2]} "
                  f"heads) repeated {reps}x in {elapsed:.1f} s, float64 NumPy {np.__version__}, {workers} worker "
                  f"processes x 1 BLAS thread, one (sequence, KV head) unit per task, {_cpu_model()}",
    }


def cpu_baseline():
    """Runs cpu_baseline_worker in a child process (started with subprocess: nothing is forked from
    this process, which has initialised the GPU) and returns its JSON result."""
    import subprocess
    res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-worker"],
                         capture_output=True, text=True, timeout=600)
    if res.returncode != 0:
        raise RuntimeError(f"CPU baseline worker failed ({res.returncode}):\n{res.stderr[-2000:]}")
    return json.loads(res.stdout.strip().splitlines()[-1])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-multi", action="store_true", help="skip the multi-token decode detail")
    ap.add_argument("--no-moe", action="store_true", help="skip the MoE routing detail")
    ap.add_argument("--no-long", action="store_true", help="skip the long-decode and mixed workloads")
    ap.add_argument("--no-linear", action="store_true", help="skip the linear-layer detail")
    ap.add_argument("--no-hot", action="store_true",
                    help="skip the steps that reuse one K/V set (cache-resident; never the headline)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the measured HBM and MFMA ceilings")
    ap.add_argument("--cpu-baseline-worker", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_baseline_worker:
        print(json.dumps(cpu_baseline_worker()), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the hot path here is a "
              "single-GPU kernel library; no multi-GPU configuration exists.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gqa_learned_softmax_amd as sa
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------------------------------------------------------- counter calibration
    # One plain device-to-device copy of known size (256 MiB read + 256 MiB written). Under
    # rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE give the scale from counter units to bytes.
    calib_src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    # The same copy, timed: a measured HBM ceiling (read + write) beside the spec peak.
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        calib_dst.copy_(calib_src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * CALIB_BYTES / (c0.elapsed_time(c1) / 5 * 1e-3) / 1e9
    del calib_src, calib_dst
    ceilings = None
    if not args.no_ceilings:
        _log("measuring the HBM streaming-read and bf16 MFMA ceilings")
        ceilings = measure_ceilings(torch, dev)
        _log(f"ceilings: {ceilings}")

    # ---------------------------------------------------------------- decode workload (value)
    _log("generating decode workload (8 x 8192, 64/8 heads, bf16)")
    w = workloads.make(2)
    case = w.decode
    kv_bytes = workloads.decode_kv_bytes(case)
    batch, hq, dim = case.q.shape
    chunks = case.num_chunks
    io_bytes = case.q.numel() * 2 + batch * hq * dim * 2 + case.sinks.numel() * 4
    step_bytes = kv_bytes + io_bytes
    split_bytes = kv_bytes + case.q.numel() * 2 + case.sinks.numel() * 4

    set_bytes = case.k.numel() * 2 * 2
    n_sets = max(2, -(-ROTATE_BYTES // set_bytes) + 1)
    k0, v0 = case.k.to(dev), case.v.to(dev)
    ks = [k0] + [k0.clone() for _ in range(n_sets - 1)]
    vs = [v0] + [v0.clone() for _ in range(n_sets - 1)]
    q = case.q.to(dev)
    sinks = case.sinks.to(dev)
    seqlens = case.seqlens_k.to(dev)
    po = torch.empty((batch, hq, chunks, dim), dtype=torch.float32, device=dev)
    pm = torch.empty((batch, hq, chunks), dtype=torch.float32, device=dev)
    pd = torch.empty((batch, hq, chunks), dtype=torch.float32, device=dev)
    out = torch.empty((batch, hq, dim), dtype=torch.bfloat16, device=dev)
    ws = sa.decode_workspace(batch, hq, case.k.shape[2], chunks, dev)

    def fused(i):
        sa.decode_fused(q, ks[i % n_sets], vs[i % n_sets], sinks, seqlens, chunks, case.scale, ws, out=out)

    def split(i):
        sa.decode_split(q, ks[i % n_sets], vs[i % n_sets], sinks, seqlens, chunks, case.scale, po, pm, pd)

    def merge(i):
        sa.decode_merge(po, pm, pd, out=out)

    def split_merge(i):
        split(i)
        merge(i)

    step = split_merge

    def step_hot(i):
        sa.decode_split(q, k0, v0, sinks, seqlens, chunks, case.scale, po, pm, pd)
        merge(i)

    _log(f"decode: {n_sets} rotating K/V sets of {set_bytes / 2**20:.0f} MiB; warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    steps_graph = _capture(step, args.steps, torch)
    steps_graph.replay()  # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    # Timed region: exactly `steps` steps (one replay of the captured steps), synchronised and
    # event-bracketed on both sides.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    # A short spin kernel ahead of the start event keeps the GPU busy while the host submits the
    # graph's kernels, so the events bracket the steps' GPU time and not the host's submission.
    torch.cuda._sleep(1_000_000)
    start.record()
    steps_graph.replay()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    _log(f"decode step {ms_step * 1e3:.2f} us ({wall * 1e3:.2f} ms wall for {args.steps} steps)")
    n_rep = max(args.steps, 50)
    ms_fused = _time_graph(_capture(fused, n_rep, torch), n_rep, torch)
    ms_split = _time_graph(_capture(split, n_rep, torch), n_rep, torch)
    ms_merge = _time_graph(_capture(merge, n_rep, torch), n_rep, torch)
    ms_two = _time_graph(_capture(split_merge, n_rep, torch), n_rep, torch)
    ms_hot = _time_graph(_capture(step_hot, n_rep, torch), n_rep, torch) if not args.no_hot else None
    ms_eager = None
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_rep):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms_eager = e0.elapsed_time(e1) / n_rep
    # The single launch, launched eagerly the same way (one Python call per step instead of two).
    torch.cuda.synchronize()
    e0.record()
    for i in range(n_rep):
        fused(i)
    e1.record()
    torch.cuda.synchronize()
    ms_fused_eager = e0.elapsed_time(e1) / n_rep
    value = step_bytes / (ms_step * 1e-3) / 1e9
    fused_gbs = step_bytes / (ms_fused * 1e-3) / 1e9
    split_gbs = split_bytes / (ms_split * 1e-3) / 1e9
    _log(f"split {ms_split * 1e3:.2f} us ({split_gbs:.0f} GB/s), merge {ms_merge * 1e3:.2f} us, "
         f"split+merge {ms_two * 1e3:.2f} us; fused {ms_fused * 1e3:.2f} us ({fused_gbs:.0f} GB/s)"
         + (f", hot step {ms_hot * 1e3:.2f} us" if ms_hot else ""))

    traffic = _traffic_from_profile(_source_hash(SPLIT_SOURCES))
    # The kernel the split call dispatches for this shape, as the library reports it.
    (split_launch,) = sa.plan_decode(q, k0, v0, sinks, seqlens, chunks, case.scale, form="split")
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode_b8_hq64_hkv8_d64_len8192_chunks8",
            "batch": batch, "kv_len": 8192, "num_q_heads": hq, "num_kv_heads": case.k.shape[2],
            "head_dim": dim, "num_chunks": chunks, "step": "decode_split + decode_merge",
            "rotating_kv_sets": n_sets, "algorithmic_bytes_per_step": step_bytes,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": split_launch["kernel"],
            "grid": split_launch["grid"],
            "achieved": round(split_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(split_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": split_bytes,
            "avg_launch_us": round(ms_split * 1e3, 3),
            "measured_copy_gbs": round(copy_gbs, 1),
            "frac_of_measured_copy": round(split_gbs / copy_gbs, 4),
            "measured_stream_read_gbs": ceilings["stream_read_128MiB_gbs"] if ceilings else None,
            "frac_of_measured_stream_read": (round(split_gbs / ceilings["stream_read_128MiB_gbs"], 4)
                                             if ceilings else None),
            "measured_decode_slices_read_gbs": ceilings["stream_read_decode_slices_gbs"] if ceilings else None,
            "frac_of_measured_decode_slices_read": (round(split_gbs / ceilings["stream_read_decode_slices_gbs"], 4)
                                                    if ceilings else None),
        },
        "ceilings": ceilings,
        "decode_detail": {
            "split_us": round(ms_split * 1e3, 3), "merge_us": round(ms_merge * 1e3, 3),
            "split_plus_merge_us": round(ms_two * 1e3, 3),
            "fused_sinkattn_decode_us": round(ms_fused * 1e3, 3),
            "fused_gbs": round(fused_gbs, 2),
            "step_us_rotated": round(ms_step * 1e3, 3),
            "step_us_hot": round(ms_hot * 1e3, 3) if ms_hot else None,
            "step_us_eager_python_launch": round(ms_eager * 1e3, 3),
            "fused_us_eager_python_launch": round(ms_fused_eager * 1e3, 3),
            "timing": "HIP graph replay of back-to-back calls, events on the replay stream",
            "step_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
            "step_frac_of_measured_stream_read": (round(value / ceilings["stream_read_128MiB_gbs"], 4)
                                                  if ceilings else None),
            "step_frac_of_measured_decode_slices_read": (
                round(value / ceilings["stream_read_decode_slices_gbs"], 4) if ceilings else None),
        },
    }

    # ---------------------------------------------------------------- multi-token decode (detail)
    if not args.no_multi:
        multi = {"workload": "decode_multi_b8_hq64_hkv8_d64_len8192_chunks8", "tokens": {}}
        gen = torch.Generator().manual_seed(1007)
        for t in (2, 4, 8):
            qm = torch.randn((batch, t, hq, dim), generator=gen).to(torch.bfloat16).to(dev)
            mpo = torch.empty((batch * t, hq, chunks, dim), dtype=torch.float32, device=dev)
            mpm = torch.empty((batch * t, hq, chunks), dtype=torch.float32, device=dev)
            mpd = torch.empty_like(mpm)
            mout = torch.empty((batch, t, hq, dim), dtype=torch.bfloat16, device=dev)
            mws = sa.decode_workspace(batch * t, hq, case.k.shape[2], chunks, dev)

            def m_split_merge(i, qm=qm, mpo=mpo, mpm=mpm, mpd=mpd, mout=mout):
                sa.decode_multi_split(qm, ks[i % n_sets], vs[i % n_sets], sinks, seqlens, chunks, case.scale,
                                      mpo, mpm, mpd)
                sa.decode_merge(mpo, mpm, mpd, out=mout.view(batch * t, hq, dim))

            def m_fused(i, qm=qm, mws=mws, mout=mout):
                sa.decode_multi_fused(qm, ks[i % n_sets], vs[i % n_sets], sinks, seqlens, chunks, case.scale,
                                      mws, out=mout)

            m_split_merge(0)
            m_fused(0)
            ms_m2 = _time_graph(_capture(m_split_merge, n_rep, torch), n_rep, torch)
            ms_mf = _time_graph(_capture(m_fused, n_rep, torch), n_rep, torch)
            m_bytes = kv_bytes + 2 * qm.numel() * 2 + case.sinks.numel() * 4
            multi["tokens"][str(t)] = {
                "split_plus_merge_us": round(ms_m2 * 1e3, 3), "fused_us": round(ms_mf * 1e3, 3),
                "split_plus_merge_gbs": round(m_bytes / (ms_m2 * 1e-3) / 1e9, 1),
                "fused_gbs": round(m_bytes / (ms_mf * 1e-3) / 1e9, 1),
            }
            _log(f"multi-token decode T={t}: split+merge {ms_m2 * 1e3:.2f} us, fused {ms_mf * 1e3:.2f} us "
                 f"({m_bytes / (ms_mf * 1e-3) / 1e9:.0f} GB/s)")
        result["decode_multi"] = multi
    del ks, vs, k0, v0

    # ---------------------------------------------------------------- prefill (second half of metric)
    if not args.no_prefill:
        _log("generating prefill workload (1 x 8192 causal, 64/8 heads, bf16)")
        pre = workloads.make(3).prefill
        pairs = workloads.prefill_causal_pairs(pre)
        flops = 4.0 * dim * pre.q.shape[1] * pairs
        pq, pk, pv = pre.q.to(dev), pre.k.to(dev), pre.v.to(dev)
        ps, pcq, pck = pre.sinks.to(dev), pre.cu_seqlens_q.to(dev), pre.cu_seqlens_k.to(dev)
        pout = torch.empty_like(pq)

        def prefill(i):
            sa.prefill(pq, pk, pv, ps, pcq, pck, pre.scale, True, out=pout)

        for i in range(max(2, args.warmup // 2)):
            prefill(i)
        n_pre = max(5, args.steps // 2)
        ms_pre = _time_graph(_capture(prefill, n_pre, torch), n_pre, torch, replays=7)
        tflops = flops / (ms_pre * 1e-3) / 1e12
        _log(f"prefill {ms_pre * 1e3:.1f} us, {tflops:.1f} TFLOP/s")
        result["prefill"] = {
            "workload": "prefill_b1_s8192_hq64_hkv8_d64_causal",
            "ms_per_call": round(ms_pre, 4),
            "value": round(tflops, 2),
            "unit": "TFLOP/s",
            "roofline": {"bound": "mfma",
                         "kernel": sa.plan_prefill(pq, pk, pv, ps, pcq, pck, pre.scale, True)[0]["kernel"],
                         "achieved": round(tflops, 2),
                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                         "algorithmic_flop_per_launch": flops,
                         "measured_mfma_loop_tflops": ceilings["mfma_bf16_loop_tflops"] if ceilings else None,
                         "frac_of_measured_mfma_loop": (round(tflops / ceilings["mfma_bf16_loop_tflops"], 4)
                                                        if ceilings else None),
                         "measured_mfma_random_loop_tflops": (ceilings["mfma_bf16_random_loop_tflops"]
                                                              if ceilings else None),
                         "frac_of_measured_mfma_random_loop": (
                             round(tflops / ceilings["mfma_bf16_random_loop_tflops"], 4) if ceilings else None)},
        }

    # ---------------------------------------------------------------- split-KV (append) prefill
    if not args.no_prefill:
        # Chunked prefill: 512 new tokens against a 32768-key cache. Its 16 query tiles x 8 KV heads
        # are 128 work-groups, half a GPU; splitting the KV length 4 ways gives 512 (merged after).
        _log("generating append workload (512 new tokens x 32768 keys, 64/8 heads, bf16)")
        app = workloads.make_prefill([512], [32768], seed=1006)
        a_pairs = workloads.prefill_causal_pairs(app)
        a_flops = 4.0 * dim * app.q.shape[1] * a_pairs
        aq, ak, av = app.q.to(dev), app.k.to(dev), app.v.to(dev)
        as_, acq, ack = app.sinks.to(dev), app.cu_seqlens_q.to(dev), app.cu_seqlens_k.to(dev)
        aout = torch.empty_like(aq)
        splits = 4  # measured best on this shape: 2 -> 322 us, 4 -> 285 us, 8 -> 289 us, 16 -> 304 us
        apo = torch.empty((aq.shape[0], aq.shape[1], splits, dim), dtype=torch.float32, device=dev)
        apm = torch.empty((aq.shape[0], aq.shape[1], splits), dtype=torch.float32, device=dev)
        apd = torch.empty_like(apm)

        def app_plain(i):
            sa.prefill(aq, ak, av, as_, acq, ack, app.scale, True, out=aout)

        def app_split(i):
            sa.prefill_split(aq, ak, av, as_, acq, ack, app.scale, True, splits, apo, apm, apd)
            sa.decode_merge(apo, apm, apd, out=aout)

        n_app = max(5, args.steps // 2)
        ms_plain = _time_graph(_capture(app_plain, n_app, torch), n_app, torch, replays=5)
        ms_split = _time_graph(_capture(app_split, n_app, torch), n_app, torch, replays=5)
        _log(f"append prefill: unsplit {ms_plain * 1e3:.1f} us, {splits}-way KV split + merge "
             f"{ms_split * 1e3:.1f} us")
        result["prefill_append"] = {
            "workload": "prefill_append_q512_k32768_hq64_hkv8_d64_causal",
            "kv_splits": splits,
            "unsplit_us": round(ms_plain * 1e3, 2),
            "split_plus_merge_us": round(ms_split * 1e3, 2),
            "unsplit_tflops": round(a_flops / (ms_plain * 1e-3) / 1e12, 2),
            "split_tflops": round(a_flops / (ms_split * 1e-3) / 1e12, 2),
            "algorithmic_flop": a_flops,
        }

    # ---------------------------------------------------------------- long decode and mixed workloads
    if not args.no_long:
        # Long decode: 32 sequences of 16K-32K keys in a 32768-key cache, 16 chunks. Its K/V
        # (2 GiB allocated, ~1.6 GB read) exceed the Infinity Cache without rotation.
        _log("generating long-decode workload (32 x 16K-32K keys) and mixed workload")
        lc = workloads.make(4).decode
        l_bytes = workloads.decode_kv_bytes(lc) + lc.q.numel() * 2 * 2 + lc.sinks.numel() * 4
        lq, lk, lv = lc.q.to(dev), lc.k.to(dev), lc.v.to(dev)
        ls_, lsl = lc.sinks.to(dev), lc.seqlens_k.to(dev)
        lb, lhq = lc.q.shape[0], lc.q.shape[1]
        lpo = torch.empty((lb, lhq, lc.num_chunks, dim), dtype=torch.float32, device=dev)
        lpm = torch.empty((lb, lhq, lc.num_chunks), dtype=torch.float32, device=dev)
        lpd = torch.empty_like(lpm)
        lout = torch.empty((lb, lhq, dim), dtype=torch.bfloat16, device=dev)

        def long_step(i):
            sa.decode_split(lq, lk, lv, ls_, lsl, lc.num_chunks, lc.scale, lpo, lpm, lpd)
            sa.decode_merge(lpo, lpm, lpd, out=lout)

        long_step(0)
        ms_long = _time_graph(_capture(long_step, 20, torch), 20, torch)
        del lk, lv, lc
        # Mixed: 128 decode sequences of 1-8192 keys (8 chunks) and 16 prefill sequences.
        mx = workloads.make(5)
        md = mx.decode
        m_bytes = workloads.decode_kv_bytes(md) + md.q.numel() * 2 * 2 + md.sinks.numel() * 4
        mq, mk, mv, ms_, msl = (t.to(dev) for t in (md.q, md.k, md.v, md.sinks, md.seqlens_k))
        mb, mhq = md.q.shape[0], md.q.shape[1]
        mpo = torch.empty((mb, mhq, md.num_chunks, dim), dtype=torch.float32, device=dev)
        mpm = torch.empty((mb, mhq, md.num_chunks), dtype=torch.float32, device=dev)
        mpd = torch.empty_like(mpm)
        mout = torch.empty((mb, mhq, dim), dtype=torch.bfloat16, device=dev)

        def mixed_decode(i):
            sa.decode_split(mq, mk, mv, ms_, msl, md.num_chunks, md.scale, mpo, mpm, mpd)
            sa.decode_merge(mpo, mpm, mpd, out=mout)

        mp = mx.prefill
        m_flops = 4.0 * dim * mp.q.shape[1] * workloads.prefill_causal_pairs(mp)
        pq, pk, pv, ps, pcq, pck = (t.to(dev) for t in (mp.q, mp.k, mp.v, mp.sinks, mp.cu_seqlens_q, mp.cu_seqlens_k))
        pout = torch.empty_like(pq)

        def mixed_prefill(i):
            sa.prefill(pq, pk, pv, ps, pcq, pck, mp.scale, True, out=pout)

        mixed_decode(0)
        mixed_prefill(0)
        ms_md = _time_graph(_capture(mixed_decode, 20, torch), 20, torch)
        ms_mp = _time_graph(_capture(mixed_prefill, 5, torch), 5, torch, replays=10)
        _log(f"long decode {ms_long * 1e3:.1f} us ({l_bytes / (ms_long * 1e-3) / 1e9:.0f} GB/s); mixed decode "
             f"{ms_md * 1e3:.1f} us ({m_bytes / (ms_md * 1e-3) / 1e9:.0f} GB/s), mixed prefill {ms_mp * 1e3:.1f} us "
             f"({m_flops / (ms_mp * 1e-3) / 1e12:.0f} TFLOP/s)")
        result["decode_long"] = {
            "workload": "decode_b32_len16k_32k_cap32768_hq64_hkv8_d64_chunks16_outliers",
            "step_us": round(ms_long * 1e3, 2), "gbs": round(l_bytes / (ms_long * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(l_bytes / (ms_long * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": l_bytes, "target_us": 288.0,
        }
        result["mixed"] = {
            "workload": "decode_b128_len1_8192_chunks8 + prefill_16x512_4096_causal",
            "decode_step_us": round(ms_md * 1e3, 2), "decode_gbs": round(m_bytes / (ms_md * 1e-3) / 1e9, 1),
            "decode_algorithmic_bytes": m_bytes, "decode_target_us": 192.0,
            "prefill_us": round(ms_mp * 1e3, 2), "prefill_tflops": round(m_flops / (ms_mp * 1e-3) / 1e12, 1),
            "prefill_algorithmic_flop": m_flops, "prefill_target_us": 669.0,
        }
        del mk, mv, pk, pv, mx

    # ---------------------------------------------------------------- MoE routing softmax (detail)
    if not args.no_moe:
        tokens, experts, top_k = 65536, 128, 4
        gen = torch.Generator().manual_seed(1008)
        n_lsets = 8  # 8 x 16 MiB of logits: more than the Infinity Cache holds
        logit_sets = [torch.randn((tokens, experts), generator=gen).to(torch.bfloat16).to(dev)
                      for _ in range(n_lsets)]
        ids = torch.empty((tokens, top_k), dtype=torch.int32, device=dev)
        wts = torch.empty((tokens, top_k), dtype=torch.bfloat16, device=dev)

        def route(i):
            sa.moe_topk_softmax(logit_sets[i % n_lsets], top_k, ids=ids, weights=wts)

        route(0)
        ms_route = _time_graph(_capture(route, n_rep, torch), n_rep, torch)
        r_bytes = tokens * experts * 2 + tokens * top_k * (4 + 2)
        r_gbs = r_bytes / (ms_route * 1e-3) / 1e9
        _log(f"MoE routing {tokens} x {experts} top-{top_k}: {ms_route * 1e3:.2f} us ({r_gbs:.0f} GB/s)")
        result["moe_route"] = {
            "workload": "moe_topk_softmax_t65536_e128_k4_bf16",
            "us_per_call": round(ms_route * 1e3, 3),
            "gbs": round(r_gbs, 1),
            "frac_of_hbm_peak": round(r_gbs / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": r_bytes,
        }
        del logit_sets

    # ---------------------------------------------------------------- linear layers (detail)
    if not args.no_linear:
        gm = gn = gk = 4096
        gen = torch.Generator().manual_seed(1009)
        lx = torch.randn((gm, gk), generator=gen).to(torch.bfloat16).to(dev)
        lw = torch.randn((gn, gk), generator=gen).to(torch.bfloat16).to(dev)
        lb = torch.randn(gn, generator=gen).to(dev)
        ly = torch.empty((gm, gn), dtype=torch.bfloat16, device=dev)
        qx = (torch.randn((gm, gk), generator=gen) * 2).to(torch.float8_e4m3fn).to(dev)
        qw = (torch.randn((gn, gk), generator=gen) * 2).to(torch.float8_e4m3fn).to(dev)
        qsx = (torch.rand((gm, gk // 128), generator=gen) + 0.5).to(dev)
        qsw = (torch.rand((gn // 128, gk // 128), generator=gen) * 0.1 + 0.01).to(dev)
        n_lin = max(10, args.steps // 2)
        gflop = 2.0 * gm * gn * gk

        def lin_bf16(i):
            sa.linear_bias(lx, lw, lb, out=ly)

        def lin_fp8(i):
            sa.linear_fp8_block_scaled(qx, qsx, qw, qsw, lb, out=ly)

        def lin_torch(i):
            torch.nn.functional.linear(lx, lw, lb.to(torch.bfloat16))

        lin_bf16(0)
        lin_fp8(0)
        lin_torch(0)
        ms_lb = _time_graph(_capture(lin_bf16, n_lin, torch), n_lin, torch)
        ms_lf = _time_graph(_capture(lin_fp8, n_lin, torch), n_lin, torch)
        ms_lt = _time_graph(_capture(lin_torch, n_lin, torch), n_lin, torch)
        tf_b, tf_f, tf_t = (gflop / (ms * 1e-3) / 1e12 for ms in (ms_lb, ms_lf, ms_lt))
        _log(f"linear 4096^3: bf16+bias {ms_lb * 1e3:.1f} us ({tf_b:.0f} TFLOP/s), fp8 block-scaled "
             f"{ms_lf * 1e3:.1f} us ({tf_f:.0f} TFLOP/s); torch bf16 linear {ms_lt * 1e3:.1f} us ({tf_t:.0f})")
        result["linear"] = {
            "workload": "linear_m4096_n4096_k4096_bias",
            "bf16_us": round(ms_lb * 1e3, 2), "bf16_tflops": round(tf_b, 1),
            "bf16_frac_of_mfma_peak": round(tf_b / BF16_MFMA_PEAK_TFLOPS, 4),
            "fp8_block_scaled_us": round(ms_lf * 1e3, 2), "fp8_tflops": round(tf_f, 1),
            "fp8_frac_of_mfma_peak": round(tf_f / FP8_MFMA_PEAK_TFLOPS, 4),
            "torch_bf16_linear_us": round(ms_lt * 1e3, 2),
            "algorithmic_flop": gflop,
        }
        del lx, lw, qx, qw

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline:
        _log("timing the CPU oracle on the decode workload over the host cores (~10 s)")
        result["cpu_baseline"] = cpu_baseline()
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
