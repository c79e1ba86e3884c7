"""Benchmark of the MI355X retention library on one GPU.

Default workload (the `value`): chunkwise retention forward of the multi-scale
bf16 workload with rotation, B=2, H=8, N=2048, d_k=d_v=64, chunk 64. One step
is one retention_chunkwise_fwd call over the batch (rotation, intra-chunk
parallel form, state carry and, when the sequence is split, the segment
pre-pass and scan), inputs resident in HBM. The other workloads (7B-shaped
layer, batched decode, long context with the parallel-form crossover, the
single-head fp32 case) are measured after it and reported under "also".

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

Prints one JSON line. Timing uses HIP events on the stream the library
launches on (torch's current stream).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "retention fwd tokens/s & MFMA util (chunkwise); decode state-updates/s & HBM GB/s"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3


def chunk_alg_bytes(B, H, N, dk, dv, elt=2):
    """Algorithmic HBM bytes of one chunkwise forward: read q, k, v and write o once."""
    return B * H * N * elt * (2 * dk + dv + dv)


def chunk_alg_flops(B, H, N, dk, dv, C):
    """Algorithmic FLOPs: causal in-chunk Q K^T and P V, plus Q S and K^T V per token."""
    return B * H * N * ((C + 1) * (dk + dv) + 4 * dk * dv)


def parallel_alg_flops(B, H, N, dk, dv):
    return B * H * N * (N + 1) * (dk + dv)


def bwd_alg_bytes(B, H, N, dk, dv, elt=2):
    """Algorithmic HBM bytes of one backward: read q, k, v, dO; write dq, dk, dv."""
    return B * H * N * elt * (2 * dk + 2 * dv + 2 * dk + dv)


def decode_alg_bytes(B, H, dk, dv, elt=2):
    return B * H * (2 * dk * dv * 4 + elt * (2 * dk + dv) + elt * dv)


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
CSRC = "linear_attention_sequence_fwd_amd/csrc"
# the source file of each workload's dominant kernel; with the shared headers it
# decides that kernel's code (the traffic of the others is not affected by it)
KERNEL_SOURCES = {
    "layer7b_bf16": "chunk_wide.hip",
    "msr_bf16_rotary": "chunk_bf16.hip",
    "longctx_bf16": "chunk_wide.hip",
    "decode_bf16": "decode.hip",
}
SHARED_HEADERS = ("common.hpp", "tiles.hpp", "wide.hpp", "kernels.hpp")


def source_fingerprint(workload):
    """sha256 (first 16 hex digits) over the workload's kernel source and the shared headers."""
    import hashlib

    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), CSRC)
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[workload],) + SHARED_HEADERS:
        h.update(name.encode())
        with open(os.path.join(root, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of the workload's dominant kernel from the committed
    counter summary (profiles/hbm_traffic.json: FETCH_SIZE and WRITE_SIZE, each
    scaled by what it reads for a plain copy of known size), or None when that
    kernel's sources changed since the counters were taken."""
    path = os.path.join(PROFILES, "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    w = rec.get("workloads", {}).get(workload)
    if w is None or workload not in KERNEL_SOURCES or w.get("source_fingerprint") != source_fingerprint(workload):
        return None
    return w["read_bytes"] + w["write_bytes"]


def measured_dram(workload):
    """The same launch's bytes requested from memory (32-byte TCC_EA0 read and
    write requests to DRAM: what left the L2s; these counters cannot tell
    whether the memory-side cache served a request), or None like
    measured_traffic."""
    if measured_traffic(workload) is None:
        return None
    with open(os.path.join(PROFILES, "hbm_traffic.json")) as f:
        w = json.load(f)["workloads"][workload]
    return w.get("dram_read_bytes", 0) + w.get("dram_write_bytes", 0) if "dram_read_bytes" in w else None


def time_events(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per step


def time_phases(R, q, k, v, kw, steps):
    """Average duration (ms) of each kernel of the chunkwise call (segment
    pre-pass, segment scan, main pass), from start/stop events the library
    records around each kernel's execution (hipExtLaunchKernelGGL)."""
    import torch

    sets = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for evs in sets:
        R.retention_chunkwise_fwd(q, k, v, events=evs, **kw)
    torch.cuda.synchronize()
    tot = [0.0, 0.0, 0.0]
    for evs in sets:
        for i in range(3):
            tot[i] += evs[2 * i].elapsed_time(evs[2 * i + 1])
    return [t / steps for t in tot]


def time_graph(fn, steps, warmup, per_graph=20):
    """Per-step time with the step captured in a HIP graph and replayed, so host
    launch overhead is not in the measurement. Exactly `steps` steps are timed:
    the graph holds the largest divisor of `steps` that is <= per_graph, and an
    event between consecutive replays gives the per-step spread.
    Returns (mean ms per step over all timed steps, {p10, p50, p90} of the
    per-replay ms per step)."""
    import numpy as np
    import torch

    per = max(d for d in range(1, min(per_graph, steps) + 1) if steps % d == 0)
    reps = steps // per
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(warmup, 3)):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) / per for i in range(reps)])
    mean = ev[0].elapsed_time(ev[reps]) / steps
    pct = {f"p{q}": float(np.percentile(per_step, q)) for q in (10, 50, 90)}
    return mean, pct


def measured_peaks():
    """What this machine delivers on plain library work, beside the spec peaks:
    a 1 GiB device-to-device copy (HBM read + write) and a bf16 8192^3 matrix
    product (hipBLASLt through torch)."""
    import torch

    def timed(f, reps):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            f()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ms_copy = timed(lambda: dst.copy_(src), 20)
    del src, dst
    n = 8192
    x = torch.randn((n, n), dtype=torch.bfloat16, device="cuda:0")
    y = torch.randn((n, n), dtype=torch.bfloat16, device="cuda:0")
    ms_mm = timed(lambda: torch.mm(x, y), 10)
    del x, y
    torch.cuda.empty_cache()
    return {"copy_gbs": 2 * (1 << 30) / (ms_copy * 1e-3) / 1e9,
            "bf16_gemm_tflops": 2 * n ** 3 / (ms_mm * 1e-3) / 1e12,
            "how": "1 GiB device copy; torch.mm bf16 8192x8192x8192 (hipBLASLt)"}


# ---------------------------------------------------------------- CPU baseline (the fp64 oracle)
#
# The oracle runs in worker processes started before this process touches the
# GPU (spawn context), one head per task, single-threaded numpy each, so the
# host's cores work on independent heads. Each worker draws its inputs with the
# workloads' recipe on the CPU generator (same shapes, distributions and
# dtypes as the GPU inputs; the timing does not depend on the values).


def _oracle_task(kind, shape, seed, reps):
    """One timed oracle run in a worker: returns (seconds, units of work)."""
    import time as _t

    import numpy as np
    import torch

    from linear_attention_sequence_fwd_amd import workloads as W
    from oracle import retention as orc

    torch.set_num_threads(1)
    if kind == "recurrent":
        N, dk, dv, dtype, h, rot = shape
        q, k, v = W.make_qkv(1, 1, N, dk, dv, getattr(torch, dtype), seed)
        q64, k64, v64 = (x.float().numpy().astype(np.float64) for x in (q, k, v))
        g = orc.head_gammas(h + 1)[h:h + 1]
        th = W.rotary_theta(dk).double().numpy() if rot else None
        t0 = _t.perf_counter()
        for _ in range(reps):
            orc.recurrent(q64, k64, v64, g, theta=th)
        return _t.perf_counter() - t0, reps * N
    if kind == "decode":  # reps consecutive steps of one head
        dk, dv, h = shape
        s0, qs, ks, vs = W.make_decode(1, 1, dk, dv, torch.bfloat16, reps, 0.01, seed)
        st = s0.double().numpy()
        q64, k64, v64 = (x.float().numpy().astype(np.float64) for x in (qs, ks, vs))
        g = orc.head_gammas(h + 1)[h:h + 1]
        t0 = _t.perf_counter()
        for n in range(reps):
            _, st = orc.decode_step(q64[n], k64[n], v64[n], st, g)
        return _t.perf_counter() - t0, reps
    raise ValueError(kind)


def _oracle_worker_init():
    """Import what the oracle tasks use before any task is timed."""
    import numpy  # noqa: F401
    import torch

    from linear_attention_sequence_fwd_amd import workloads  # noqa: F401
    from oracle import retention  # noqa: F401

    torch.set_num_threads(1)


def host_cores():
    """Cores this process may use, capped at 16 (the host cores that come with one MI355X)."""
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def start_oracle_pool():
    """Worker pool for the CPU baseline, started before any GPU use (workers
    never touch the GPU; numpy/BLAS single-threaded in each)."""
    import multiprocessing as mp

    n = host_cores()
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        pool = mp.get_context("spawn").Pool(n, initializer=_oracle_worker_init)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return pool, n


def cpu_baselines(pool, cores):
    """The fp64 oracle on every workload, one head per worker task; per workload
    a bounded sample of heads (and of decode steps), scaled to the workload's
    unit. Returns {workload: {...}}."""
    import numpy as np

    from linear_attention_sequence_fwd_amd import workloads as W

    def run(tasks):
        """Runs the tasks (at most one per core at a time) and returns the job's
        time: each worker times its own oracle runs, and tasks that share a
        worker run one after another."""
        res = pool.starmap(_oracle_task, tasks, chunksize=1)
        per_core = sorted((r[0] for r in res), reverse=True)
        # tasks are dealt to `cores` workers: the job lasts as long as the busiest worker
        busy = [0.0] * cores
        for t in per_core:
            busy[busy.index(min(busy))] += t
        return max(busy), res

    out = {}
    # 7B-shaped layer: `cores` heads (of B*H = 64), full N; the job is B*H heads
    w = W.WORKLOADS["layer7b_bf16"]
    nh = min(cores, w["B"] * w["H"])
    wall, res = run([("recurrent", (w["N"], w["dk"], w["dv"], "bfloat16", i % w["H"], False), 100 + i, 1)
                     for i in range(nh)])
    job_s = wall * (w["B"] * w["H"]) / nh
    out["layer7b_bf16"] = {"value": w["B"] * w["N"] / job_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                           "sample": f"fp64 recurrent oracle on {nh} of the {w['B'] * w['H']} heads (full N="
                                     f"{w['N']}, d_k={w['dk']}, d_v={w['dv']}), one head per core, {wall:.1f} s "
                                     f"wall; whole-job time scaled by {w['B'] * w['H']}/{nh}",
                           "wall_s": wall, "cpu_s": float(sum(r[0] for r in res))}
    # multi-scale workload: all B*H = 16 heads, with rotation
    w = W.WORKLOADS["msr_bf16_rotary"]
    heads = w["B"] * w["H"]
    wall, res = run([("recurrent", (w["N"], w["dk"], w["dv"], "bfloat16", i % w["H"], True), 200 + i, 4)
                     for i in range(heads)])
    out["msr_bf16_rotary"] = {"value": 4 * w["B"] * w["N"] / wall, "unit": "tokens/s", "cores": cores,
                              "kind": "oracle", "sample": f"fp64 recurrent oracle with rotation, all {heads} heads, "
                                                          f"4 repetitions, {wall:.1f} s wall", "wall_s": wall}
    # long context: all 8 heads over the first 16384 tokens (the recurrent form is linear in N)
    w = W.WORKLOADS["longctx_bf16"]
    n = 16384
    wall, res = run([("recurrent", (n, w["dk"], w["dv"], "bfloat16", i, False), 300 + i, 1) for i in range(w["H"])])
    out["longctx_bf16"] = {"value": w["B"] * n / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                           "sample": f"fp64 recurrent oracle, all {w['H']} heads over the first {n} of "
                                     f"{w['N']} tokens, {wall:.1f} s wall", "wall_s": wall}
    # decode: 16 heads per core for 64 steps each (of 64 x 16 heads x 512 steps)
    w = W.WORKLOADS["decode_bf16"]
    nh = 16 * cores
    steps = 64
    wall, res = run([("decode", (w["dk"], w["dv"], i % w["H"]), 400 + i, steps) for i in range(nh)])
    out["decode_bf16"] = {"value": nh * steps / wall, "unit": "state updates/s", "cores": cores, "kind": "oracle",
                          "sample": f"fp64 decode-step oracle, {nh} of the {w['B'] * w['H']} heads for {steps} "
                                    f"consecutive steps each, {wall:.1f} s wall", "wall_s": wall}
    # single head fp32: the whole workload, one core (one head)
    w = W.WORKLOADS["single_head_f32"]
    wall, res = run([("recurrent", (w["N"], w["dk"], w["dv"], "float32", 0, False), 1, 50)])
    out["single_head_f32"] = {"value": 50 * w["N"] / wall, "unit": "tokens/s", "cores": 1, "kind": "oracle",
                              "sample": f"fp64 recurrent oracle, the whole workload 50 times, {wall:.2f} s wall",
                              "wall_s": wall}
    return out


def run_only(name, steps, warmup, dev):
    """One workload, timed with events; prints a short JSON line."""
    import torch

    import linear_attention_sequence_fwd_amd as R
    from linear_attention_sequence_fwd_amd import workloads as W

    if name == "copy":
        # plain device copy of a known size: calibrates HBM byte counters
        src = torch.ones(256 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        ms = time_events(lambda: dst.copy_(src), steps, warmup)
        print(json.dumps({"workload": "copy 1 GiB -> 1 GiB", "ms_per_call": ms, "bytes_read": src.numel() * 4,
                          "bytes_written": dst.numel() * 4}))
        return
    if name == "parallel":
        # the parallel form on the long-context heads at the longest crossover length
        w = W.WORKLOADS["longctx_bf16"]
        n = max(w["parallel_lengths"])
        q, k, v, _ = W.make_workload("longctx_bf16", device=dev)
        qn, kn, vn = q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous()
        del q, k, v
        out = torch.empty_like(vn)
        ms = time_events(lambda: R.retention_parallel_fwd(qn, kn, vn, out=out), steps, warmup)
        print(json.dumps({"workload": f"parallel form, B=1 H=8 N={n} d_k=d_v=128 bf16", "ms_per_call": ms,
                          "steps": steps}))
        return
    key = {"msr": "msr_bf16_rotary", "layer7b": "layer7b_bf16", "decode": "decode_bf16",
           "longctx": "longctx_bf16", "single": "single_head_f32", "bwd": "msr_bf16_rotary",
           "epi": "layer7b_bf16", "decmsr": "decode_bf16"}[name]
    w = W.WORKLOADS[key]
    if name == "bwd":
        fn = backward_step(R, W, key, dev)
        key = "msr_bf16_rotary backward"
    elif name == "epi":
        fn = epilogue_step(R, W, dev)
        key = "layer7b output stage"
    elif name == "decmsr":
        s0, qs, ks, vs = W.make_decode_workload(device=dev, steps=8)
        _, w_o, gw, gb, gt = W.make_epilogue(w["B"], w["H"], 1, w["dv"], 4096, 8, device=dev)
        gt = gt[:, 0, :].contiguous()
        it = iter(range(10 ** 9))

        def fn():
            t = next(it) % 8
            R.retention_recurrent_step_msr(qs[t], ks[t], vs[t], s0, w_o, gate=gt, gn_weight=gw, gn_bias=gb)
        key = "decode step + output stage"
    elif name == "decode":
        s0, qs, ks, vs = W.make_decode_workload(device=dev, steps=steps + warmup)
        o = torch.empty((w["B"], w["H"], w["dv"]), dtype=w["dtype"], device=dev)
        it = iter(range(steps + warmup))

        def fn():
            t = next(it)
            R.retention_recurrent_step(qs[t], ks[t], vs[t], s0, out=o)
    else:
        q, k, v, theta = W.make_workload(key, device=dev)
        out = torch.empty_like(v)
        ws_bytes = R.retention_chunkwise_workspace_size(w["B"], w["H"], w["N"], w["dk"], w["dv"], q.dtype,
                                                        w["chunk"])
        ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

        def fn():
            R.retention_chunkwise_fwd(q, k, v, chunk=w["chunk"], theta=theta, out=out, workspace=ws)
    ms = time_events(fn, steps, warmup)
    print(json.dumps({"workload": key, "ms_per_call": ms, "steps": steps}))


def backward_step(R, W, name, dev):
    """One retention_chunkwise_bwd call over a named workload (dO drawn once)."""
    import torch

    w = W.WORKLOADS[name]
    q, k, v, theta = W.make_workload(name, device=dev)
    d_o, _ = W.make_upstream_grads(w["B"], w["H"], w["N"], w["dk"], w["dv"], w["dtype"], w["seed"] + 1000,
                                   device=dev)
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    nbytes = R.retention_chunkwise_bwd_workspace_size(w["B"], w["H"], w["N"], w["dk"], w["dv"], q.dtype,
                                                      w["chunk"])
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    th = R.HostFloats(theta) if theta is not None else None

    def fn():
        R.retention_chunkwise_bwd(q, k, v, d_o, chunk=w["chunk"], theta=th, out=outs, workspace=ws)

    return fn


EPI_SHAPE = dict(B=4, H=16, N=8192, dv=512, d_out=4096)  # the 7B-shaped layer's heads into d_model 4096


def epilogue_step(R, W, dev):
    """One retention_msr_epilogue call on the 7B-shaped layer's outputs."""
    import torch

    e = EPI_SHAPE
    o, w_o, gw, gb, gt = W.make_epilogue(e["B"], e["H"], e["N"], e["dv"], e["d_out"], 7, device=dev)
    y = torch.empty((e["B"], e["N"], e["d_out"]), dtype=torch.bfloat16, device=dev)
    nbytes = R.retention_msr_epilogue_workspace_size(e["B"], e["H"], e["N"], e["dv"], e["d_out"], torch.bfloat16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def fn():
        R.retention_msr_epilogue(o, w_o, gn_weight=gw, gn_bias=gb, gate=gt, out=y, workspace=ws)

    return fn


def sweep_chunk(dev):
    """Chunkwise forward time against the chunk size (64 and 128: the kernel
    tile; larger: 128-token tiles with the state exchanged between chunks) on
    the multi-scale and long-context workloads: one JSON line per point."""
    import torch

    import linear_attention_sequence_fwd_amd as R
    from linear_attention_sequence_fwd_amd import workloads as W

    for name in ("msr_bf16_rotary", "longctx_bf16"):
        w = W.WORKLOADS[name]
        q, k, v, theta = W.make_workload(name, device=dev)
        th = R.HostFloats(theta) if theta is not None else None
        out = torch.empty_like(v)
        for C in (64, 128, 256, 512, 1024, 2048, 4096, 8192):
            if C >= w["N"]:
                break
            nb = R.retention_chunkwise_workspace_size(w["B"], w["H"], w["N"], w["dk"], w["dv"], q.dtype, C)
            ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device=dev)

            def fn():
                R.retention_chunkwise_fwd(q, k, v, chunk=C, theta=th, out=out, workspace=ws)

            ms, spread = time_graph(fn, 50 if w["N"] <= 4096 else 10, 5)
            # FLOPs the kernel does: its tile is min(C, 128) tokens
            fl = chunk_alg_flops(w["B"], w["H"], w["N"], w["dk"], w["dv"], min(C, 128))
            print(json.dumps({"sweep": "chunk", "workload": name, "chunk": C, "ms": ms, "ms_spread": spread,
                              "tokens_per_s": w["B"] * w["N"] / (ms * 1e-3),
                              "tile_tflops": fl / (ms * 1e-3) / 1e12}), flush=True)
        del q, k, v, out
        torch.cuda.empty_cache()


def sweep_decode_batch(dev):
    """Decode step latency against the number of sequences (H=16, 256x512 fp32
    state per head, bf16 q/k/v): one JSON line per batch size."""
    import torch

    import linear_attention_sequence_fwd_amd as R
    from linear_attention_sequence_fwd_amd import workloads as W

    H, dk, dv = 16, 256, 512
    for B in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        s0, qs, ks, vs = W.make_decode(B, H, dk, dv, torch.bfloat16, 8, 0.01, seed=B, device=dev)
        o = torch.empty((B, H, dv), dtype=torch.bfloat16, device=dev)
        it = [0]

        def fn():
            t = it[0] % 8
            it[0] += 1
            R.retention_recurrent_step(qs[t], ks[t], vs[t], s0, out=o)

        ms, spread = time_graph(fn, 100, 10)
        by = decode_alg_bytes(B, H, dk, dv)
        print(json.dumps({"sweep": "decode_batch", "B": B, "H": H, "dk": dk, "dv": dv, "ms_per_step": ms,
                          "ms_per_step_spread": spread, "state_updates_per_s": B * H / (ms * 1e-3),
                          "gbs": by / (ms * 1e-3) / 1e9, "hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}),
              flush=True)
        del s0, qs, ks, vs, o
        torch.cuda.empty_cache()


def time_kernel(R, q, k, v, kw, reps, evict=None, phases=False):
    """Durations (ms) of the chunkwise call's main kernel from the events the
    library records around its execution, one call at a time; with `evict`
    (a callable that writes 1 GiB) the caches are flushed before each call;
    with `phases`, the sum of its three phases (segment state pass, scan, main
    pass; a phase that does not run has zero length). Returns (median,
    {p10, p50, p90})."""
    import numpy as np
    import torch

    ts = []
    for i in range(reps + 2):
        if evict is not None:
            evict()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        R.retention_chunkwise_fwd(q, k, v, events=evs, **kw)
        torch.cuda.synchronize()
        if i >= 2:
            ts.append(sum(evs[j].elapsed_time(evs[j + 1]) for j in ((0, 2, 4) if phases else (4,))))
    ts = np.array(ts)
    return float(np.median(ts)), {f"p{p}": float(np.percentile(ts, p)) for p in (10, 50, 90)}


def make_evict(dev):
    """A 1 GiB device write: evicts the XCD L2 caches and the 256 MB MALL."""
    import torch

    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def evict():
        scratch.fill_(1.0)

    return evict, scratch


LAYER7B_DESC = ("7B-shaped retention layer forward, chunkwise: B=4 H=16 N=8192 d_k=256 d_v=512 bf16, "
                "gamma_h=1-2^(-5-h), chunk 128")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["msr", "layer7b", "decode", "longctx", "single", "copy", "bwd", "epi", "parallel",
                                       "decmsr"],
                    help="time one workload only (no CPU baseline); for profilers")
    ap.add_argument("--sweep", choices=["decode-batch", "chunk"], help="print one JSON line per point of a sweep")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(sequence and head sharding across GPUs is a design note, not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    pool = cores = None
    if not (args.only or args.sweep or args.no_cpu):
        pool, cores = start_oracle_pool()  # before the first GPU call

    import linear_attention_sequence_fwd_amd as R
    from linear_attention_sequence_fwd_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    R.load_library()
    dev = "cuda:0"
    if args.only:
        run_only(args.only, args.steps, args.warmup, dev)
        return
    if args.sweep == "decode-batch":
        sweep_decode_batch(dev)
        return
    if args.sweep == "chunk":
        sweep_chunk(dev)
        return

    # ---------------- headline: the 7B-shaped layer
    name = "layer7b_bf16"
    w = W.WORKLOADS[name]
    q, k, v, _ = W.make_workload(name, device=dev)
    out = torch.empty_like(v)
    kw = dict(chunk=w["chunk"], out=out)
    step = lambda: R.retention_chunkwise_fwd(q, k, v, **kw)  # noqa: E731
    ms_eager = time_events(step, args.steps, args.warmup)
    ms, spread = time_graph(step, args.steps, args.warmup)
    kernel_ms, kspread = time_kernel(R, q, k, v, kw, max(20, args.steps // 4))
    flops = chunk_alg_flops(w["B"], w["H"], w["N"], w["dk"], w["dv"], w["chunk"])
    nbytes = chunk_alg_bytes(w["B"], w["H"], w["N"], w["dk"], w["dv"])
    tflops = flops / (kernel_ms * 1e-3) / 1e12
    gbs = nbytes / (kernel_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": w["B"] * w["N"] / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": LAYER7B_DESC, "global_batch": w["B"], "seq_len": w["N"],
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "kernel": "chunk_wide_kernel<256> (the whole step is this one launch)",
            "achieved": tflops,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / BF16_PEAK_TFLOPS,
            "traffic": measured_traffic(name),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x copy calibration + WRITE_SIZE)",
            "dram_traffic": measured_dram(name),
            "alg_flops_per_launch": flops,
            "alg_bytes_per_launch": nbytes,
            "kernel_ms": kernel_ms,
            "kernel_ms_spread": kspread,
            "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS},
            "binding": "HBM by arithmetic intensity (198.8 FLOP/B against a ridge of 312.5): the MFMA fraction "
                       "at the HBM roofline is 0.636",
        },
        "timing": "ms_per_step from HIP-graph replay of exactly `steps` steps (up to 20 per graph, an event "
                  "between replays for the spread); eager_ms_per_step launches each call from Python; "
                  "kernel_ms is the kernel's own duration from events recorded around its execution",
        "ms_per_step_spread": spread,
        "eager_ms_per_step": ms_eager,
    }
    del q, k, v, out
    torch.cuda.empty_cache()
    result["measured_peaks"] = measured_peaks()

    also = []
    if not args.quick:
        also = run_also(R, W, torch, dev)
    if pool is not None:
        cpu = cpu_baselines(pool, cores)
        pool.close()
        pool.join()
        result["cpu_baseline"] = cpu.pop("layer7b_bf16")
        for entry in also:
            key = entry.get("key")
            if key in cpu:
                entry["cpu_baseline"] = cpu[key]
    for entry in also:
        entry.pop("key", None)
    if also:
        result["also"] = also
    print(json.dumps(result))


def run_also(R, W, torch, dev):
    also = []
    evict, scratch = make_evict(dev)

    # ---------------- multi-scale workload with rotation (warm and cold caches)
    name = "msr_bf16_rotary"
    w = W.WORKLOADS[name]
    q, k, v, theta = W.make_workload(name, device=dev)
    out = torch.empty_like(v)
    ws_bytes = R.retention_chunkwise_workspace_size(w["B"], w["H"], w["N"], w["dk"], w["dv"], q.dtype, w["chunk"])
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    kw = dict(chunk=w["chunk"], theta=R.HostFloats(theta), out=out, workspace=ws)
    ms2, sp2 = time_graph(lambda: R.retention_chunkwise_fwd(q, k, v, **kw), 200, 20)
    warm_ms, warm_sp = time_kernel(R, q, k, v, kw, 50)
    cold_ms, cold_sp = time_kernel(R, q, k, v, kw, 20, evict=evict)
    by2 = chunk_alg_bytes(w["B"], w["H"], w["N"], w["dk"], w["dv"])
    also.append({
        "key": name,
        "workload": "multi-scale retention forward, chunkwise: B=2 H=8 N=2048 d_k=d_v=64 bf16, rotary "
                    "theta_j=10000^(-2j/64), gamma_h=1-2^(-5-h), chunk 64",
        "tokens_per_s": w["B"] * w["N"] / (ms2 * 1e-3), "ms": ms2, "ms_spread": sp2,
        "kernel_ms_warm": warm_ms, "kernel_ms_warm_spread": warm_sp,
        "kernel_ms_cold": cold_ms, "kernel_ms_cold_spread": cold_sp,
        "cold": "a 1 GiB device write before each call evicts the L2 caches and the 256 MB MALL",
        "roofline": {"bound": "hbm", "kernel": "chunk_bf16_kernel<64, 64, 64, local pass>",
                     "achieved": by2 / (warm_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": by2 / (warm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "frac_cold": by2 / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic(name), "dram_traffic": measured_dram(name),
                     "alg_bytes_per_launch": by2},
    })
    del q, k, v, out, ws
    torch.cuda.empty_cache()

    # ---------------- decode
    name = "decode_bf16"
    w = W.WORKLOADS[name]
    s0, qs, ks, vs = W.make_decode_workload(device=dev)
    state = s0.clone()
    o = torch.empty((w["B"], w["H"], w["dv"]), dtype=torch.bfloat16, device=dev)
    steps = w["steps"]

    def run_decode():
        for t in range(steps):
            R.retention_recurrent_step(qs[t], ks[t], vs[t], state, out=o)

    ms4 = time_events(run_decode, 2, 1) / steps
    by4 = decode_alg_bytes(w["B"], w["H"], w["dk"], w["dv"])
    also.append({
        "key": name,
        "workload": "recurrent decode: 64 sequences x H=16, fp32 state 256x512, bf16 q/k/v, 512 steps",
        "ms_per_step": ms4, "state_updates_per_s": w["B"] * w["H"] / (ms4 * 1e-3),
        "roofline": {"bound": "hbm", "kernel": "recurrent_step_kernel", "achieved": by4 / (ms4 * 1e-3) / 1e9,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": by4 / (ms4 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic(name), "dram_traffic": measured_dram(name),
                     "alg_bytes_per_launch": by4},
    })
    del s0, qs, ks, vs, state, o
    torch.cuda.empty_cache()

    # ---------------- long context + parallel crossover
    name = "longctx_bf16"
    w = W.WORKLOADS[name]
    q, k, v, _ = W.make_workload(name, device=dev)
    kw5 = dict(chunk=w["chunk"])
    ms5 = time_events(lambda: R.retention_chunkwise_fwd(q, k, v, **kw5), 10, 3)
    k5, _ = time_kernel(R, q, k, v, kw5, 5, phases=True)
    by5 = chunk_alg_bytes(w["B"], w["H"], w["N"], w["dk"], w["dv"])
    fl5 = chunk_alg_flops(w["B"], w["H"], w["N"], w["dk"], w["dv"], w["chunk"])
    cross = []
    for n in w["parallel_lengths"]:
        qn, kn, vn = q[:, :, :n].contiguous(), k[:, :, :n].contiguous(), v[:, :, :n].contiguous()
        tp = time_events(lambda: R.retention_parallel_fwd(qn, kn, vn), 20, 5)
        tc = time_events(lambda: R.retention_chunkwise_fwd(qn, kn, vn, chunk=w["chunk"]), 20, 5)
        pf = parallel_alg_flops(w["B"], w["H"], n, w["dk"], w["dv"])
        cross.append({"N": n, "parallel_ms": tp, "chunkwise_ms": tc, "parallel_tflops": pf / (tp * 1e-3) / 1e12,
                      "parallel_mfma_frac": pf / (tp * 1e-3) / 1e12 / BF16_PEAK_TFLOPS})
    also.append({
        "key": name,
        "workload": "long-context chunkwise: B=1 H=8 N=65536 d_k=d_v=128 bf16, chunk 128",
        "tokens_per_s": w["B"] * w["N"] / (ms5 * 1e-3), "ms": ms5, "kernel_ms": k5,
        "roofline": {"bound": "hbm", "kernel": "chunk_wide_state_kernel<128> + segment_scan_kernel + "
                               "chunk_wide_seg_kernel<128> (32 segments; kernel_ms sums the three)",
                     "achieved": by5 / (k5 * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": by5 / (k5 * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": measured_traffic(name),
                     "dram_traffic": measured_dram(name),
                     "alg_bytes_per_launch": by5, "tflops": fl5 / (k5 * 1e-3) / 1e12},
        "parallel_crossover": cross,
    })
    del q, k, v
    torch.cuda.empty_cache()

    # ---------------- backward of the multi-scale workload
    w = W.WORKLOADS["msr_bf16_rotary"]
    bstep = backward_step(R, W, "msr_bf16_rotary", dev)
    msb, spb = time_graph(bstep, 100, 10)
    flb = 3 * chunk_alg_flops(w["B"], w["H"], w["N"], w["dk"], w["dv"], w["chunk"])
    byb = bwd_alg_bytes(w["B"], w["H"], w["N"], w["dk"], w["dv"])
    also.append({
        "workload": "backward of the multi-scale workload (dq, dk, dv; rotation; B=2 H=8 N=2048 d=64 "
                    "bf16, chunk 64): a row kernel (rotated K, Q), then the three chunkwise passes in one "
                    "launch (dq, dk rotated back as they are stored)",
        "ms": msb, "ms_spread": spb, "tokens_per_s": w["B"] * w["N"] / (msb * 1e-3),
        "tflops": flb / (msb * 1e-3) / 1e12, "mfma_frac": flb / (msb * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "gbs": byb / (msb * 1e-3) / 1e9, "alg_bytes": byb, "alg_flops": flb,
    })
    del bstep
    torch.cuda.empty_cache()

    # ---------------- backward of the long-context workload
    w = W.WORKLOADS["longctx_bf16"]
    bstep = backward_step(R, W, "longctx_bf16", dev)
    msl = time_events(bstep, 5, 2)
    fll = 3 * chunk_alg_flops(w["B"], w["H"], w["N"], w["dk"], w["dv"], w["chunk"])
    also.append({
        "workload": "backward of the long-context workload (B=1 H=8 N=65536 d=128 bf16, chunk 128): the three passes on the segmented wide kernel (state passes, scans, segment passes: one launch each)",
        "ms": msl, "tokens_per_s": w["B"] * w["N"] / (msl * 1e-3), "tflops": fll / (msl * 1e-3) / 1e12,
        "mfma_frac": fll / (msl * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
    })
    del bstep
    torch.cuda.empty_cache()

    # ---------------- backward of the 7B-shaped layer
    w = W.WORKLOADS["layer7b_bf16"]
    bstep = backward_step(R, W, "layer7b_bf16", dev)
    ms7 = time_events(bstep, 3, 1)
    fl7 = (4 * chunk_alg_flops(w["B"], w["H"], w["N"], w["dv"] // 2, w["dk"], w["chunk"]) +
           chunk_alg_flops(w["B"], w["H"], w["N"], w["dk"], w["dv"], w["chunk"]))
    also.append({
        "workload": "backward of the 7B-shaped layer (B=4 H=16 N=8192 d_k=256 d_v=512 bf16, chunk 128): "
                    "passes 1 and 2 over the two halves of d_v, pass 3 at full width",
        "ms": ms7, "tokens_per_s": w["B"] * w["N"] / (ms7 * 1e-3), "tflops": fl7 / (ms7 * 1e-3) / 1e12,
        "mfma_frac": fl7 / (ms7 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
    })
    del bstep
    torch.cuda.empty_cache()

    # ---------------- output stage of the 7B-shaped layer
    e = EPI_SHAPE
    estep = epilogue_step(R, W, dev)
    mse = time_events(estep, 10, 3)
    fle = 2.0 * e["B"] * e["N"] * e["H"] * e["dv"] * e["d_out"]
    also.append({
        "workload": "output stage of the 7B-shaped layer: GroupNorm (16 heads of 512) + gate + W_O "
                    "(8192 -> 4096) over 32768 tokens, bf16",
        "ms": mse, "tokens_per_s": e["B"] * e["N"] / (mse * 1e-3), "tflops": fle / (mse * 1e-3) / 1e12,
        "mfma_frac": fle / (mse * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, "alg_flops": fle,
    })
    del estep
    torch.cuda.empty_cache()

    # ---------------- decode step + output stage (one token per sequence through the layer's W_O)
    w = W.WORKLOADS["decode_bf16"]
    s0, qs, ks, vs = W.make_decode_workload(device=dev, steps=8)
    _, w_o, gw, gb, gt = W.make_epilogue(w["B"], w["H"], 1, w["dv"], 4096, 8, device=dev)
    gt = gt[:, 0, :].contiguous()
    yd = torch.empty((w["B"], 4096), dtype=torch.bfloat16, device=dev)
    od = torch.empty((w["B"], w["H"], w["dv"]), dtype=torch.bfloat16, device=dev)
    itd = [0]

    def dstep():
        t = itd[0] % 8
        itd[0] += 1
        R.retention_recurrent_step_msr(qs[t], ks[t], vs[t], s0, w_o, gate=gt, gn_weight=gw, gn_bias=gb, o=od,
                                       out=yd)

    msd, spd = time_graph(dstep, 100, 10)
    itd[0] = 0

    def ostep():
        R.retention_msr_epilogue(od.view(w["B"], w["H"], 1, w["dv"]), w_o, gn_weight=gw, gn_bias=gb,
                                 gate=gt.view(w["B"], 1, -1), out=yd.view(w["B"], 1, 4096))

    mso, _ = time_graph(ostep, 100, 10)
    wbytes = 4096 * w["H"] * w["dv"] * 2
    also.append({
        "workload": "decode step + output stage: 64 sequences x H=16 (state 256x512) -> GroupNorm, gate, "
                    "W_O 8192 -> 4096, bf16",
        "ms_per_token_step": msd, "spread": spd, "output_stage_ms": mso,
        "output_stage_w_o_gbs": wbytes / (mso * 1e-3) / 1e9,
    })
    del s0, qs, ks, vs, w_o, gw, gb, gt, yd, od
    torch.cuda.empty_cache()

    # ---------------- single-head fp32 (warm and cold caches)
    name = "single_head_f32"
    q, k, v, _ = W.make_workload(name, device=dev)
    kw1 = dict(chunk=64)
    ms1 = time_events(lambda: R.retention_chunkwise_fwd(q, k, v, **kw1), 50, 5)
    msp = time_events(lambda: R.retention_parallel_fwd(q, k, v), 50, 5)
    c1_warm, _ = time_kernel(R, q, k, v, kw1, 20)
    c1_cold, _ = time_kernel(R, q, k, v, kw1, 10, evict=evict)
    also.append({"key": name, "workload": "single-head fp32 B=1 H=1 N=256 d=64", "chunkwise_ms": ms1,
                 "parallel_ms": msp, "main_kernel_ms_warm": c1_warm, "main_kernel_ms_cold": c1_cold})
    del q, k, v, scratch
    torch.cuda.empty_cache()
    return also


if __name__ == "__main__":
    main()
