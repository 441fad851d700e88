"""Benchmark: fused attention forward on one MI355X, long-context causal workload by default.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--pass fwd|bwd] [--no-cpu-baseline]
                    [--cold] [--graph] [--cpu-threads N]
    python bench.py --gemm-reference N   (vendor bf16 GEMM rate, for scale)

One step = one call of the whole hot path (attn_fwd over one batch of synthetic input already
resident in HBM; attn_decode, key splits and merge, for the KV-cache decode workloads, whose
line reports HBM GB/s against the 8 TB/s peak instead of TFLOP/s; with --pass bwd, one call of
attn_bwd, both of its kernels, on the forward's O and LSE and a seeded dO).  W untimed warm-up steps, then K timed steps bracketed by device
synchronisation, timed with HIP events recorded on the stream the kernel is launched on.
Prints ONE JSON line on stdout (everything else goes to stderr).

--graph captures one step in a HIP graph and times replays of it: the per-step time then holds
no host launch cost (what a serving loop that replays graphs pays for the tiny cases).
--cold reads a 512 MiB buffer before every step (outside the step's event pair), which evicts
the L2 caches and the 256 MB MALL and leaves only clean lines in them (a write would leave dirty
lines whose write-back then competes with the step's reads); the line then reports the median
per-launch time instead of the region average, since the region holds the flushes.  Every line
also gives the median and minimum per-launch times and the device memory the steps allocated
(torch's peak counter and the driver's free-memory count, both expected unchanged: the library
allocates nothing).

The CPU baseline times the fp64 oracle, untouched, on a bounded random sample of the same
workload's rows and scales it to the same unit; the same rows are compared with the GPU
output.  Only this leg loads the oracle.  --cpu-threads N limits it to N OpenMP threads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (4·B·H·N²·D, causal halved) and % of bf16 MFMA peak"
METRIC_WINDOW = "sliding-window attention fwd TFLOP/s (4·D per (query, key) pair inside the band)"
METRIC_DECODE = "KV-cache decode attention HBM GB/s (Q, valid K/V rows, O and LSE bytes per step)"
METRIC_BWD = "attention bwd TFLOP/s (2.5 x the forward's 4·B·H·N²·D, causal halved: five N²·D products)"
# MI355X published dense peaks (256 CUs at 2.4 GHz).
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["attn_common.h", "attn_fwd_api.hip", "attn_fwd_mfma.hip", "attn_fwd_f32.hip", "attn_merge.hip"]
BWD_KERNEL_SOURCES = ["attn_common.h", "attn_bwd.h", "attn_bwd_api.hip", "attn_bwd_mfma.hip", "attn_bwd_f32.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for fn in sources:
        with open(os.path.join(ROOT, "transformer_scaled_dot_amd", "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def read_traffic(workload: str, src_hash: str, family: str = "attn_fwd"):
    """HBM bytes per step measured by rocprofv3 counters (profiles/<family>_<workload>_traffic.md),
    if they were taken on the current kernel sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"{family}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != src_hash:
        return None
    return float(m_bytes.group(1))


def algorithmic_bytes(w, key_lens=None) -> float:
    """Bytes one step must move at least: Q and O, K and V once (their valid rows when key
    lengths are given), LSE in fp32."""
    eb = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    kv_rows = w.B * w.Nk if key_lens is None else \
        int(sum(min(max(int(n), 0), w.Nk) for n in key_lens))
    return eb * (2 * w.B * w.H * w.Nq * w.D + 2 * w.H * kv_rows * w.D) + 4 * w.B * w.H * w.Nq


def bwd_algorithmic_bytes(w) -> float:
    """Backward: read Q, K, V, O, dO and LSE once, write dQ, dK, dV once."""
    eb = {"f32": 4, "f16": 2, "bf16": 2}[w.dtype]
    nq, nk = w.B * w.H * w.Nq * w.D, w.B * w.H * w.Nk * w.D
    return eb * (4 * nq + 4 * nk) + 4 * w.B * w.H * w.Nq


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_bwd(w, x, do, grads, target_s: float, seed: int = 1234, nthreads: int = 0):
    """Time the oracle's backward on whole (b, h) slices (random, growing until ~target_s / 2)."""
    import numpy as np

    import oracle

    impl = oracle.default()
    cores = nthreads if nthreads > 0 else impl.max_threads()
    rng = np.random.default_rng(seed)
    order = rng.permutation(w.B * w.H)
    args = (x["q"], x["k"], x["v"], do, w.dtype, float(x["scale"]), w.causal, x["key_lens"])
    n, spent, done = 1, 0.0, []
    wkw = {} if w.window is None else {"window": w.window}
    while True:
        sel = order[len(done):len(done) + n]
        if sel.size == 0:
            break
        t0 = time.perf_counter()
        want = impl.attn_bwd(*args, None, sel, nthreads=nthreads, **wkw)
        spent += time.perf_counter() - t0
        done.append((sel, want))
        if spent >= 0.5 * target_s:
            break
        n = max(1, min(16, n * 2))
    slices = np.concatenate([d[0] for d in done])
    kl = x["key_lens"]
    pairs = 0
    for bh in slices:
        L = w.Nk if kl is None else int(np.clip(kl[bh // w.H], 0, w.Nk))
        pairs += int(row_pairs(w, np.arange(w.Nq, dtype=np.int64), None if kl is None else
                               np.full(w.B, L, np.int32)).sum())
    flops = 2.5 * 4.0 * w.D * pairs
    errs = []
    for sel, want in done:
        for name, got, ref in zip(("dq", "dk", "dv"), grads, want):
            g = got.detach().reshape(-1, *got.shape[2:])[np.asarray(sel)].double().cpu().numpy()
            errs.append(float(np.max(np.abs(g - ref)) / max(float(np.max(np.abs(ref))), 1e-30)))
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{slices.size} random (b, h) slices of the same workload (seed {seed}), fp64 oracle "
                  f"backward with {cores} OpenMP threads, {spent:.2f} s; flops counted as 2.5 x 4*D per "
                  f"visible (query, key) pair, as in the metric",
        "seconds": spent,
        "sample_max_rel_err_grads": max(errs),
    }


def oracle_causal(w) -> int:
    """The oracle's mask code: 2 puts the queries at the end of each key sequence."""
    return 2 if (w.causal and w.kv_cache) else int(w.causal)


def row_pairs(w, rows, key_lens):
    """Number of (query, valid key) pairs of each flat row id."""
    import numpy as np

    i = rows % w.Nq
    b = rows // (w.H * w.Nq)
    L = np.full(rows.shape, w.Nk, dtype=np.int64) if key_lens is None else \
        np.clip(key_lens.astype(np.int64), 0, w.Nk)[b]
    if w.kv_cache:
        return np.clip(i + 1 + L - w.Nq, 0, L) if w.causal else L
    hi = np.minimum(L, i + 1) if w.causal else L
    if w.window is None:
        return hi
    hi = np.minimum(hi, i + w.window + 1)
    return np.maximum(hi - np.maximum(i - w.window, 0), 0)


def cpu_baseline(w, x, o_dev, lse_dev, target_s: float, seed: int = 1234, nthreads: int = 0):
    """Time the oracle on a random sample of rows (pilot run, then ~target_s of work)."""
    import numpy as np
    import torch

    import oracle

    impl = oracle.default()
    cores = nthreads if nthreads > 0 else impl.max_threads()
    rng = np.random.default_rng(seed)
    total = w.B * w.H * w.Nq
    args = (x["q"], x["k"], x["v"], w.dtype, float(x["scale"]), oracle_causal(w), x["key_lens"])

    # Size the sample from a timed pilot, growing it until it covers at least half the target.
    n = 256
    while True:
        n = min(n, total)
        rows = np.sort(rng.choice(total, size=n, replace=False)) if n < total else np.arange(total)
        t0 = time.perf_counter()
        ro, rl = impl.attn_rows(*args, rows=rows, nthreads=nthreads, window=w.window)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or n >= total:
            break
        n = int(n * min(64.0, max(2.0, target_s / max(dt, 1e-3))))
    reps = 1
    if n >= total and dt < 0.5 * target_s:  # the whole workload is small: time repeats of it
        reps = max(1, int(0.5 * target_s / max(dt, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            ro, rl = impl.attn_rows(*args, rows=rows, nthreads=nthreads, window=w.window)
        dt = (time.perf_counter() - t0) / reps
    pairs = float(row_pairs(w, rows, x["key_lens"]).sum())
    flops = 4.0 * w.D * pairs

    D = w.D
    o = o_dev.detach().reshape(-1, D)[torch.from_numpy(rows).to(o_dev.device)].double().cpu().numpy()
    lse = lse_dev.detach().reshape(-1)[torch.from_numpy(rows).to(o_dev.device)].double().cpu().numpy()
    fin = np.isfinite(rl)
    err_o = float(np.max(np.abs(o - ro)))
    err_l = float(np.max(np.abs(lse[fin] - rl[fin]))) if fin.any() else 0.0
    if w.kv_cache:  # the metric's unit: the step's algorithmic bytes, prorated by visible pairs
        all_rows = np.arange(total, dtype=np.int64)
        share = pairs / max(float(row_pairs(w, all_rows, x["key_lens"]).sum()), 1.0)
        value, unit = algorithmic_bytes(w, x["key_lens"]) * share / dt / 1e9, "GB/s"
        counted = "bytes counted as the step's algorithmic bytes times the sample's share of the " \
                  "visible (query, key) pairs, as in the metric"
    else:
        value, unit = flops / dt / 1e12, "TFLOP/s"
        counted = "flops counted as 4*D per valid (query, key) pair, as in the metric"
    return {
        "value": value,
        "unit": unit,
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{rows.size} random query rows of the same workload (seed {seed}), fp64 oracle "
                  f"with {cores} OpenMP threads, {dt:.3f} s per pass ({reps} passes); {counted}",
        "seconds": dt,
        "sample_max_abs_err_o": err_o,
        "sample_max_abs_err_lse": err_l,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the backward (attn_bwd)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-threads", type=int, default=0, help="OpenMP threads of the CPU baseline (0: all)")
    ap.add_argument("--gemm-reference", type=int, default=0, metavar="N",
                    help="instead of attention, time torch's bf16 N x N x N matmul (the vendor GEMM) "
                         "as a reference for what dense MFMA work sustains on this GPU")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time replays of it (no host launch cost)")
    ap.add_argument("--cold", action="store_true",
                    help="evict L2 and MALL (512 MiB read) before every step; report the median launch time")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(reference dispatch for HBM byte counters)")
    a = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py: the library runs on exactly one GPU (asked for --gpus {a.gpus}, "
              f"WORLD_SIZE={world}); heads shard across GPUs with no communication, but no "
              f"multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from transformer_scaled_dot_amd import binding, inputs

    if a.gemm_reference > 0:
        n = a.gemm_reference
        x0 = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        x1 = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(a.warmup):
            torch.matmul(x0, x1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(a.steps):
            torch.matmul(x0, x1)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / a.steps
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"metric": "reference: vendor bf16 GEMM TFLOP/s (torch.matmul)", "value": tf,
                          "unit": "TFLOP/s", "ms_per_step": ms, "steps": a.steps, "warmup": a.warmup,
                          "config": {"workload": f"gemm_bf16_{n}x{n}x{n}"},
                          "frac_of_peak": tf / PEAK_TFLOPS["bf16"]}), flush=True)
        return

    name = a.workload or inputs.BENCH_WORKLOAD
    w = inputs.WORKLOADS[name]
    log(f"[bench] workload {name}: generating inputs")
    t0 = time.perf_counter()
    x = inputs.make_inputs(w)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s")

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    def to_dev(arr):
        t = torch.from_numpy(np.ascontiguousarray(arr))
        if w.dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(dev)

    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    kl = None if x["key_lens"] is None else torch.from_numpy(x["key_lens"]).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    scale = float(x["scale"])

    # The tensor-level wrappers check every argument on each call; a decode step is only tens of
    # microseconds of GPU work, so the timed loop calls the C entry points directly with the
    # arguments marshalled once (after one checked call through the wrapper).
    code = inputs.DTYPE_CODE[w.dtype]
    kl_ptr = None if kl is None else kl.data_ptr()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())
    dims = (w.B, w.H, w.Nq, w.Nk, w.D, scale, int(w.causal))
    lib = binding.load_library()
    bwd = a.which == "bwd"
    if bwd:
        if w.kv_cache:
            raise SystemExit(f"bench.py: the backward takes workloads without a KV cache ({name})")
        binding.fwd(q, k, v, causal=w.causal, key_lens=kl, scale=scale, out=o, lse=lse, stream=stream,
                    window=w.window)
        do_np = inputs.make_grad_out(w)
        do = to_dev(do_np)
        grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        ws_bytes = binding.attn_bwd_workspace_size(w.B, w.H, w.Nq)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        binding.bwd(q, k, v, o, lse, do, causal=w.causal, key_lens=kl, scale=scale, dq=grads[0],
                    dk=grads[1], dv=grads[2], workspace=workspace, stream=stream, window=w.window)
        win = -1 if w.window is None else min(int(w.window), 2**31 - 1)
        args = (*ptrs[:4], do.data_ptr(), lse.data_ptr(), None, *(t.data_ptr() for t in grads), *dims,
                win, kl_ptr, code, workspace.data_ptr(), ws_bytes, stream.cuda_stream)

        def step(handle=None):  # handle: the stream to enqueue on (default: the bench's stream)
            rc = lib.attn_bwd_window(*args[:-1], args[-1] if handle is None else handle)
            if rc != binding.ATTN_OK:
                raise binding.AttnError(rc)
    elif w.kv_cache:
        ws_bytes = binding.attn_decode_workspace_size(w.B, w.H, w.Nq, w.Nk, w.D, code)
        workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        log(f"[bench] decode workspace {ws_bytes} bytes")
        binding.decode(q, k, v, causal=w.causal, key_lens=kl, scale=scale, out=o, lse=lse,
                       workspace=workspace, stream=stream)
        args = (*ptrs, *dims, kl_ptr, code, workspace.data_ptr(), ws_bytes, stream.cuda_stream)

        def step(handle=None):  # handle: the stream to enqueue on (default: the bench's stream)
            rc = lib.attn_decode(*args[:-1], args[-1] if handle is None else handle)
            if rc != binding.ATTN_OK:
                raise binding.AttnError(rc)
    else:
        binding.fwd(q, k, v, causal=w.causal, key_lens=kl, scale=scale, out=o, lse=lse,
                    stream=stream, window=w.window)
        win = -1 if w.window is None else min(int(w.window), 2**31 - 1)
        args = (*ptrs, *dims, win, kl_ptr, code, stream.cuda_stream)

        def step(handle=None):  # handle: the stream to enqueue on (default: the bench's stream)
            rc = lib.attn_fwd_window(*args[:-1], args[-1] if handle is None else handle)
            if rc != binding.ATTN_OK:
                raise binding.AttnError(rc)

    if a.graph:
        # One step captured on a side stream; replays then run on the bench's stream.  The entry
        # points enqueue only kernels (no allocation, memset or host synchronisation), so a
        # captured call replays exactly.
        eager_step = step
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            eager_step(side.cuda_stream)
        stream.wait_stream(side)
        torch.cuda.synchronize(dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            eager_step(torch.cuda.current_stream(dev).cuda_stream)
        torch.cuda.synchronize(dev)

        def step(handle=None):
            graph.replay()
        log("[bench] timing replays of a captured HIP graph of one step")
    flush = torch.zeros(128 << 20, dtype=torch.float32, device=dev) if a.cold else None  # 512 MiB
    for _ in range(a.warmup):
        if flush is not None:
            flush.sum()
        step()
    torch.cuda.synchronize(dev)
    log(f"[bench] warm-up done ({a.warmup} steps)")
    alloc0 = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    free0 = torch.cuda.mem_get_info(dev)[0]

    # Timed region: K steps; an event pair around every launch on the launch stream.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    wall0 = time.perf_counter()
    region0.record(stream)
    for i in range(a.steps):
        if flush is not None:
            flush.sum()
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    region1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    free1 = torch.cuda.mem_get_info(dev)[0]
    peak_alloc = torch.cuda.max_memory_allocated(dev) - alloc0
    region_ms = region0.elapsed_time(region1)
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    med_launch_ms = sorted(launch_ms)[len(launch_ms) // 2]
    # with --cold the region holds the flushes: the step time is the median launch
    ms_per_step = med_launch_ms if a.cold else region_ms / a.steps
    log(f"[bench] {a.steps} steps: region {region_ms:.3f} ms, {ms_per_step:.4f} ms/step, "
        f"avg launch {avg_launch_ms:.4f} ms (min {min(launch_ms):.4f}), wall {wall:.3f} s")

    if a.calib_copy_mib > 0:
        n = a.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        log(f"[bench] calibration copy: {a.calib_copy_mib} MiB read + {a.calib_copy_mib} MiB written")
        del src, dst

    flops = w.flops() * (2.5 if bwd else 1.0)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    src_hash = kernel_source_hash(BWD_KERNEL_SOURCES if bwd else KERNEL_SOURCES)
    family = "attn_bwd" if bwd else ("attn_decode" if w.kv_cache else "attn_fwd")
    traffic = read_traffic(name, src_hash, family)
    abytes = bwd_algorithmic_bytes(w) if bwd else algorithmic_bytes(w, x["key_lens"])
    if bwd:
        metric, unit = METRIC_BWD, "TFLOP/s"
        value = tflops
        achieved = flops / (avg_launch_ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[w.dtype]
        roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                    "frac": achieved / peak, "traffic": traffic,
                    "kernels": "attn_bwd_dq_kernel + attn_bwd_dkdv_kernel, timed together"}
    elif w.kv_cache:
        # HBM-bound: K and V are read once and each byte feeds 2 flops per query.
        metric, unit = METRIC_DECODE, "GB/s"
        value = abytes / (ms_per_step * 1e-3) / 1e9
        achieved = abytes / (avg_launch_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                    "kernels": "attn_fwd_mfma_kernel (key splits) + attn_merge_kernel, timed together"}
        peak = PEAK_HBM_GBS
    else:
        metric, unit = (METRIC if w.window is None else METRIC_WINDOW), "TFLOP/s"
        value = tflops
        achieved = flops / (avg_launch_ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[w.dtype]
        roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                    "frac": achieved / peak, "traffic": traffic}

    result = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "D": w.D,
                   "causal": w.causal, "key_padding": w.padded, "window": w.window,
                   "kv_cache": w.kv_cache, "pass": a.which, "seed": x["seed"],
                   "cache": "cold" if a.cold else "warm", "launch": "hip graph replay" if a.graph else "eager",
                   "parallelism": "none (1 GPU)"},
        "pct_of_peak": 100.0 * value / peak,
        "roofline": roofline,
        "tflops": tflops,
        "avg_launch_ms": avg_launch_ms,
        "median_launch_ms": med_launch_ms,
        "min_launch_ms": min(launch_ms),
        "step_alloc_bytes": {"torch_peak": int(peak_alloc), "device_free_delta": int(free0 - free1)},
        "algorithmic_bytes": abytes,
        "algorithmic_gbs": abytes / (avg_launch_ms * 1e-3) / 1e9,
        "kernel_source_sha256": src_hash,
        "input_sha256": inputs.input_hashes(x),
    }
    if not a.no_cpu_baseline and bwd:
        log(f"[bench] cpu baseline: oracle backward on sampled slices (~{a.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline_bwd(w, x, do_np, grads, a.cpu_seconds, nthreads=a.cpu_threads)
        cb = result["cpu_baseline"]
        log(f"[bench] cpu baseline {cb['value']:.4g} {cb['unit']} on {cb['cores']} threads; "
            f"sample max relative gradient error {cb['sample_max_rel_err_grads']:.3e}")
    elif not a.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on a sample (~{a.cpu_seconds:.0f} s)")
        result["cpu_baseline"] = cpu_baseline(w, x, o, lse, a.cpu_seconds, nthreads=a.cpu_threads)
        cb = result["cpu_baseline"]
        log(f"[bench] cpu baseline {cb['value']:.4g} {cb['unit']} on {cb['cores']} threads; "
            f"sample max|dO|={cb['sample_max_abs_err_o']:.3e} max|dLSE|={cb['sample_max_abs_err_lse']:.3e}")
    else:
        result["cpu_baseline"] = None
    # The CPU baseline's sample doubles as a parity check at the benchmarked size and launch
    # configuration: the line is printed either way, and the run fails if the sample breaks the
    # tolerance (O: 2e-2 for bf16/fp16, 1e-4 for fp32; LSE: 1e-3; backward: each gradient's max
    # error within 2e-2 (1e-4 for fp32) of its largest entry).
    parity_ok = True
    cb = result["cpu_baseline"]
    if cb is not None:
        tol_o = 1e-4 if w.dtype == "f32" else 2e-2
        if bwd:
            parity_ok = cb["sample_max_rel_err_grads"] <= tol_o
            result["parity"] = {"checked": cb["sample"].split(" random")[0] + " (b, h) slices",
                                "max_rel_err_grads": cb["sample_max_rel_err_grads"], "tol": tol_o,
                                "pass": parity_ok}
        else:
            parity_ok = cb["sample_max_abs_err_o"] <= tol_o and cb["sample_max_abs_err_lse"] <= 1e-3
            result["parity"] = {"checked": cb["sample"].split(" random")[0] + " rows",
                                "max_abs_err_o": cb["sample_max_abs_err_o"], "tol_o": tol_o,
                                "max_abs_err_lse": cb["sample_max_abs_err_lse"], "tol_lse": 1e-3,
                                "pass": parity_ok}
    print(json.dumps(result), flush=True)
    if not parity_ok:
        log(f"[bench] PARITY FAILURE against the oracle on the sampled rows: {result['parity']}")
        sys.exit(1)


if __name__ == "__main__":
    main()
