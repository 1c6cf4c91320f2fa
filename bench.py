"""Benchmark of the GDN hot path on one MI355X.

A step is one pass of the path over one batch: ``gdn_verify`` (T=4 tokens per
request, every intermediate state stored) followed by ``gdn_commit`` of the accepted
prefix, on the MTP verify workload (B=64, Hk=4, Hv=8, d=128, bf16 state, pool of
256 slots; synthetic seeded inputs). Inputs are resident in HBM before timing starts.

Timing: the steps run from HIP graphs (launch cost off the clock) over R rotating
buffer sets whose state reads together exceed the 256 MB Infinity Cache four times, so
every launch reads and writes HBM. The sets are used in one rotation that continues
across the warm-up, the timed steps and every later timing: at any step count each
timed launch uses a set that the previous R-1 launches did not touch. W warm-up steps,
then exactly K timed steps between two synchronisations (HIP events on the launch
stream); value = B*T*K / elapsed (tokens/s). The dominant kernel (verify) is then timed
on its own the same way; its average launch duration gives the roofline fraction with
the algorithmic bytes of one call, and its rate is also compared with a streaming copy
of the same read:write mix timed under the same protocol (the practical ceiling).

Prints ONE JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, AMD published figure
# fp32 vector FMA without packed (two-lane) instructions, which the library is compiled without:
# 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz (half the 157.3 TFLOP/s packed figure)
VALU_F32_PEAK_TFLOPS = 78.6
INFINITY_CACHE_BYTES = 256 << 20
# launches of the dominant kernel before and in each roofline window (about 30 ms of verify
# calls): enough for the chip's clocks to settle whatever K and W are
SETTLE_LAUNCHES = 2000
SETTLE_SECONDS = 0.02  # untimed calls before the warm-up in the single-kernel modes
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "linear_attention_speculative_gdn_amd", "csrc")
KERNEL_SRCS = {
    "recurrent": ["gdn_kernels.hip", "gdn_device.h", "gdn_internal.h", "gdn_api.cpp"],
    "conv": ["gdn_conv.hip", "gdn_device.h", "gdn_internal.h", "gdn_api.cpp"],
    "prefill": ["gdn_prefill.hip", "gdn_device.h", "gdn_internal.h", "gdn_api.cpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(kind: str) -> str:
    """Hash of a kernel family's sources (and the launch code) without comments and blank
    lines: a comment edit does not invalidate counter figures taken on the same code."""
    code = []
    for name in KERNEL_SRCS[kind]:
        with open(os.path.join(CSRC, name)) as fh:
            for line in fh:
                line = line.split("//", 1)[0].strip()
                if line:
                    code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def profile_record(entry: str, workload_name: str, kind: str):
    """The committed rocprofv3 counter summary ``profiles/<entry>_<workload>_traffic.json``,
    if it was taken on the current source of the kernel family; else None."""
    path = os.path.join(PROFILES, f"{entry}_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(kind):
        log(f"[bench] {os.path.basename(path)} was taken on other kernel sources: counters not reported")
        return None
    return rec


def traffic_from_profiles(entry: str, workload_name: str, kind: str):
    """HBM bytes per call (FETCH_SIZE + WRITE_SIZE, calibrated) from the committed summary."""
    rec = profile_record(entry, workload_name, kind)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, x, budget_s: float) -> dict:
    """The float64 oracle, as it stands, on the same inputs: full verify + commit calls
    (the oracle's own C functions on prepared float64 arrays, input preparation outside
    the clock), repeated for budget/3 seconds, three times; the median rate of the three.
    Threads: every CPU this process may use, within OMP_NUM_THREADS (the box's share)."""
    import numpy as np

    import oracle
    nthreads = oracle.host_threads()
    f = {n: np.ascontiguousarray(x[n].double().numpy()) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias")}
    idx, acc = x["idx"].numpy().astype(np.int32), x["accept"].numpy().astype(np.int32)
    d = oracle.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, w.state_dtype == "bf16", scale=w.scale)
    pool0 = np.ascontiguousarray(x["pool"].double().numpy())
    cache = np.zeros((w.batch, w.cache_T, w.Hv, w.dk, w.dv))
    rates, calls = [], []
    for _ in range(3):
        pool = pool0.copy()
        reps, el = 0, 0.0
        while el < budget_s / 3 or reps == 0:
            t0 = time.perf_counter()
            oracle.verify_commit_inplace(d, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], pool,
                                         idx, cache, w.cache_T, acc, nthreads=nthreads)
            el += time.perf_counter() - t0
            reps += 1
        rates.append(reps * w.batch * w.T / el)
        calls.append(reps)
    try:
        nproc = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        nproc = os.cpu_count() or 1
    return {"value": statistics.median(rates), "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"3 runs of about {budget_s / 3:.0f} s, each full verify + commit calls of the workload "
                      f"(B*T={w.batch * w.T} tokens per call; {'/'.join(map(str, calls))} calls), float64, "
                      f"OpenMP over (row, v-head) tiles; median of the 3 rates",
            "runs_tokens_per_s": rates, "nproc": nproc, "hardware_concurrency": os.cpu_count(),
            "cpu_model": cpu_model(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


class Rotation:
    """Position of the next launch in the rotation over the buffer sets, shared by every
    runner of those sets."""

    def __init__(self, nsets: int):
        self.nsets, self.pos = nsets, 0


class Runner:
    """n calls of ``fn`` over rotating buffer sets from the rotation's current position,
    replayed from HIP graphs captured beforehand (``prepare(n)`` captures whatever
    ``run(n)`` replays), or launched eagerly."""

    def __init__(self, fn, sets, rot: Rotation, stream, eager: bool, per_replay: int):
        assert per_replay % len(sets) == 0
        self.fn, self.sets, self.rot, self.stream, self.eager = fn, sets, rot, stream, eager
        self.per_replay = per_replay
        self.graphs = {}

    def _capture(self, start, n):
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for i in range(n):
                self.fn(self.sets[(start + i) % len(self.sets)])
        return g

    def _pieces(self, n, ahead=0):
        """(first set, calls) of the graph replays that make n calls from the current position
        (plus `ahead` calls)."""
        full, rest = divmod(n, self.per_replay)
        start = (self.rot.pos + ahead) % len(self.sets)
        out = [(start, self.per_replay)] * full        # a multiple of the set count: same start
        if rest:
            out.append((start, rest))
        return out

    def prepare(self, n, ahead=0):
        """Captures the graphs that n calls starting `ahead` calls from now will replay."""
        if self.eager:
            return
        for key in self._pieces(n, ahead):
            if key not in self.graphs:
                self.graphs[key] = self._capture(*key)

    def run(self, n):
        if self.eager:
            for i in range(n):
                self.fn(self.sets[(self.rot.pos + i) % len(self.sets)])
        else:
            for key in self._pieces(n):
                self.graphs[key].replay()
        self.rot.pos += n

    def warm(self, n):
        import torch
        self.prepare(n)
        with torch.cuda.stream(self.stream):
            self.run(n)
        torch.cuda.synchronize()

    def timed(self, n) -> float:
        """Seconds for n calls, HIP events on the launch stream. The stream is held for
        200 us (gdn_stream_wait) before the first event, so that the event is stamped when
        the calls behind it are queued and the host's submission latency stays off the
        clock."""
        import torch
        self.prepare(n)
        cs = self.stream if not self.eager else torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(cs):
            st = stream_lib().gdn_stream_wait(200000, ctypes.c_void_p(cs.cuda_stream))
            if st != 0:
                raise RuntimeError(f"gdn_stream_wait returned {st}")
            e0.record(cs)
            self.run(n)
            e1.record(cs)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3


def settled_timing(run: Runner, warmup: int, steps: int, est_us: float) -> float:
    """Seconds for exactly `steps` calls after exactly `warmup` warm-up calls, preceded by
    untimed calls worth about SETTLE_SECONDS (at `est_us` per call) so that the chip's clocks
    have settled whatever the step counts; all graphs captured before any of them runs."""
    n_settle = 0 if run.eager else max(1, int(SETTLE_SECONDS / (est_us * 1e-6)))
    run.prepare(n_settle)
    run.prepare(warmup, ahead=n_settle)
    run.prepare(steps, ahead=n_settle + warmup)
    run.warm(n_settle)
    run.warm(warmup)
    return run.timed(steps)


def rotating_sets(read_bytes: int, set_bytes: int) -> int:
    """Buffer sets so that the state reads of one rotation exceed the Infinity Cache four
    times (nontemporal writes do not displace read data from it, so reads are what count),
    within 16 GB of buffers."""
    R = max(2, math.ceil(4 * INFINITY_CACHE_BYTES / max(1, read_bytes)))
    return min(R, 1024, max(2, int(16e9 // max(1, set_bytes))))


def per_replay_of(R: int) -> int:
    return R * max(1, 200 // R)


_stream_lib = None


def stream_lib():
    global _stream_lib
    if _stream_lib is None:
        path = os.path.join(ROOT, "linear_attention_speculative_gdn_amd", "libgdn_stream.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(path)
        L.gdn_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_int32] * 4 + [
            ctypes.c_void_p]
        L.gdn_stream_copy.restype = ctypes.c_int32
        L.gdn_stream_wait.argtypes = [ctypes.c_int64, ctypes.c_void_p]
        L.gdn_stream_wait.restype = ctypes.c_int32
        _stream_lib = L
    return _stream_lib


# (threads per workgroup, 16-byte chunks per thread, flags: 1 nontemporal loads, 2
# nontemporal stores, 4 copy-major) of the streaming-copy variants timed for the ceiling:
# the fastest of a sweep over 64/256/1024 threads, 1-8 chunks and the flags, at the read:write
# mixes of decode (1:1), the MTP T=4 verify (1:4) and the T=8 verify (1:9)
COPY_VARIANTS = ((64, 8, 7), (64, 1, 3), (64, 1, 4), (256, 2, 3), (256, 2, 7))


def copy_ceiling(dev, read_bytes: int, writes: int, launches: int, eager: bool) -> dict:
    """The streaming copy of libgdn_stream.so moving the state bytes of one call
    (`read_bytes` in, `writes` x out) over rotating cold buffer sets, replayed from graphs
    like the kernel it is compared with, for each variant of COPY_VARIANTS: the best rate is
    the practical HBM ceiling for that mix."""
    import torch
    L = stream_lib()
    unit = 64 * 8 * 16                                # a multiple of every variant's block
    rd = max(1, read_bytes // unit) * unit
    R = rotating_sets(rd, rd * (1 + writes))
    sets = [{"src": torch.empty(rd, dtype=torch.uint8, device=dev).fill_(i & 0xFF),
             "dst": torch.empty(rd * writes, dtype=torch.uint8, device=dev)} for i in range(R)]
    stream = torch.cuda.Stream()
    moved = rd * (1 + writes)
    n = max(launches, 2 * R)
    results = []
    for th, ch, fl in COPY_VARIANTS:
        def call(s, th=th, ch=ch, fl=fl):
            st = L.gdn_stream_copy(ctypes.c_void_p(s["src"].data_ptr()), ctypes.c_void_p(s["dst"].data_ptr()), rd,
                                   writes, th, ch, fl, ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
            if st != 0:
                raise RuntimeError(f"gdn_stream_copy returned {st}")
        with torch.cuda.stream(stream):
            call(sets[0])
        torch.cuda.synchronize()
        run = Runner(call, sets, Rotation(R), stream, eager, per_replay_of(R))
        run.warm(R)
        us = run.timed(n) / n * 1e6
        results.append({"threads": th, "chunks": ch, "nontemporal_loads": bool(fl & 1),
                        "nontemporal_stores": bool(fl & 2), "order": "copy-major" if fl & 4 else "block-major",
                        "us_per_launch": us, "GBps": moved / (us * 1e-6) / 1e9})
        del run
    del sets
    torch.cuda.empty_cache()
    best = max(results, key=lambda r: r["GBps"])
    return {"GBps": best["GBps"], "us_per_launch": best["us_per_launch"], "bytes_per_launch": moved,
            "mix": f"1 read : {writes} write{'s' if writes > 1 else ''}", "rotating_buffer_sets": R,
            "launches": n, "kernel": "gdn_stream_copy (libgdn_stream.so)", "best": best, "variants": results}


def single_cold_launches(fn, sets, stream, dev, n: int = 21) -> dict:
    """Cross-check of the rotating-set protocol: n single launches of ``fn``, each after a
    1 GiB scratch fill that evicts the L2s and the 256 MB Infinity Cache, timed one by one
    with HIP events on the launch stream (each figure also holds one launch's event and
    dispatch overhead, so it bounds the kernel time from above)."""
    import torch
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    us = []
    with torch.cuda.stream(stream):
        for i in range(n):
            scratch.fill_(i & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(sets[i % len(sets)])
            e1.record(stream)
            e1.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    us.sort()
    return {"launches": n, "median_us": us[n // 2], "min_us": us[0],
            "protocol": "each launch alone after a 1 GiB scratch fill"}


def calibration_copy(dev):
    """256 MiB read + 256 MiB written, launched alone: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters of a rocprofv3 pass to bytes."""
    import torch
    a_ = torch.ones(1 << 27, dtype=torch.bfloat16, device=dev)
    b_ = torch.empty_like(a_)
    torch.cuda.synchronize()
    for _ in range(3):
        b_.copy_(a_)
        torch.cuda.synchronize()
    del a_, b_


def conv_main(args):
    """The short causal convolution kept next to the GDN state: one gdn_conv_update per
    step (fused commit of the previous step's accepted prefix, then this step's tokens;
    write-back for the decode workload), same cold protocol as the GDN path."""
    import torch

    import linear_attention_speculative_gdn_amd as gdn
    import workloads

    wi = workloads.CONV_HEADLINE if args.workload is None else args.workload
    w = workloads.CONV_WORKLOADS[wi]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] conv workload {wi}: {w.description}")
    x = workloads.make_conv_inputs(w, seed=0)
    idx, plen = x["idx"].numpy(), x["prev_len"].numpy()
    fused, wb = w.mode == "fused", w.mode == "decode"
    nbytes = workloads.conv_bytes(w, idx, plen if fused else None)
    esz = x["x"].element_size()
    state_read = int(((idx >= 0) & (idx < w.pool)).sum()) * (w.width - 1) * w.channels * esz
    set_bytes = sum(x[n].numel() * x[n].element_size() for n in ("x", "prev_x", "pool")) + x["x"].numel() * esz
    R = rotating_sets(state_read, set_bytes)
    shared = {n: x[n].to(dev) for n in ("idx", "prev_len", "w", "bias")}
    sets = []
    for _ in range(R):
        s = {n: x[n].to(dev) for n in ("x", "prev_x", "pool")}
        s.update(shared)
        s["y"] = torch.empty_like(s["x"])
        sets.append(s)
    torch.cuda.synchronize()
    log(f"[bench] {R} rotating buffer sets, {nbytes / 1e6:.2f} MB algorithmic per call")

    def call(s):
        gdn.gdn_conv_update(s["x"], s["w"], s["bias"], s["pool"], s["idx"], s["y"],
                            prev_x=s["prev_x"] if fused else None, prev_len=s["prev_len"] if fused else None,
                            write_back=wb, activation=w.activation)

    call(sets[0])
    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibration_copy(dev)
    run = Runner(call, sets, Rotation(R), torch.cuda.Stream(), args.eager, per_replay_of(R))
    t = settled_timing(run, args.warmup, args.steps, est_us=6.0)
    us = t / args.steps * 1e6
    achieved = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] conv: {us:.2f} us/launch, {achieved:.1f} GB/s algorithmic, {achieved / HBM_PEAK_GBPS:.3f} of 8 TB/s")
    res = {
        "metric": "GDN short-conv update tokens/s (batch x T) + achieved HBM GB/s vs peak",
        "value": w.batch * w.T / (us * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us * 1e-3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "storage_dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "T": w.T, "channels": w.channels, "width": w.width,
                   "pool_slots": w.pool, "dtype": w.dtype, "activation": w.activation,
                   "step": "conv update" + (" with fused commit" if fused else "") + (" + write-back" if wb else ""),
                   "rotating_buffer_sets": R, "launch": "eager" if args.eager else "hip_graph",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic_from_profiles("gdn_conv_update", w.name, "conv"),
                     "kernel": "gdn_conv_update (conv_kernel)",
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": us},
    }
    print(json.dumps(res), flush=True)


def prefill_main(args):
    """The chunked prefill (gdn_prefill) on the prefill workloads: one call per step over
    the whole batch of sequences. Priced against whichever roof binds it: its algorithmic
    bytes at 8 TB/s or the flops of the chunked form at the 2.5 PFLOP/s bf16 dense MFMA
    peak (the bytes, at d = 128: about 13 us against 6 us of matrix-core time on 8 x 2048)."""
    import torch

    import linear_attention_speculative_gdn_amd as gdn
    import workloads

    wi = workloads.PREFILL_HEADLINE if args.workload is None else args.workload
    w = workloads.PREFILL_WORKLOADS[wi]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] prefill workload {wi}: {w.description}")
    x = workloads.make_prefill_inputs(w, seed=0)
    flops = workloads.prefill_flops(w)
    nbytes = workloads.prefill_bytes(w)
    R = 2
    ws_bytes = gdn.gdn_prefill_workspace_bytes(w.batch, w.tokens, w.Hk, w.Hv, w.dk, w.dv,
                                               workloads.torch_dtype(w.state_dtype))
    sets = []
    for _ in range(R):
        s = {n: x[n].to(dev) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx", "fresh", "cu_seqlens")}
        s["pool"] = workloads.to_device_state(x["pool"]).to(dev)
        s["o"] = torch.empty((w.tokens, w.Hv, w.dv), dtype=torch.bfloat16, device=dev)
        s["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        sets.append(s)
    log(f"[bench] prefill workspace {ws_bytes / 2**20:.1f} MiB per call")

    def call(s):
        gdn.gdn_prefill(s["q"], s["k"], s["v"], s["a"], s["b"], s["A_log"], s["dt_bias"], s["o"], s["pool"],
                        s["idx"], s["cu_seqlens"], s["fresh"], scale=w.scale, workspace=s["ws"])

    call(sets[0])
    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibration_copy(dev)
    run = Runner(call, sets, Rotation(R), torch.cuda.Stream(), args.eager, 2)
    t = settled_timing(run, args.warmup, args.steps, est_us=100.0)
    us = t / args.steps * 1e6
    tflops = flops / (us * 1e-6) / 1e12
    log(f"[bench] prefill: {us:.1f} us/launch, {w.tokens / (us * 1e-6) / 1e6:.1f} M tokens/s, {tflops:.1f} TFLOP/s "
        f"({flops / 1e9:.2f} GFLOP of the chunked form), {nbytes / (us * 1e-6) / 1e9:.0f} GB/s")
    gbps = nbytes / (us * 1e-6) / 1e9
    hbm_bound = nbytes / (HBM_PEAK_GBPS * 1e9) >= flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    roof = ({"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS}
            if hbm_bound else
            {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": tflops / MFMA_BF16_PEAK_TFLOPS})
    roof.update({"traffic": traffic_from_profiles("gdn_prefill", w.name, "prefill"),
                 "kernel": "gdn_prefill (chunk_kernel + scan_kernel)",
                 "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
                 "avg_launch_us": us, "mfma_TFLOPs": tflops,
                 "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS})
    res = {
        "metric": "GDN chunked prefill tokens/s + achieved HBM GB/s or MFMA TFLOP/s vs the binding peak",
        "value": w.tokens / (us * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us * 1e-3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "storage_dtype": w.state_dtype, "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.batch, "tokens": w.tokens, "num_k_heads": w.Hk,
                   "num_v_heads": w.Hv, "d_k": w.dk, "d_v": w.dv, "state_dtype": w.state_dtype,
                   "io_dtype": w.io_dtype, "chunk": 16, "launch": "eager" if args.eager else "hip_graph",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
    }
    print(json.dumps(res), flush=True)


def replay_flops(w, idx, rlen) -> int:
    """Flops of one cached-replay call, each multiply-add counted as 2: per state element,
    a new token takes S^T k, S^T q and the rank-1 update (3 multiply-adds, plus the decay
    scaling: 7 flop), a replayed token S^T k and the update (5 flop); valid rows only."""
    import numpy as np
    valid = (idx >= 0) & (idx < w.pool)
    n = np.where(valid & (rlen >= 0) & (rlen <= w.T), rlen, 0)
    elems = w.Hv * w.dk * w.dv
    return int(valid.sum()) * w.T * 7 * elems + int(n.sum()) * 5 * elems


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8000)
    ap.add_argument("--warmup", type=int, default=800)
    ap.add_argument("--workload", type=int, default=None, help="workload index (default: the MTP verify T=4 one)")
    ap.add_argument("--mode", choices=("intermediate", "gated", "replay", "conv", "prefill"), default="intermediate",
                    help="intermediate: verify storing every intermediate state, then commit (the "
                         "workload as defined); replay: cached-replay verify with in-kernel commit of the "
                         "previous step's accepted prefix (one launch per step, no per-token states); gated: "
                         "intermediate with the gated RMS-norm output epilogue fused into verify; prefill: the chunked "
                         "prefill on the matrix cores (--workload indexes the prefill workloads); conv: "
                         "the short causal convolution next to the GDN state (--workload indexes the "
                         "convolution workloads)")
    ap.add_argument("--eager", action="store_true", help="launch without HIP graphs (for counter collection)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="time budget of the CPU oracle baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the copy ceiling and the single cold launches (for profiler runs)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device copy (known bytes) for counter calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); the GDN state update "
              "shards by v-head or by request row with no collective, so N GPUs each run this one-GPU step "
              "on their share", file=sys.stderr)
        sys.exit(2)
    if args.mode == "conv":
        return conv_main(args)
    if args.mode == "prefill":
        return prefill_main(args)

    import numpy as np
    import torch

    import linear_attention_speculative_gdn_amd as gdn
    import workloads

    wi = workloads.HEADLINE if args.workload is None else args.workload
    w = workloads.WORKLOADS[wi]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {wi}: {w.description}")
    x = workloads.make_inputs(w, seed=0)
    idx = x["idx"].numpy()
    replay = args.mode == "replay"
    gated = args.mode == "gated"
    rlen = None
    if replay:
        if w.mode == "decode":
            sys.exit("bench.py: replay mode needs a verify workload")
        # the previous step's tokens (its k, v, a, b) and accept lengths
        xp = workloads.make_inputs(w, seed=1)
        rlen = np.random.default_rng(2).integers(1, w.T + 1, w.batch).astype(np.int32)
        v_bytes = workloads.replay_bytes(w, idx, rlen)
        c_bytes = 0
    else:
        v_bytes = workloads.algorithmic_bytes(w, idx, "verify")
        c_bytes = workloads.algorithmic_bytes(w, idx, "commit") if w.commit else 0
    if gated:  # z of valid rows and the norm weights are read as well
        xg = workloads.make_gate_inputs(w, seed=3)
        nvalid = int(((idx >= 0) & (idx < w.pool)).sum())
        v_bytes += nvalid * w.T * w.Hv * w.dv * xg["z"].element_size() + w.dv * 4

    # Rotating buffer sets, so that every launch reads its state from HBM. Slot indices and
    # accept lengths are shared by all sets, as every GDN layer of a serving step uses the
    # same ones; everything else is per set.
    touched = v_bytes + c_bytes
    state_read = workloads.state_read_bytes(w, idx)
    set_bytes = (x["pool"].numel() * x["pool"].element_size() * (1 + (w.cache_T / w.pool * w.batch if w.cache_T else 0))
                 + sum(x[n].numel() * x[n].element_size() for n in ("q", "k", "v", "a", "b")))
    R = rotating_sets(state_read, set_bytes)
    shared = {n: x[n].to(dev) for n in ("idx", "accept", "prev_accept") if n in x}
    base = {n: x[n].to(dev) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias")}
    if gated:
        shared["norm_weight"] = xg["norm_weight"].to(dev)
        base["z"] = xg["z"].to(dev)
    if replay:
        shared["rlen"] = torch.from_numpy(rlen).to(dev)
        base.update({"r" + n: xp[n].to(dev) for n in ("k", "v", "a", "b")})
    pool0 = workloads.to_device_state(x["pool"]).to(dev)
    cache0 = None
    if w.cache_T:
        cache0 = (workloads.to_device_state(x["cache_prev"]).to(dev) if "cache_prev" in x else
                  torch.zeros((w.batch, w.cache_T, w.Hv, w.dv, w.dk), dtype=pool0.dtype, device=dev))
    sets = []
    for _ in range(R):
        s = {n: t.clone() for n, t in base.items()}
        s.update(shared)
        s["pool"] = pool0.clone()
        s["cache"] = None if (cache0 is None or replay) else cache0.clone()
        s["o"] = torch.empty((w.batch, w.T, w.Hv, w.dv), dtype=x["v"].dtype, device=dev)
        sets.append(s)
    del pool0, cache0
    torch.cuda.synchronize()
    log(f"[bench] {R} rotating buffer sets, {touched / 1e6:.2f} MB touched per step")

    def verify(s):
        if replay:
            gdn.gdn_verify_replay(s["q"], s["k"], s["v"], s["a"], s["b"], s["A_log"], s["dt_bias"], s["o"],
                                  s["pool"], s["idx"], s["rk"], s["rv"], s["ra"], s["rb"], s["rlen"], True,
                                  scale=w.scale)
        elif gated:
            gdn.gdn_verify_gated(s["q"], s["k"], s["v"], s["a"], s["b"], s["A_log"], s["dt_bias"], s["z"],
                                 s["norm_weight"], s["o"], s["pool"], s["idx"], s["cache"],
                                 w.write_final or w.mode == "decode", s.get("prev_accept"), scale=w.scale)
        elif w.mode == "decode":
            gdn.gdn_decode(s["q"], s["k"], s["v"], s["a"], s["b"], s["A_log"], s["dt_bias"], s["o"], s["pool"],
                           s["idx"], scale=w.scale)
        else:
            gdn.gdn_verify(s["q"], s["k"], s["v"], s["a"], s["b"], s["A_log"], s["dt_bias"], s["o"], s["pool"],
                           s["idx"], s["cache"], w.write_final, s.get("prev_accept"), scale=w.scale)

    def commit(s):
        if w.commit and not replay:
            gdn.gdn_commit(s["cache"], s["idx"], s["accept"], s["pool"])

    def step(s):
        verify(s)
        commit(s)

    stream = torch.cuda.Stream()
    step(sets[0])  # first launches load the code objects, outside any capture
    torch.cuda.synchronize()
    if args.calibrate_copy:
        calibration_copy(dev)
    rot = Rotation(R)
    run_step = Runner(step, sets, rot, stream, args.eager, per_replay_of(R))
    run_verify = Runner(verify, sets, rot, stream, args.eager, per_replay_of(R))

    # Every graph is captured first, so that no capture (an idle GPU) sits between the
    # phases, and one rotation over the buffer sets runs through all of them. The dominant
    # kernel is timed on its own first, independently of K and W: a warm-up of at least
    # SETTLE_LAUNCHES launches (the chip's clocks settle within milliseconds of load; after a
    # 5-launch warm-up, 200-launch windows ran up to 20 % slow), then five windows of at
    # least SETTLE_LAUNCHES launches; the median window's average launch duration prices the
    # roofline. The step timing follows on the warm chip: exactly W warm-up steps, then
    # exactly K timed steps.
    # (eager launches serve counter collection, one row per dispatch: W and K as given there)
    n_vwarm = args.warmup if args.eager else max(args.warmup, SETTLE_LAUNCHES)
    n_ver = args.steps if args.eager else max(args.steps, SETTLE_LAUNCHES)
    run_verify.prepare(n_vwarm)
    for k_ in range(5):
        run_verify.prepare(n_ver, ahead=n_vwarm + k_ * n_ver)
    off = n_vwarm + 5 * n_ver
    run_step.prepare(args.warmup, ahead=off)
    run_step.prepare(args.steps, ahead=off + args.warmup)
    run_verify.warm(n_vwarm)
    windows_us = [run_verify.timed(n_ver) / n_ver * 1e6 for _ in range(5)]
    us_ver = statistics.median(windows_us)
    log(f"[bench] verify windows of {n_ver} launches: " + " ".join(f"{u:.2f}" for u in windows_us) + " us")

    run_step.warm(args.warmup)
    t_step = run_step.timed(args.steps)
    log(f"[bench] {args.steps} steps in {t_step * 1e3:.3f} ms -> {t_step / args.steps * 1e6:.2f} us/step")
    achieved = v_bytes / (us_ver * 1e-6) / 1e9
    log(f"[bench] verify alone: {us_ver:.2f} us/launch, {achieved:.1f} GB/s algorithmic "
        f"({v_bytes / 1e6:.2f} MB), {achieved / HBM_PEAK_GBPS:.3f} of 8 TB/s")

    extras = {}
    if not args.no_extras:
        # practical ceiling: a streaming copy of the call's state traffic (read once, written
        # once per stored state) under the same protocol
        writes = 1 if (replay or w.mode == "decode" or not w.cache_T) else w.T + (1 if w.mode == "verify_fused" else 0)
        ceil = copy_ceiling(dev, state_read, writes, args.steps, args.eager)
        log(f"[bench] streaming copy ceiling ({ceil['mix']}, {ceil['bytes_per_launch'] / 1e6:.1f} MB): "
            f"{ceil['us_per_launch']:.2f} us, {ceil['GBps']:.1f} GB/s")
        extras["copy_ceiling"] = ceil
        extras["single_cold_launch"] = single_cold_launches(verify, sets, stream, dev)
        log(f"[bench] verify, single launches after a 1 GiB scratch fill: median "
            f"{extras['single_cold_launch']['median_us']:.2f} us, min {extras['single_cold_launch']['min_us']:.2f} us")

    tokens = w.batch * w.T
    n_valid = int(((idx >= 0) & (idx < w.pool)).sum())
    value = tokens * args.steps / t_step
    entry = "gdn_verify_replay" if replay else "gdn_verify_gated" if gated else (
        "gdn_decode" if w.mode == "decode" else "gdn_verify")
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic_from_profiles(entry, w.name, "recurrent"),
            "kernel": entry + " (recurrent_kernel)", "algorithmic_bytes_per_launch": v_bytes,
            "avg_launch_us": us_ver, "timed_launches_per_window": n_ver,
            "window_avg_launch_us": windows_us}
    if "copy_ceiling" in extras:
        roof["copy_ceiling_GBps"] = extras["copy_ceiling"]["GBps"]
        roof["frac_of_copy_ceiling"] = achieved / extras["copy_ceiling"]["GBps"]
    if replay:
        # cached replay re-runs the accepted tokens instead of storing their states: its
        # bound is the fp32 vector ALU (flops below at the non-packed FMA rate); the HBM
        # figures stay beside it
        fl = replay_flops(w, idx, rlen)
        tf = fl / (us_ver * 1e-6) / 1e12
        hbm = {k_: roof[k_] for k_ in ("achieved", "peak", "unit", "frac")}
        roof.update({"bound": "alu", "achieved": tf, "peak": VALU_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / VALU_F32_PEAK_TFLOPS, "algorithmic_flops_per_launch": fl, "hbm": hbm})
        rec = profile_record(entry, w.name, "recurrent")
        if rec and rec.get("valu_wave_instructions_per_launch"):
            # share of the call during which a SIMD issues vector instructions: SQ_INSTS_VALU of one
            # call (counter pass) x 4 clocks per wave64 instruction on a 16-lane SIMD, over 1024
            # SIMDs and the live launch duration at 2.4 GHz
            roof["valu_busy_frac"] = rec["valu_wave_instructions_per_launch"] * 4 / 1024 / (us_ver * 1e-6 * 2.4e9)
    res = {
        "metric": "GDN verify tokens/s (batch x T) + achieved HBM GB/s vs peak, T=4 bf16 state",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # every product and sum is fp32; the state and the io are stored in the workload's dtypes
        "dtype": "f32",
        "storage_dtype": w.state_dtype if w.state_dtype == w.io_dtype else f"{w.state_dtype} state, {w.io_dtype} io",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "T": w.T, "num_k_heads": w.Hk, "num_v_heads": w.Hv,
                   "d_k": w.dk, "d_v": w.dv, "pool_slots": w.pool, "state_dtype": w.state_dtype,
                   "io_dtype": w.io_dtype,
                   "step": ("cached-replay verify with in-kernel commit (accept lengths U{1..T})" if replay else
                            ("verify" if w.mode != "decode" else "decode") + (" with gated-norm output" if gated else "")
                            + (" + commit" if w.commit else "")),
                   "rotating_buffer_sets": R,
                   "launch": "eager" if args.eager else "hip_graph", "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "verify_tokens_per_s": tokens / (us_ver * 1e-6),
        # padding rows cost a launch slot but no state traffic: the rate over the rows that do work
        "valid_rows": n_valid,
        "verify_valid_tokens_per_s": n_valid * w.T / (us_ver * 1e-6),
    }
    res.update(extras)
    if not args.no_cpu and not replay and not gated and w.commit:
        log("[bench] CPU oracle baseline ...")
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
        cb = res["cpu_baseline"]
        log(f"[bench] CPU oracle: {cb['value']:.1f} tokens/s on {cb['cores']} threads "
            f"({cb['nproc']} CPUs available, {cb['hardware_concurrency']} on the host, {cb['cpu_model']})")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
