"""Benchmark of the GDN hot path on one MI355X.

A step is one pass of the path over one batch: ``gdn_verify`` (T=4 tokens per
request, every intermediate state stored) followed by ``gdn_commit`` of the accepted
prefix, on the MTP verify workload (B=64, Hk=4, Hv=8, d=128, bf16 state, pool of
256 slots; synthetic seeded inputs). Inputs are resident in HBM before timing starts.

Timing: the steps run from a HIP graph (launch cost off the clock) over R rotating
buffer sets whose combined footprint exceeds the 256 MB Infinity Cache, so every
launch reads and writes HBM. W warm-up steps, then exactly K timed steps between two
synchronisations; value = B*T*K / elapsed (tokens/s). The dominant kernel (verify) is
also timed on its own the same way to give its average launch duration, from which
the roofline fraction is computed with the algorithmic bytes of one call.

Prints ONE JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD published figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak, AMD published figure
INFINITY_CACHE_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRCS = [os.path.join(ROOT, "linear_attention_speculative_gdn_amd", "csrc", f)
               for f in ("gdn_kernels.hip", "gdn_device.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the recurrent kernel's sources without comments and blank lines: a
    comment edit does not invalidate counter figures taken on the same code."""
    code = []
    for path in KERNEL_SRCS:
        with open(path) as fh:
            for line in fh:
                line = line.split("//", 1)[0].strip()
                if line:
                    code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def traffic_from_profiles(workload_name: str):
    """HBM bytes per verify launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"gdn_verify_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, x, budget_s: float) -> dict:
    """The float64 oracle, as it stands, on the same inputs: full verify + commit calls,
    repeated until the time budget is spent (at least once)."""
    import oracle
    import numpy as np
    nthreads = min(16, os.cpu_count() or 1)
    f = {n: x[n].double().numpy() for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "pool")}
    idx, acc = x["idx"].numpy(), x["accept"].numpy()
    d = oracle.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, w.state_dtype == "bf16", scale=w.scale)
    reps = 0
    t0 = time.perf_counter()
    while True:
        r = oracle.verify(d, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"], idx,
                          cache_T=w.cache_T, write_final=w.write_final, nthreads=nthreads)
        oracle.commit(d, r["cache"], w.cache_T, idx, acc, r["pool"], nthreads=nthreads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    del np
    return {"value": reps * w.batch * w.T / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{reps} full verify+commit calls of the workload (B*T={w.batch * w.T} tokens each) "
                      f"in {el:.1f} s, float64, OpenMP over (row, v-head) tiles"}


class Runner:
    """n calls of ``fn`` over rotating buffer sets, replayed from HIP graphs captured
    beforehand (``prepare(n)`` captures whatever ``run(n)`` replays), or launched eagerly."""

    def __init__(self, fn, sets, stream, eager: bool, per_replay: int):
        self.fn, self.sets, self.stream, self.eager, self.per_replay = fn, sets, stream, eager, per_replay
        self.graphs, self.pos = {}, 0

    def _capture(self, n):
        import torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for i in range(n):
                self.fn(self.sets[i % len(self.sets)])
        return g

    def prepare(self, n):
        if self.eager:
            return
        full, rest = divmod(n, self.per_replay)
        for k in ([self.per_replay] if full else []) + ([rest] if rest else []):
            if k not in self.graphs:
                self.graphs[k] = self._capture(k)

    def run(self, n):
        if self.eager:
            for i in range(n):
                self.fn(self.sets[(self.pos + i) % len(self.sets)])
            self.pos += n
            return
        full, rest = divmod(n, self.per_replay)
        for _ in range(full):
            self.graphs[self.per_replay].replay()
        if rest:
            self.graphs[rest].replay()

    def warm(self, n):
        import torch
        self.prepare(n)
        with torch.cuda.stream(self.stream):
            self.run(n)
        torch.cuda.synchronize()

    def timed(self, n) -> float:
        """Seconds for n calls, HIP events on the launch stream."""
        import torch
        self.prepare(n)
        cs = self.stream if not self.eager else torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(cs):
            e0.record(cs)
            self.run(n)
            e1.record(cs)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3


def copy_ceiling_gbps(dev) -> float:
    """A plain 1 GiB device copy, same event protocol: the practical streaming ceiling."""
    import torch
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 10 * 2 * src.numel() * 2 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbps


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


def conv_main(args):
    """The short causal convolution kept next to the GDN state: one gdn_conv_update per
    step (fused commit of the previous step's accepted prefix, then this step's tokens;
    write-back for the decode workload), same cold protocol as the GDN path."""
    import numpy as np
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
    R = max(2, math.ceil(4 * INFINITY_CACHE_BYTES / max(1, state_read)))
    R = min(R, 1024, max(2, int(16e9 // set_bytes)))
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
    run = Runner(call, sets, torch.cuda.Stream(), args.eager, R * max(1, 200 // R))
    run.warm(args.warmup)
    t = run.timed(args.steps)
    us = t / args.steps * 1e6
    achieved = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] conv: {us:.2f} us/launch, {achieved:.1f} GB/s algorithmic, {achieved / HBM_PEAK_GBPS:.3f} of 8 TB/s")
    res = {
        "metric": "GDN short-conv update tokens/s (batch x T) + achieved HBM GB/s vs peak",
        "value": w.batch * w.T / (us * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us * 1e-3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "T": w.T, "channels": w.channels, "width": w.width,
                   "pool_slots": w.pool, "dtype": w.dtype, "activation": w.activation,
                   "step": "conv update" + (" with fused commit" if fused else "") + (" + write-back" if wb else ""),
                   "rotating_buffer_sets": R, "launch": "eager" if args.eager else "hip_graph",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None, "kernel": "gdn_conv_update (conv_kernel)",
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_us": us},
    }
    del np
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
    run = Runner(call, sets, torch.cuda.Stream(), args.eager, 2)
    run.warm(args.warmup)
    t = run.timed(args.steps)
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
    roof.update({"traffic": None, "kernel": "gdn_prefill (chunk_kernel + scan_kernel)",
                 "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": flops,
                 "avg_launch_us": us, "mfma_TFLOPs": tflops,
                 "mfma_frac": tflops / MFMA_BF16_PEAK_TFLOPS})
    res = {
        "metric": "GDN chunked prefill tokens/s + achieved HBM GB/s or MFMA TFLOP/s vs the binding peak",
        "value": w.tokens / (us * 1e-6), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us * 1e-3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "sequences": w.batch, "tokens": w.tokens, "num_k_heads": w.Hk,
                   "num_v_heads": w.Hv, "d_k": w.dk, "d_v": w.dv, "state_dtype": w.state_dtype,
                   "io_dtype": w.io_dtype, "chunk": 16, "launch": "eager" if args.eager else "hip_graph",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
    }
    print(json.dumps(res), flush=True)


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

    # Rotating buffer sets, so that every launch reads its state from HBM: the pool
    # reads of all sets together exceed the 256 MB Infinity Cache four times over
    # (nontemporal cache writes do not displace them, so only the reads are counted).
    # Slot indices and accept lengths are shared by all sets, as every GDN layer of a
    # serving step uses the same ones; everything else is per set.
    touched = v_bytes + c_bytes
    set_bytes = (x["pool"].numel() * x["pool"].element_size() * (1 + (w.cache_T / w.pool * w.batch if w.cache_T else 0))
                 + sum(x[n].numel() * x[n].element_size() for n in ("q", "k", "v", "a", "b")))
    R = max(2, math.ceil(4 * INFINITY_CACHE_BYTES / max(1, workloads.state_read_bytes(w, idx))))
    R = min(R, 1024, max(2, int(16e9 // set_bytes)))   # tiny workloads: latency-bound anyway
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
    per_replay = R * max(1, 200 // R)
    run_step = Runner(step, sets, stream, args.eager, per_replay)
    run_verify = Runner(verify, sets, stream, args.eager, per_replay)

    run_step.warm(args.warmup)
    t_step = run_step.timed(args.steps)
    log(f"[bench] {args.steps} steps in {t_step * 1e3:.3f} ms -> {t_step / args.steps * 1e6:.2f} us/step")

    # the dominant kernel on its own, same protocol
    run_verify.warm(args.warmup)
    t_ver = run_verify.timed(args.steps)
    us_ver = t_ver / args.steps * 1e6
    achieved = v_bytes / (us_ver * 1e-6) / 1e9
    log(f"[bench] verify alone: {us_ver:.2f} us/launch, {achieved:.1f} GB/s algorithmic "
        f"({v_bytes / 1e6:.2f} MB), {achieved / HBM_PEAK_GBPS:.3f} of 8 TB/s")

    if args.calibrate_copy:
        # 256 MiB read + 256 MiB written, launched alone: the reference for scaling
        # FETCH_SIZE / WRITE_SIZE counters to bytes
        a_ = torch.ones(1 << 27, dtype=torch.bfloat16, device=dev)
        b_ = torch.empty_like(a_)
        torch.cuda.synchronize()
        for _ in range(3):
            b_.copy_(a_)
            torch.cuda.synchronize()
        del a_, b_

    copy_gbps = copy_ceiling_gbps(dev)
    log(f"[bench] device copy ceiling: {copy_gbps:.1f} GB/s")
    cold = single_cold_launches(verify, sets, stream, dev)
    log(f"[bench] verify, single launches after a 1 GiB scratch fill: median {cold['median_us']:.2f} us, "
        f"min {cold['min_us']:.2f} us")

    tokens = w.batch * w.T
    n_valid = int(((idx >= 0) & (idx < w.pool)).sum())
    value = tokens * args.steps / t_step
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
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "T": w.T, "num_k_heads": w.Hk, "num_v_heads": w.Hv,
                   "d_k": w.dk, "d_v": w.dv, "pool_slots": w.pool, "state_dtype": w.state_dtype,
                   "io_dtype": w.io_dtype,
                   "step": ("cached-replay verify with in-kernel commit (accept lengths U{1..T})" if replay else
                            ("verify" if w.mode != "decode" else "decode") + (" with gated-norm output" if gated else "")
                            + (" + commit" if w.commit else "")),
                   "rotating_buffer_sets": R,
                   "launch": "eager" if args.eager else "hip_graph", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": None if (replay or gated) else traffic_from_profiles(w.name),
                     "kernel": ("gdn_verify_replay" if replay else "gdn_verify_gated" if gated else "gdn_verify")
                     + " (recurrent_kernel)",
                     "algorithmic_bytes_per_launch": v_bytes,
                     "avg_launch_us": us_ver},
        "verify_tokens_per_s": tokens / (us_ver * 1e-6),
        # padding rows cost a launch slot but no state traffic: the rate over the rows that do work
        "valid_rows": n_valid,
        "verify_valid_tokens_per_s": n_valid * w.T / (us_ver * 1e-6),
        "copy_ceiling_GBps": copy_gbps,
        "single_cold_launch": cold,
    }
    if not args.no_cpu and not replay and not gated:
        log("[bench] CPU oracle baseline ...")
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
        log(f"[bench] CPU oracle: {res['cpu_baseline']['value']:.1f} tokens/s on {res['cpu_baseline']['cores']} threads")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
