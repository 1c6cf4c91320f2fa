"""Helpers of the GPU tests: run one workload step through the C ABI and through the
oracle on the same seeded inputs, and compare.

Tolerances (absolute, on outputs and on every stored state): 1e-4 for an fp32 state,
2e-2 for a bf16 state. Bookkeeping (which slots and cache entries are written, what
is left untouched) is compared bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import linear_attention_speculative_gdn_amd as gdn
import oracle
import workloads
from workloads import from_device_state, to_device_state

SENTINEL = 123.0  # exactly representable in bf16 and fp32; marks cache entries nobody may write


def tol(w: workloads.Workload) -> float:
    return 1e-4 if w.state_dtype == "f32" else 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def oracle_dims(w, T=None):
    return oracle.make_dims(w.batch, w.T if T is None else T, w.Hk, w.Hv, w.dk, w.dv, w.pool,
                            w.state_dtype == "bf16", scale=w.scale, eps=1e-6)


def to_gpu(w, x, dev="cuda"):
    """Generator outputs -> device tensors (states in device layout) + output buffers."""
    g = {n: x[n].to(dev) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx")}
    g["pool"] = to_device_state(x["pool"]).to(dev)
    g["o"] = torch.full((w.batch, w.T, w.Hv, w.dv), float("nan"), dtype=x["v"].dtype, device=dev)
    if w.cache_T:
        if "cache_prev" in x:
            g["cache"] = to_device_state(x["cache_prev"]).to(dev)
        else:
            g["cache"] = torch.full((w.batch, w.cache_T, w.Hv, w.dv, w.dk), SENTINEL,
                                    dtype=x["pool"].dtype, device=dev)
    for n in ("accept", "prev_accept"):
        if n in x:
            g[n] = x[n].to(dev)
    return g


def gpu_step(w, g):
    """The workload's hot-path call on the GPU (no commit)."""
    if w.mode == "decode":
        gdn.gdn_decode(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], g["o"], g["pool"],
                       g["idx"], scale=w.scale)
    else:
        gdn.gdn_verify(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], g["o"], g["pool"],
                       g["idx"], g.get("cache"), w.write_final, g.get("prev_accept"), scale=w.scale)


def oracle_step(w, x, nthreads=None):
    f = {n: f64(x[n]) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "pool")}
    idx = x["idx"].numpy()
    d = oracle_dims(w)
    if w.mode == "decode":
        r = oracle.decode(d, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"], idx,
                          nthreads=nthreads)
        r["cache"] = None
        return r
    cache_in = f64(x["cache_prev"]) if "cache_prev" in x else None
    if cache_in is None and w.cache_T:
        cache_in = np.full((w.batch, w.cache_T, w.Hv, w.dk, w.dv), SENTINEL)
    prev = x["prev_accept"].numpy() if "prev_accept" in x else None
    return oracle.verify(d, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"], idx,
                         cache_T=w.cache_T, write_final=w.write_final, prev_accept=prev, cache_in=cache_in,
                         nthreads=nthreads)


def max_abs(a: np.ndarray, b: np.ndarray) -> float:
    if a.size == 0:
        return 0.0
    return float(torch.max(torch.abs(torch.from_numpy(np.ascontiguousarray(a)) -
                                     torch.from_numpy(np.ascontiguousarray(b)))).item())


def compare_pool(w, pool_gpu_dev_layout: torch.Tensor, pool_ref: np.ndarray, touched: np.ndarray, pool_before):
    """Touched slots within tolerance; every other slot bit-identical to ``pool_before``."""
    gpu = from_device_state(pool_gpu_dev_layout.cpu())
    t_idx = torch.from_numpy(np.nonzero(touched)[0])
    u_idx = torch.from_numpy(np.nonzero(~touched)[0])
    err = max_abs(gpu[t_idx].double().numpy(), pool_ref[t_idx.numpy()])
    untouched_equal = bool(torch.equal(gpu[u_idx], pool_before[u_idx]))
    return err, untouched_equal
