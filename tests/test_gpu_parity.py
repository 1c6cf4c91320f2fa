"""HIP path vs the float64 oracle on every workload, element by element, at full size
and in the launch configuration the benchmark times.

Besides the workloads as defined (q and k drawn as unit vectors, decays with a median
of a few 1e-3), every mode runs at full size on inputs that exercise what those leave
unseen: q and k stored unnormalised (norms 0.05-20, one zero vector and one of norm
1e-3 each), so the kernels' own L2 normalisation decides the result; and weak decay
(g about 0.9-0.999), so the state carried from token to token, into the intermediate
cache and through the fused commit dominates every step. Both state dtypes run in each
mode (decode, verify with cache and commit, verify with fused commit)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_harness import SENTINEL, compare_pool, f64, gpu_step, max_abs, oracle_step, say, to_gpu, tol

import linear_attention_speculative_gdn_amd as gdn
import oracle

pytestmark = pytest.mark.gpu


def _raw_weak(w, **kw):
    kw.setdefault("name", w.name)
    return w.replace(qk="raw", decay="weak", **kw).replace(name=kw["name"] + "-rawqk-weakdecay")


W = workloads.WORKLOADS
VARIANTS = [
    _raw_weak(W[1]),                                                             # decode, fp32
    _raw_weak(W[1], name="decode-t1-bf16", state_dtype="bf16", io_dtype="bf16"),  # decode, bf16
    _raw_weak(W[2]),                                                             # verify + commit, bf16
    _raw_weak(W[2], name="mtp-verify-t4-f32", state_dtype="f32", io_dtype="f32"),  # verify + commit, fp32
    _raw_weak(W[3]),                                                             # verify + commit, fp32, B=256
    _raw_weak(W[4]),                                                             # fused commit, bf16
    _raw_weak(W[4], name="verify-t8-f32-fused", state_dtype="f32", io_dtype="f32", batch=64, n_pad=6),
]


@pytest.mark.parametrize("wi", range(len(workloads.WORKLOADS)))
def test_workload_parity(wi):
    run_parity(workloads.WORKLOADS[wi], wi)


@pytest.mark.parametrize("w", VARIANTS, ids=[v.name for v in VARIANTS])
def test_unnormalised_qk_weak_decay_parity(w):
    x = workloads.make_inputs(w, seed=0)
    n = x["q"].double().norm(dim=-1)
    assert float(n.max()) > 10 and float(n[n > 0].min()) < 1e-2 and int((n == 0).sum()) == 1
    run_parity(w, w.name, x)


def run_parity(w, label, x=None):
    say(f"[parity] workload {label} {w.name}: generating")
    if x is None:
        x = workloads.make_inputs(w, seed=0)
    g = to_gpu(w, x)
    say(f"[parity] {w.name}: GPU {w.mode}")
    gpu_step(w, g)
    torch.cuda.synchronize()
    say(f"[parity] {w.name}: oracle")
    ref = oracle_step(w, x)
    idx = x["idx"].numpy()
    valid = (idx >= 0) & (idx < w.pool)
    T = tol(w)

    o_err = max_abs(f64(g["o"]), ref["o"])
    assert np.all(f64(g["o"])[~valid] == 0.0), "padding rows must have o = 0"
    say(f"[parity] {w.name}: max |o - oracle| = {o_err:.3e} (tol {T})")
    assert o_err <= T

    touched = np.zeros(w.pool, dtype=bool)
    if w.mode == "decode" or w.write_final or w.mode == "verify_fused":
        touched[idx[valid]] = True
    if w.mode == "verify_fused":
        pa = x["prev_accept"].numpy()
        assert np.all((pa >= 1) & (pa <= w.cache_T))
    pool_err, untouched_ok = compare_pool(w, g["pool"], ref["pool"], touched, x["pool"])
    say(f"[parity] {w.name}: pool max err {pool_err:.3e}, untouched slots bit-identical: {untouched_ok}")
    assert pool_err <= T and untouched_ok

    if w.cache_T:
        gc = workloads.from_device_state(g["cache"].cpu())
        vt = torch.from_numpy(np.nonzero(valid)[0])
        c_err = max_abs(gc[vt, :w.T].double().numpy(), ref["cache"][vt.numpy(), :w.T])
        say(f"[parity] {w.name}: cache max err {c_err:.3e}")
        assert c_err <= T
        # entries the call must not write keep their previous content, bit for bit
        before = (workloads.from_device_state(workloads.to_device_state(x["cache_prev"]))
                  if "cache_prev" in x else torch.full_like(gc, SENTINEL))
        pt = torch.from_numpy(np.nonzero(~valid)[0])
        assert torch.equal(gc[pt], before[pt])
        assert torch.equal(gc[:, w.T:], before[:, w.T:])

    if w.commit:
        say(f"[parity] {w.name}: GPU commit")
        pool_before = g["pool"].clone()
        gdn.gdn_commit(g["cache"], g["idx"], g["accept"], g["pool"])
        torch.cuda.synchronize()
        acc = x["accept"].numpy()
        # the oracle commits its own cache; the GPU must also commit exactly its own cache
        ref_pool = oracle.commit(oracle.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool,
                                                  w.state_dtype == "bf16"),
                                 ref["cache"], w.cache_T, idx, acc, ref["pool"])
        ctouched = np.zeros(w.pool, dtype=bool)
        ctouched[idx[valid & (acc >= 1) & (acc <= w.cache_T)]] = True
        err, untouched_ok = compare_pool(w, g["pool"], ref_pool, ctouched,
                                         workloads.from_device_state(pool_before.cpu()))
        say(f"[parity] {w.name}: pool after commit max err {err:.3e}")
        assert err <= T and untouched_ok
        gp = g["pool"]
        gc = g["cache"]
        rows = np.nonzero(valid)[0]
        for r in rows:
            assert torch.equal(gp[int(idx[r])], gc[int(r), int(acc[r]) - 1]), f"commit of row {r} not bit-exact"
