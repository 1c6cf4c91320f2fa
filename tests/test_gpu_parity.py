"""HIP path vs the float64 oracle on every workload, element by element, at full size
and in the launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import workloads
from gpu_harness import SENTINEL, compare_pool, f64, gpu_step, max_abs, oracle_step, say, to_gpu, tol

import linear_attention_speculative_gdn_amd as gdn
import oracle

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wi", range(len(workloads.WORKLOADS)))
def test_workload_parity(wi):
    w = workloads.WORKLOADS[wi]
    say(f"[parity] workload {wi} {w.name}: generating")
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
