"""GPU tests of the gated RMS-norm output epilogue (gdn_verify_gated) through the C ABI.

y = weight * o / sqrt(mean(o^2) + eps) * silu(z) per (row, token, v-head) vector. Two
comparisons:
- against the oracle chain (oracle verify, then the oracle's gated norm), within the bound
  the o tolerance implies: |dy_j| <= |w_j silu(z_j)| * tol_o / rms * (1 + |o_j| / rms),
  plus the rounding of y to the io dtype (2^-9 relative in bf16);
- against the oracle's gated norm of the GPU's own o from gdn_verify on the same inputs:
  that o is rounded to the io dtype, so bf16 allows 2^-7 relative, fp32 1e-5.
The states (intermediates, write-back, pool) must equal gdn_verify's bit for bit: the
epilogue touches only the output.
"""
import numpy as np
import pytest
import torch

import linear_attention_speculative_gdn_amd as gdn
import oracle
import workloads
from gpu_harness import f64, oracle_step, say, to_gpu, tol
from workloads import Workload

pytestmark = pytest.mark.gpu
EPS = 1e-6


def gated_call(w, g, gate, y):
    if w.mode == "decode":
        gdn.gdn_verify_gated(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], gate["z"],
                             gate["norm_weight"], y, g["pool"], g["idx"], None, True, norm_eps=EPS, scale=w.scale)
    else:
        gdn.gdn_verify_gated(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], gate["z"],
                             gate["norm_weight"], y, g["pool"], g["idx"], g.get("cache"), w.write_final,
                             g.get("prev_accept"), norm_eps=EPS, scale=w.scale)


def plain_call(w, g):
    if w.mode == "decode":
        gdn.gdn_decode(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], g["o"], g["pool"],
                       g["idx"], scale=w.scale)
    else:
        gdn.gdn_verify(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], g["o"], g["pool"],
                       g["idx"], g.get("cache"), w.write_final, g.get("prev_accept"), scale=w.scale)


def run_case(w, seed=0):
    x = workloads.make_inputs(w, seed=seed)
    gate_cpu = workloads.make_gate_inputs(w, seed=seed + 100)
    gate = {n: t.to("cuda") for n, t in gate_cpu.items()}
    g1, g2 = to_gpu(w, x), to_gpu(w, x)
    y = torch.full(g1["o"].shape, float("nan"), dtype=g1["o"].dtype, device="cuda")
    gated_call(w, g1, gate, y)
    plain_call(w, g2)
    torch.cuda.synchronize()
    # the states are the plain path's, bit for bit
    assert torch.equal(g1["pool"], g2["pool"])
    if "cache" in g1:
        assert torch.equal(g1["cache"], g2["cache"])
    z, nw = f64(gate_cpu["z"]), f64(gate_cpu["norm_weight"])
    gain = np.abs(nw * z / (1.0 + np.exp(-z)))
    # 1. against the oracle chain
    idx = x["idx"].numpy()
    o_ref = oracle_step(w, x)["o"]
    y_ref = oracle.gated_norm(o_ref, z, nw, EPS)
    rms = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True) + EPS)
    t_o = tol(w) if w.io_dtype == "f32" else max(tol(w), 2e-2)
    out_round = 2.0 ** -9 if w.io_dtype == "bf16" else 1e-7
    bound = gain * t_o / rms * (1.0 + np.abs(o_ref) / rms) + out_round * np.abs(y_ref) + 1e-6
    yg = f64(y)
    err = np.abs(yg - y_ref)
    say(f"[gated] {w.name}: y err vs oracle chain {err.max():.2e} (bound min {bound.min():.1e})")
    assert np.all(err <= bound)
    # 2. against the gated norm of the GPU's own o
    y_own = oracle.gated_norm(f64(g2["o"]), z, nw, EPS)
    rt = 2.0 ** -7 if w.io_dtype == "bf16" else 1e-5
    err2 = np.abs(yg - y_own)
    say(f"[gated] {w.name}: y err vs norm of the GPU's o {err2.max():.2e}")
    assert np.all(err2 <= rt * (np.abs(y_own) + gain) + 1e-6)
    pad = (idx < 0) | (idx >= w.pool)
    assert bool(torch.all(y[torch.from_numpy(pad)] == 0))


GATED_WL = [workloads.WORKLOADS[i] for i in (1, 2, 4)]
GATED_WL += [w.replace(name=w.name + "-rawqk-weakdecay", qk="raw", decay="weak") for w in GATED_WL]


@pytest.mark.parametrize("w", GATED_WL, ids=[w.name for w in GATED_WL])
def test_gated_parity_workloads(w):
    """The decode, MTP T=4 and T=8 fused workloads at full size; the rawqk-weakdecay
    copies store q and k unnormalised and draw weak decays."""
    run_case(w)


GEOM = [
    Workload("g-dk16-dv256-bf16", batch=5, T=3, Hk=1, Hv=2, dk=16, dv=256, pool=8, state_dtype="bf16",
             io_dtype="bf16", mode="verify", cache_T=3, n_pad=1),
    Workload("g-dk32-dv64-f32", batch=4, T=9, Hk=2, Hv=2, dk=32, dv=64, pool=6, state_dtype="f32",
             io_dtype="f32", mode="verify", cache_T=9, write_final=True),
    Workload("g-dk64-dv256-mixed", batch=3, T=4, Hk=1, Hv=3, dk=64, dv=256, pool=5, state_dtype="f32",
             io_dtype="bf16", mode="verify", cache_T=4, n_pad=1),
    Workload("g-dk128-dv80-bf16-f32io", batch=6, T=2, Hk=2, Hv=4, dk=128, dv=80, pool=9, state_dtype="bf16",
             io_dtype="f32", mode="verify", cache_T=2),
    Workload("g-dk256-dv48-bf16", batch=3, T=5, Hk=1, Hv=2, dk=256, dv=48, pool=4, state_dtype="bf16",
             io_dtype="bf16", mode="verify", cache_T=5, write_final=True),
    Workload("g-decode-dk128-f32", batch=16, T=1, Hk=2, Hv=4, dk=128, dv=128, pool=32, state_dtype="f32",
             io_dtype="f32", mode="decode", n_pad=3),
    Workload("g-t16-dk128-bf16", batch=4, T=16, Hk=1, Hv=2, dk=128, dv=128, pool=6, state_dtype="bf16",
             io_dtype="bf16", mode="verify", cache_T=16),
    Workload("g-t6-dk128-dv48-f32", batch=5, T=6, Hk=1, Hv=2, dk=128, dv=48, pool=7, state_dtype="f32",
             io_dtype="f32", mode="verify", cache_T=6, write_final=True, n_pad=1),
]


@pytest.mark.parametrize("variant", ["as-drawn", "rawqk-weakdecay"])
@pytest.mark.parametrize("w", GEOM, ids=[w.name for w in GEOM])
def test_gated_geometries(w, variant):
    run_case(w if variant == "as-drawn" else w.replace(qk="raw", decay="weak"), seed=3)


def test_gated_unsupported_wide_dv():
    w = Workload("g-dk128-dv256", batch=2, T=1, Hk=1, Hv=1, dk=128, dv=256, pool=2, state_dtype="f32",
                 io_dtype="f32", mode="decode")
    x = workloads.make_inputs(w)
    g = to_gpu(w, x)
    gate = {n: t.to("cuda") for n, t in workloads.make_gate_inputs(w).items()}
    with pytest.raises(gdn.GdnError) as e:
        gated_call(w, g, gate, g["o"])
    assert e.value.status == 5
