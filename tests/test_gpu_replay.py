"""GPU tests of cached replay (gdn_verify_replay, gdn_commit_replay): parity with the
oracle, and bit-exact equality with the intermediate-state path it replaces."""
import numpy as np
import pytest
import torch

import linear_attention_speculative_gdn_amd as gdn
import oracle
import workloads
from gpu_harness import f64, max_abs, say, tol
from workloads import Workload, from_device_state, to_device_state

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_step(w, seed, A_log=None, dt_bias=None):
    x = workloads.make_inputs(w, seed=seed)
    if A_log is not None:
        x["A_log"], x["dt_bias"] = A_log, dt_bias
    g = {n: x[n].to(DEV) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx")}
    return x, g


def oracle_replay(w, x_cur, x_prev, pool_logical, idx, rlen, commit):
    d = oracle.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, w.state_dtype == "bf16", scale=w.scale)
    return oracle.verify_replay(d, f64(x_cur["q"]), f64(x_cur["k"]), f64(x_cur["v"]), f64(x_cur["a"]),
                                f64(x_cur["b"]), f64(x_cur["A_log"]), f64(x_cur["dt_bias"]), pool_logical, idx,
                                f64(x_prev["k"]), f64(x_prev["v"]), f64(x_prev["a"]), f64(x_prev["b"]), rlen,
                                commit=commit)


SHAPES = [
    Workload("mtp-t4-bf16", batch=64, T=4, Hk=4, Hv=8, dk=128, dv=128, pool=256, state_dtype="bf16",
             io_dtype="bf16", mode="verify", n_pad=8),
    Workload("t8-bf16", batch=128, T=8, Hk=16, Hv=32, dk=128, dv=128, pool=1024, state_dtype="bf16",
             io_dtype="bf16", mode="verify", n_pad=13),
    Workload("t4-f32", batch=32, T=4, Hk=4, Hv=8, dk=128, dv=128, pool=64, state_dtype="f32",
             io_dtype="f32", mode="verify", n_pad=3),
    Workload("dk64-dv80-f32-bf16io", batch=6, T=3, Hk=1, Hv=3, dk=64, dv=80, pool=9, state_dtype="f32",
             io_dtype="bf16", mode="verify", n_pad=1),
    Workload("dk16-bf16-f32io", batch=5, T=2, Hk=2, Hv=2, dk=16, dv=16, pool=7, state_dtype="bf16",
             io_dtype="f32", mode="verify", n_pad=1),
    Workload("dk256-bf16", batch=4, T=5, Hk=1, Hv=2, dk=256, dv=256, pool=6, state_dtype="bf16",
             io_dtype="bf16", mode="verify", n_pad=1),
]


RAW_WEAK = [s.replace(name=s.name + "-rawqk-weakdecay", qk="raw", decay="weak") for s in SHAPES]


@pytest.mark.parametrize("commit", [True, False])
@pytest.mark.parametrize("w", SHAPES + RAW_WEAK, ids=[s.name for s in SHAPES + RAW_WEAK])
def test_replay_parity(w, commit):
    """Replay lengths 0..T, with and without the commit, against the oracle. The
    rawqk-weakdecay shapes store q and k (new and replayed tokens) unnormalised and draw
    weak decays, so the replayed state carries its full weight into the new tokens."""
    say(f"[replay] {w.name} commit={commit}")
    x_prev, g_prev = dev_step(w, 1)
    x_cur, g_cur = dev_step(w, 2, x_prev["A_log"], x_prev["dt_bias"])
    x_cur["idx"] = x_prev["idx"]
    g_cur["idx"] = g_prev["idx"]
    rng = np.random.default_rng(3)
    rlen = rng.integers(0, w.T + 1, w.batch).astype(np.int32)     # includes 0: nothing replayed
    pool = to_device_state(x_prev["pool"]).to(DEV)
    pool0 = pool.clone()
    o = torch.full((w.batch, w.T, w.Hv, w.dv), float("nan"), dtype=x_cur["v"].dtype, device=DEV)
    gdn.gdn_verify_replay(g_cur["q"], g_cur["k"], g_cur["v"], g_cur["a"], g_cur["b"], g_cur["A_log"],
                          g_cur["dt_bias"], o, pool, g_cur["idx"], g_prev["k"], g_prev["v"], g_prev["a"],
                          g_prev["b"], torch.from_numpy(rlen).to(DEV), commit, scale=w.scale)
    torch.cuda.synchronize()
    idx = x_prev["idx"].numpy()
    ref = oracle_replay(w, x_cur, x_prev, f64(x_prev["pool"]), idx, rlen, commit)
    T_o = max(tol(w), 2e-2) if w.io_dtype == "bf16" else tol(w)
    o_err = max_abs(f64(o), ref["o"])
    gp = from_device_state(pool.cpu()).double().numpy()
    p_err = max_abs(gp, ref["pool"])
    say(f"[replay] {w.name}: o err {o_err:.2e}, pool err {p_err:.2e}")
    assert o_err <= T_o and p_err <= tol(w)
    valid = (idx >= 0) & (idx < w.pool)
    touched = np.zeros(w.pool, bool)
    if commit:
        touched[idx[valid & (rlen >= 1)]] = True
    ut = torch.from_numpy(np.nonzero(~touched)[0])
    assert torch.equal(pool[ut], pool0[ut])
    assert bool(torch.all(o[torch.from_numpy(~valid)] == 0))


@pytest.mark.parametrize("state", ["bf16", "f32"])
def test_commit_replay_equals_commit_of_intermediates(state):
    w = Workload("r", batch=16, T=4, Hk=2, Hv=4, dk=128, dv=128, pool=24, state_dtype=state, io_dtype=state,
                 mode="verify", n_pad=2)
    x, g = dev_step(w, 4)
    pool_a = to_device_state(x["pool"]).to(DEV)
    pool_b = pool_a.clone()
    cache = torch.zeros((w.batch, w.T, w.Hv, w.dv, w.dk), dtype=pool_a.dtype, device=DEV)
    o = torch.empty((w.batch, w.T, w.Hv, w.dv), dtype=x["v"].dtype, device=DEV)
    gdn.gdn_verify(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], o, pool_a, g["idx"], cache,
                   False, None, scale=w.scale)
    acc = torch.from_numpy(np.random.default_rng(5).integers(0, 6, w.batch).astype(np.int32)).to(DEV)
    gdn.gdn_commit(cache, g["idx"], acc, pool_a)
    gdn.gdn_commit_replay(g["A_log"], g["dt_bias"], pool_b, g["idx"], g["k"], g["v"], g["a"], g["b"], acc)
    torch.cuda.synchronize()
    assert torch.equal(pool_a, pool_b)


def test_fused_replay_equals_commit_replay_then_verify():
    w = SHAPES[0]
    x_prev, g_prev = dev_step(w, 6)
    x_cur, g_cur = dev_step(w, 7, x_prev["A_log"], x_prev["dt_bias"])
    g_cur["idx"] = g_prev["idx"]
    rlen = torch.from_numpy(np.random.default_rng(8).integers(0, w.T + 1, w.batch).astype(np.int32)).to(DEV)
    pool_a = to_device_state(x_prev["pool"]).to(DEV)
    pool_b = pool_a.clone()
    oa = torch.empty((w.batch, w.T, w.Hv, w.dv), dtype=torch.bfloat16, device=DEV)
    ob = torch.empty_like(oa)
    gdn.gdn_verify_replay(g_cur["q"], g_cur["k"], g_cur["v"], g_cur["a"], g_cur["b"], g_cur["A_log"],
                          g_cur["dt_bias"], oa, pool_a, g_cur["idx"], g_prev["k"], g_prev["v"], g_prev["a"],
                          g_prev["b"], rlen, True, scale=w.scale)
    gdn.gdn_commit_replay(g_cur["A_log"], g_cur["dt_bias"], pool_b, g_cur["idx"], g_prev["k"], g_prev["v"],
                          g_prev["a"], g_prev["b"], rlen)
    gdn.gdn_verify(g_cur["q"], g_cur["k"], g_cur["v"], g_cur["a"], g_cur["b"], g_cur["A_log"], g_cur["dt_bias"],
                   ob, pool_b, g_cur["idx"], None, False, None, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(pool_a, pool_b)
    assert torch.equal(oa, ob)


def test_zero_replay_equals_plain_verify():
    w = SHAPES[0]
    x_prev, g_prev = dev_step(w, 9)
    x_cur, g_cur = dev_step(w, 10)
    g_cur["idx"] = g_prev["idx"]
    pool = to_device_state(x_prev["pool"]).to(DEV)
    pool0 = pool.clone()
    oa = torch.empty((w.batch, w.T, w.Hv, w.dv), dtype=torch.bfloat16, device=DEV)
    ob = torch.empty_like(oa)
    gdn.gdn_verify_replay(g_cur["q"], g_cur["k"], g_cur["v"], g_cur["a"], g_cur["b"], g_cur["A_log"],
                          g_cur["dt_bias"], oa, pool, g_cur["idx"], g_prev["k"], g_prev["v"], g_prev["a"],
                          g_prev["b"], torch.zeros(w.batch, dtype=torch.int32, device=DEV), True, scale=w.scale)
    gdn.gdn_verify(g_cur["q"], g_cur["k"], g_cur["v"], g_cur["a"], g_cur["b"], g_cur["A_log"], g_cur["dt_bias"],
                   ob, pool, g_cur["idx"], None, False, None, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)
    assert torch.equal(pool, pool0)


@pytest.mark.parametrize("state", ["bf16", "f32"])
def test_replay_episode_equals_intermediate_path(state):
    """Six MTP steps: path A caches T states and commits from them, path B keeps the
    per-token inputs (two alternating buffers) and replays the accepted prefix in the
    next verify. Every output and the final pool agree bit for bit."""
    w = Workload("episode", batch=24, T=4, Hk=2, Hv=4, dk=128, dv=128, pool=40, state_dtype=state,
                 io_dtype=state, mode="verify", n_pad=3)
    x0, g0 = dev_step(w, 11)
    pool_a = to_device_state(x0["pool"]).to(DEV)
    pool_b = pool_a.clone()
    cache = torch.zeros((w.batch, w.T, w.Hv, w.dv, w.dk), dtype=pool_a.dtype, device=DEV)
    rng = np.random.default_rng(12)
    prev, rlen = g0, torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    for step in range(6):
        x, g = dev_step(w, 20 + step, x0["A_log"], x0["dt_bias"])
        g["idx"] = g0["idx"]
        oa = torch.empty((w.batch, w.T, w.Hv, w.dv), dtype=x["v"].dtype, device=DEV)
        ob = torch.empty_like(oa)
        gdn.gdn_verify(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], oa, pool_a, g["idx"],
                       cache, False, None, scale=w.scale)
        gdn.gdn_verify_replay(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], ob, pool_b,
                              g["idx"], prev["k"], prev["v"], prev["a"], prev["b"], rlen, True, scale=w.scale)
        acc = torch.from_numpy(rng.integers(1, w.T + 1, w.batch).astype(np.int32)).to(DEV)
        gdn.gdn_commit(cache, g["idx"], acc, pool_a)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"step {step}"
        prev, rlen = g, acc
    gdn.gdn_commit_replay(x0["A_log"].to(DEV), x0["dt_bias"].to(DEV), pool_b, g0["idx"], prev["k"], prev["v"],
                          prev["a"], prev["b"], rlen)
    torch.cuda.synchronize()
    assert torch.equal(pool_a, pool_b)


def test_replay_graph_capture():
    w = SHAPES[0]
    x_prev, st_prev = dev_step(w, 30)
    x_cur, st = dev_step(w, 31, x_prev["A_log"], x_prev["dt_bias"])
    st["idx"] = st_prev["idx"]
    st["rlen"] = torch.zeros(w.batch, dtype=torch.int32, device=DEV)
    st["pool"] = to_device_state(x_prev["pool"]).to(DEV)
    st["o"] = torch.empty((w.batch, w.T, w.Hv, w.dv), dtype=torch.bfloat16, device=DEV)

    def call(s, sp):
        gdn.gdn_verify_replay(s["q"], s["k"], s["v"], s["a"], s["b"], s["A_log"], s["dt_bias"], s["o"], s["pool"],
                              s["idx"], sp["k"], sp["v"], sp["a"], sp["b"], s["rlen"], True, scale=w.scale)
    call(st, st_prev)
    torch.cuda.synchronize()
    graph, stream = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=stream):
        call(st, st_prev)
    for rep in range(3):
        xp, rp = dev_step(w, 40 + rep)
        xc, rc = dev_step(w, 50 + rep, xp["A_log"], xp["dt_bias"])
        rc["idx"] = rp["idx"]
        rc["rlen"] = torch.from_numpy(np.random.default_rng(rep).integers(0, w.T + 1, w.batch).astype(np.int32)).to(DEV)
        rc["pool"] = to_device_state(xp["pool"]).to(DEV)
        rc["o"] = torch.empty_like(st["o"])
        for key in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx", "rlen", "pool"):
            st[key].copy_(rc[key])
        for key in ("k", "v", "a", "b"):
            st_prev[key].copy_(rp[key])
        torch.cuda.synchronize()
        graph.replay()
        call(rc, rp)
        torch.cuda.synchronize()
        assert torch.equal(st["o"], rc["o"]) and torch.equal(st["pool"], rc["pool"]), rep
