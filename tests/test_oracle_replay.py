"""Pins of the oracle's cached replay against the oracle's already-pinned verify and
commit: replaying the accepted prefix of an earlier verify from the checkpoint state must
give, bit for bit, the state that verify cached after that many tokens."""
import numpy as np
import pytest

import workloads

W = workloads.Workload("replay-small", batch=7, T=4, Hk=2, Hv=4, dk=8, dv=12, pool=10,
                       state_dtype="f32", io_dtype="f32", mode="verify", cache_T=4, n_pad=2)


def f64(x):
    return {n: x[n].double().numpy() for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "pool")}


def step_inputs(w, seed):
    x = workloads.make_inputs(w, seed=seed)
    return f64(x), x["idx"].numpy()


@pytest.mark.parametrize("bf16", [False, True])
def test_commit_replay_equals_commit_of_intermediates(orc, bf16):
    w = W
    f, idx = step_inputs(w, 1)
    pool0 = np.vectorize(orc.round_bf16)(f["pool"]) if bf16 else f["pool"]
    d = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, bf16)
    r = orc.verify(d, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], pool0, idx,
                   cache_T=w.T)
    acc = np.array([1, 4, 0, 2, 5, 3, 1], np.int32)       # 0 and 5 (> T) are skipped
    by_cache = orc.commit(d, r["cache"], w.T, idx, acc, pool0)
    by_replay = orc.commit_replay(d, f["A_log"], f["dt_bias"], pool0, idx, f["k"], f["v"], f["a"], f["b"], acc)
    assert np.array_equal(by_cache, by_replay)
    assert not np.array_equal(by_replay, pool0)


@pytest.mark.parametrize("bf16", [False, True])
def test_fused_replay_equals_commit_replay_then_verify(orc, bf16):
    w = W
    prev, idx = step_inputs(w, 2)
    cur, _ = step_inputs(w, 3)
    pool0 = np.vectorize(orc.round_bf16)(prev["pool"]) if bf16 else prev["pool"]
    d = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, bf16)
    n = np.array([3, 0, 4, 1, 2, 4, 7], np.int32)        # 7 > rT: replays nothing
    fused = orc.verify_replay(d, cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], cur["A_log"], cur["dt_bias"],
                              pool0, idx, prev["k"], prev["v"], prev["a"], prev["b"], n, commit=True)
    pool1 = orc.commit_replay(d, cur["A_log"], cur["dt_bias"], pool0, idx, prev["k"], prev["v"], prev["a"],
                              prev["b"], n)
    plain = orc.verify(d, cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], cur["A_log"], cur["dt_bias"], pool1, idx)
    assert np.array_equal(fused["pool"], pool1)
    assert np.array_equal(fused["o"], plain["o"])
    # without the commit: same outputs, pool untouched
    nocommit = orc.verify_replay(d, cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], cur["A_log"],
                                 cur["dt_bias"], pool0, idx, prev["k"], prev["v"], prev["a"], prev["b"], n,
                                 commit=False)
    assert np.array_equal(nocommit["o"], fused["o"])
    assert np.array_equal(nocommit["pool"], pool0)


def test_zero_replay_is_plain_verify(orc):
    w = W
    prev, idx = step_inputs(w, 4)
    cur, _ = step_inputs(w, 5)
    d = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, False)
    z = np.zeros(w.batch, np.int32)
    rep = orc.verify_replay(d, cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], cur["A_log"], cur["dt_bias"],
                            prev["pool"], idx, prev["k"], prev["v"], prev["a"], prev["b"], z, commit=True)
    plain = orc.verify(d, cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], cur["A_log"], cur["dt_bias"],
                       prev["pool"], idx)
    assert np.array_equal(rep["o"], plain["o"])
    assert np.array_equal(rep["pool"], prev["pool"])
    pad = idx < 0
    assert np.all(rep["o"][pad] == 0.0)


@pytest.mark.parametrize("bf16", [False, True])
def test_replay_episode_equals_intermediate_path(orc, bf16):
    """Five MTP steps. Path A keeps T states per token and commits from them; path B keeps
    only the per-token inputs and replays the accepted prefix at the start of the next
    verify. Outputs of every step and the final pool are identical."""
    w = W
    d = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, bf16)
    f0, idx = step_inputs(w, 6)
    pool_a = np.vectorize(orc.round_bf16)(f0["pool"]) if bf16 else f0["pool"]
    pool_b = pool_a.copy()
    rng = np.random.default_rng(7)
    prev = None
    n_prev = np.zeros(w.batch, np.int32)
    for step in range(5):
        cur, _ = step_inputs(w, 10 + step)
        cur["A_log"], cur["dt_bias"] = f0["A_log"], f0["dt_bias"]   # per-layer parameters
        ra = orc.verify(d, cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], cur["A_log"], cur["dt_bias"],
                        pool_a, idx, cache_T=w.T)
        src = prev if prev is not None else cur
        rb = orc.verify_replay(d, cur["q"], cur["k"], cur["v"], cur["a"], cur["b"], cur["A_log"], cur["dt_bias"],
                               pool_b, idx, src["k"], src["v"], src["a"], src["b"], n_prev, commit=True)
        assert np.array_equal(ra["o"], rb["o"]), step
        pool_b = rb["pool"]
        acc = rng.integers(1, w.T + 1, w.batch).astype(np.int32)
        pool_a = orc.commit(d, ra["cache"], w.T, idx, acc, pool_a)
        prev, n_prev = cur, acc
    pool_b = orc.commit_replay(d, f0["A_log"], f0["dt_bias"], pool_b, idx, prev["k"], prev["v"], prev["a"],
                               prev["b"], n_prev)
    assert np.array_equal(pool_a, pool_b)
