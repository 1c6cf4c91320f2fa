"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each test names the fact it checks: a closed form, an invariant of the gated delta
rule, a special case that reduces to plain linear algebra, a hand-worked example, or
brute force in another formulation (matrix form, 50-digit arithmetic). Together they
are chosen so that a dropped term, a wrong sign, a wrong index or a transposed
operand anywhere in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest

import workloads

INF = float("inf")


def run(orc, *, S0, q, k, v, a, b, A_log, dt_bias, bf16=False, eps=1e-6, scale=None,
        cache=True, write_final=True):
    """Single pool slot, single row: S0 [Hv,dk,dv]; q,k [T,Hk,dk]; v [T,Hv,dv]; a,b [T,Hv]."""
    T, Hk, dk = q.shape
    Hv, _, dv = S0.shape
    dims = orc.make_dims(1, T, Hk, Hv, dk, dv, 1, bf16, scale=scale, eps=eps)
    r = orc.verify(dims, q[None], k[None], v[None], a[None], b[None], A_log, dt_bias,
                   S0[None], np.array([0], np.int32), cache_T=T if cache else 0,
                   write_final=write_final, nthreads=1)
    return dict(o=r["o"][0], pool=r["pool"][0], cache=None if r["cache"] is None else r["cache"][0])


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- gates

def test_softplus_closed_forms(orc):
    assert orc.softplus(0.0) == pytest.approx(math.log(2.0), rel=0, abs=1e-16)
    assert orc.softplus(-INF) == 0.0
    assert orc.softplus(40.0) == pytest.approx(40.0, rel=1e-16)
    assert orc.softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-15)
    # log(1 + e) at x = 1
    assert orc.softplus(1.0) == pytest.approx(1.3132616875182228, rel=1e-15)


def test_gate_closed_forms(orc):
    # A_log = 0, dt_bias = 0: g = exp(-softplus(a)) = 1 / (1 + e^a)
    for x in (-3.0, -0.5, 0.0, 0.7, 2.5):
        g, _ = orc.gates(x, 0.0, 0.0, 0.0)
        assert g == pytest.approx(1.0 / (1.0 + math.exp(x)), rel=1e-14)
    # A_log = ln 2, a + dt_bias = 0: g = exp(-2 ln 2) = 1/4; dt_bias shifts a
    g, _ = orc.gates(0.25, 0.0, math.log(2.0), -0.25)
    assert g == pytest.approx(0.25, rel=1e-15)
    # a = -inf: no decay at all, exactly
    g, _ = orc.gates(-INF, 0.0, 1.3, 0.2)
    assert g == 1.0
    # beta = sigmoid(b)
    assert orc.gates(0.0, 0.0, 0.0, 0.0)[1] == 0.5
    assert orc.gates(0.0, -INF, 0.0, 0.0)[1] == 0.0
    assert orc.gates(0.0, INF, 0.0, 0.0)[1] == 1.0
    assert orc.gates(0.0, 1.0, 0.0, 0.0)[1] == pytest.approx(math.e / (1.0 + math.e), rel=1e-15)
    # the decay only grows with A_log and with a: g in (0, 1]
    gs = [orc.gates(x, 0.0, al, 0.0)[0] for al in (0.0, 1.0, 2.0) for x in (-1.0, 0.0, 1.0)]
    assert all(0.0 < x <= 1.0 for x in gs)
    assert gs[0] > gs[1] > gs[2] and gs[0] > gs[3] > gs[6]


# ---------------------------------------------------------------- recurrence closed forms

def test_one_step_from_zero_state(orc):
    """S0 = 0: S1 = beta k^ v^T and o = beta (k^.q^) scale v (o read from the updated S)."""
    rng = np.random.default_rng(1)
    dk, dv = 8, 5
    q = rng.standard_normal((1, 1, dk)) * 3.0   # not unit: the oracle must normalise
    k = rng.standard_normal((1, 1, dk)) * 0.5
    v = rng.standard_normal((1, 1, dv))
    a, b = np.array([[0.3]]), np.array([[-0.4]])
    A_log, dt = np.array([0.9]), np.array([0.1])
    r = run(orc, S0=np.zeros((1, dk, dv)), q=q, k=k, v=v, a=a, b=b, A_log=A_log, dt_bias=dt, eps=0.0)
    beta = 1.0 / (1.0 + math.exp(0.4))
    kh, qh = unit(k[0, 0]), unit(q[0, 0])
    np.testing.assert_allclose(r["cache"][0, 0], beta * np.outer(kh, v[0, 0]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["o"][0, 0], beta * (kh @ qh) * v[0, 0] / math.sqrt(dk), rtol=0, atol=1e-15)


def test_decay_only(orc):
    """beta = 0: S_T = (prod g_t) S0 and o_t = scale * g_1..g_t * S0^T q^_t."""
    rng = np.random.default_rng(2)
    T, dk, dv = 3, 6, 4
    S0 = rng.standard_normal((1, dk, dv))
    q = rng.standard_normal((T, 1, dk))
    k = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    a = rng.standard_normal((T, 1))
    b = np.full((T, 1), -INF)
    A_log, dt = np.array([0.4]), np.array([-0.2])
    r = run(orc, S0=S0, q=q, k=k, v=v, a=a, b=b, A_log=A_log, dt_bias=dt, eps=0.0)
    G = 1.0
    for t in range(T):
        G *= math.exp(-math.exp(0.4) * math.log1p(math.exp(a[t, 0] - 0.2)))
        np.testing.assert_allclose(r["cache"][t, 0], G * S0[0], rtol=1e-14, atol=0)
        np.testing.assert_allclose(r["o"][t, 0], G * S0[0].T @ unit(q[t, 0]) / math.sqrt(dk), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("bf16", [False, True])
def test_identity_gates_bit_exact(orc, bf16):
    """g = 1 (a = -inf) and beta = 0 (b = -inf): every stored state is S0, bit for bit."""
    rng = np.random.default_rng(3)
    T, dk, dv = 4, 8, 8
    S0 = rng.standard_normal((2, dk, dv)).astype(np.float32).astype(np.float64)
    if bf16:
        S0 = np.vectorize(orc.round_bf16)(S0)
    r = run(orc, S0=S0, q=rng.standard_normal((T, 1, dk)), k=rng.standard_normal((T, 1, dk)),
            v=rng.standard_normal((T, 2, dv)), a=np.full((T, 2), -INF), b=np.full((T, 2), -INF),
            A_log=np.array([0.5, 1.5]), dt_bias=np.array([0.0, 0.3]), bf16=bf16)
    for t in range(T):
        assert np.array_equal(r["cache"][t], S0)
    assert np.array_equal(r["pool"], S0)


@pytest.mark.parametrize("a_val", [-1.0, 0.0, 2.0])
def test_delta_property(orc, a_val):
    """beta = 1 and unit k^: the updated state maps k^ onto v exactly (S'^T k^ = v), for any decay."""
    rng = np.random.default_rng(4)
    dk, dv = 16, 12
    S0 = rng.standard_normal((1, dk, dv))           # not symmetric, not square
    k = unit(rng.standard_normal((1, 1, dk)))
    v = rng.standard_normal((1, 1, dv))
    r = run(orc, S0=S0, q=rng.standard_normal((1, 1, dk)), k=k, v=v, a=np.array([[a_val]]),
            b=np.array([[INF]]), A_log=np.array([0.3]), dt_bias=np.array([0.0]), eps=0.0)
    S1 = r["cache"][0, 0]
    np.testing.assert_allclose(S1.T @ k[0, 0], v[0, 0], rtol=0, atol=1e-14)
    # and the state moved only along k: (I - k k^T) S1 = g (I - k k^T) S0
    P = np.eye(dk) - np.outer(k[0, 0], k[0, 0])
    g = math.exp(-math.exp(0.3) * math.log1p(math.exp(a_val)))
    np.testing.assert_allclose(P @ S1, g * (P @ S0[0]), rtol=0, atol=1e-14)


def test_associative_recall(orc):
    """S0 = 0, g = 1, beta = 1, orthonormal keys k_1..k_T: after T writes S^T k_t = v_t for every t."""
    rng = np.random.default_rng(5)
    T, dk, dv = 6, 8, 5
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Q[:T].reshape(T, 1, dk)
    v = rng.standard_normal((T, 1, dv))
    r = run(orc, S0=np.zeros((1, dk, dv)), q=k.copy(), k=k, v=v, a=np.full((T, 1), -INF),
            b=np.full((T, 1), INF), A_log=np.array([0.0]), dt_bias=np.array([0.0]), eps=0.0, scale=1.0)
    S = r["pool"][0]
    for t in range(T):
        np.testing.assert_allclose(S.T @ k[t, 0], v[t, 0], rtol=0, atol=1e-13)
    # o_t read with q = k_t right after writing it returns v_t
    for t in range(T):
        np.testing.assert_allclose(r["o"][t, 0], v[t, 0], rtol=0, atol=1e-13)


def _read_golden(path):
    vals = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            key, val = line.split("=")
            vals[key.strip()] = [float(x) for x in val.split()]
    return vals


def test_scalar_case_by_hand(orc):
    """d_k = d_v = 1 worked by hand: see tests/golden/scalar_two_steps.txt."""
    import os
    g = _read_golden(os.path.join(os.path.dirname(__file__), "golden", "scalar_two_steps.txt"))
    T = 2
    r = run(orc, S0=np.array(g["s0"]).reshape(1, 1, 1), q=np.array(g["q"]).reshape(T, 1, 1),
            k=np.array(g["k"]).reshape(T, 1, 1), v=np.array(g["v"]).reshape(T, 1, 1),
            a=np.array(g["a"]).reshape(T, 1), b=np.array(g["b"]).reshape(T, 1),
            A_log=np.array(g["A_log"]), dt_bias=np.array(g["dt_bias"]), eps=0.0, scale=1.0)
    np.testing.assert_allclose(r["cache"][:, 0, 0, 0], g["s"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["o"][:, 0, 0], g["o"], rtol=0, atol=1e-15)


# ---------------------------------------------------------------- brute force in another form

def _gates_np(a, b, A_log, dt_bias):
    g = np.exp(-np.exp(A_log) * np.logaddexp(0.0, a + dt_bias))
    beta = 0.5 * (1.0 + np.tanh(0.5 * b))   # sigmoid written another way
    return g, beta


def matrix_form(S0, q, k, v, a, b, A_log, dt_bias, Hk, eps, scale):
    """S_t = g_t (I - beta_t k k^T) S_{t-1} + beta_t k v^T per (row, v-head); o_t = scale S_t^T q."""
    B, T = q.shape[:2]
    Hv, dk, dv = S0.shape[1:]
    G = Hv // Hk
    o = np.zeros((B, T, Hv, dv))
    cache = np.zeros((B, T, Hv, dk, dv))
    for r in range(B):
        for h in range(Hv):
            S = S0[r, h].copy()
            for t in range(T):
                kk = k[r, t, h // G] / np.sqrt(k[r, t, h // G] @ k[r, t, h // G] + eps)
                qq = q[r, t, h // G] / np.sqrt(q[r, t, h // G] @ q[r, t, h // G] + eps)
                g, beta = _gates_np(a[r, t, h], b[r, t, h], A_log[h], dt_bias[h])
                S = g * (np.eye(dk) - beta * np.outer(kk, kk)) @ S + beta * np.outer(kk, v[r, t, h])
                cache[r, t, h] = S
                o[r, t, h] = scale * S.T @ qq
    return o, cache


def test_brute_force_matrix_form_tiny_workload(orc):
    w = workloads.WORKLOADS[0]
    x = workloads.make_inputs(w, seed=0)
    f = {n: x[n].double().numpy() for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "pool")}
    idx = x["idx"].numpy()
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, False)
    r = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"],
                   idx, cache_T=w.T, write_final=True)
    o_ref, c_ref = matrix_form(f["pool"][idx], f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"],
                               f["dt_bias"], w.Hk, 1e-6, w.scale)
    np.testing.assert_allclose(r["o"], o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["cache"], c_ref, rtol=0, atol=1e-13)


def test_brute_force_rectangular_grouped_heads(orc):
    """d_k != d_v, 3 v-heads per k-head, several rows, non-trivial slot map."""
    rng = np.random.default_rng(6)
    B, T, Hk, Hv, dk, dv, P = 3, 3, 2, 6, 5, 7, 5
    q = rng.standard_normal((B, T, Hk, dk)); k = rng.standard_normal((B, T, Hk, dk))
    v = rng.standard_normal((B, T, Hv, dv)); a = rng.standard_normal((B, T, Hv)); b = rng.standard_normal((B, T, Hv))
    A_log = np.log(rng.uniform(1, 16, Hv)); dt = rng.normal(0, 0.1, Hv)
    pool = rng.normal(0, 0.1, (P, Hv, dk, dv))
    idx = np.array([4, 1, 2], np.int32)
    dims = orc.make_dims(B, T, Hk, Hv, dk, dv, P, False)
    r = orc.verify(dims, q, k, v, a, b, A_log, dt, pool, idx, cache_T=T, write_final=True)
    o_ref, c_ref = matrix_form(pool[idx], q, k, v, a, b, A_log, dt, Hk, 1e-6, dk ** -0.5)
    np.testing.assert_allclose(r["o"], o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["cache"], c_ref, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(r["pool"][idx], r["cache"][:, -1])
    untouched = [s for s in range(P) if s not in idx]
    np.testing.assert_array_equal(r["pool"][untouched], pool[untouched])


def test_fifty_digit_reference_tiny_workload(orc):
    """The oracle's float64 error on the tiny workload, against a 50-digit matrix-form run."""
    mpmath = pytest.importorskip("mpmath")
    mp = mpmath.mp
    mp.dps = 50
    w = workloads.WORKLOADS[0]
    x = workloads.make_inputs(w, seed=0)
    f = {n: x[n].double().numpy() for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "pool")}
    idx = x["idx"].numpy()
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, False)
    r = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"],
                   idx, cache_T=w.T)
    eps = mp.mpf("1e-6")
    worst = 0.0
    for row in range(w.batch):
        for h in range(w.Hv):
            S = mp.matrix(f["pool"][idx[row], h].tolist())
            for t in range(w.T):
                kv = mp.matrix(f["k"][row, t, h // (w.Hv // w.Hk)].tolist())
                qv = mp.matrix(f["q"][row, t, h // (w.Hv // w.Hk)].tolist())
                kv = kv / mp.sqrt(sum(x_ * x_ for x_ in kv) + eps)
                qv = qv / mp.sqrt(sum(x_ * x_ for x_ in qv) + eps)
                x_ = mp.mpf(f["a"][row, t, h]) + mp.mpf(f["dt_bias"][h])
                g = mp.exp(-mp.exp(mp.mpf(f["A_log"][h])) * mp.log(1 + mp.exp(x_)))
                beta = 1 / (1 + mp.exp(-mp.mpf(f["b"][row, t, h])))
                vv = mp.matrix(f["v"][row, t, h].tolist())
                S = g * (mp.eye(w.dk) - beta * kv * kv.T) * S + beta * kv * vv.T
                o = (S.T * qv) * (1 / mp.sqrt(w.dk))
                for j in range(w.dv):
                    worst = max(worst, abs(float(o[j] - mp.mpf(r["o"][row, t, h, j]))))
                    for i in range(w.dk):
                        worst = max(worst, abs(float(S[i, j] - mp.mpf(r["cache"][row, t, h, i, j]))))
    assert worst < 1e-13, worst


# ---------------------------------------------------------------- bookkeeping of the driver

def _workload_f64(w, seed=0):
    x = workloads.make_inputs(w, seed=seed)
    f = {n: x[n].double().numpy() for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "pool")}
    f["idx"] = x["idx"].numpy()
    for n in ("accept", "prev_accept"):
        if n in x:
            f[n] = x[n].numpy()
    if "cache_prev" in x:
        f["cache_prev"] = x["cache_prev"].double().numpy()
    return f


SMALL = workloads.Workload("small-grouped", batch=6, T=4, Hk=2, Hv=4, dk=8, dv=12, pool=9,
                           state_dtype="f32", io_dtype="f32", mode="verify", cache_T=5, n_pad=2)


@pytest.mark.parametrize("bf16", [False, True])
def test_verify_equals_successive_decodes(orc, bf16):
    """T-token verify = T single-token decodes, bit for bit: cache[t] is the pool after t+1 decodes."""
    w = SMALL
    f = _workload_f64(w)
    pool0 = np.vectorize(orc.round_bf16)(f["pool"]) if bf16 else f["pool"]
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, bf16)
    r = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], pool0,
                   f["idx"], cache_T=w.cache_T, write_final=True)
    d1 = orc.make_dims(w.batch, 1, w.Hk, w.Hv, w.dk, w.dv, w.pool, bf16)
    pool = pool0.copy()
    valid = f["idx"] >= 0
    for t in range(w.T):
        s = slice(t, t + 1)
        rd = orc.decode(d1, f["q"][:, s], f["k"][:, s], f["v"][:, s], f["a"][:, s], f["b"][:, s],
                        f["A_log"], f["dt_bias"], pool, f["idx"])
        pool = rd["pool"]
        assert np.array_equal(rd["o"][:, 0], r["o"][:, t])
        assert np.array_equal(pool[f["idx"][valid]], r["cache"][valid, t])
    assert np.array_equal(pool, r["pool"])


def test_padding_rows_and_untouched_memory(orc):
    w = SMALL
    f = _workload_f64(w)
    sentinel = np.full((w.batch, w.cache_T, w.Hv, w.dk, w.dv), 7.25)
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, False)
    r = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"],
                   f["idx"], cache_T=w.cache_T, cache_in=sentinel)
    pad = f["idx"] < 0
    assert pad.sum() == 2
    assert np.all(r["o"][pad] == 0.0)
    assert np.all(r["cache"][pad] == 7.25)            # padding rows: cache untouched
    assert np.all(r["cache"][~pad, w.T:] == 7.25)      # slots t >= T untouched
    assert np.array_equal(r["pool"], f["pool"])        # verify without write_final: pool read-only
    # every valid row equals a one-row run on its own slot
    for row in np.nonzero(~pad)[0]:
        d1 = orc.make_dims(1, w.T, w.Hk, w.Hv, w.dk, w.dv, 1, False)
        sl = slice(row, row + 1)
        r1 = orc.verify(d1, f["q"][sl], f["k"][sl], f["v"][sl], f["a"][sl], f["b"][sl], f["A_log"],
                        f["dt_bias"], f["pool"][f["idx"][row]][None], np.array([0], np.int32), cache_T=w.T)
        assert np.array_equal(r1["o"][0], r["o"][row])
        assert np.array_equal(r1["cache"][0], r["cache"][row, :w.T])


def test_out_of_range_index_is_padding(orc):
    w = SMALL
    f = _workload_f64(w)
    idx = f["idx"].copy()
    idx[0] = w.pool          # one past the end
    idx[1] = -7
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, False)
    r = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"],
                   idx, cache_T=w.cache_T, write_final=True)
    assert np.all(r["o"][:2] == 0.0)


def test_head_sharing_reading(orc):
    """v-head h reads k-head h // (Hv/Hk): each v-head equals a one-head run on that k-head."""
    w = SMALL
    f = _workload_f64(w)
    G = w.Hv // w.Hk
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, False)
    r = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"],
                   f["idx"], cache_T=w.T)
    d1 = orc.make_dims(w.batch, w.T, 1, 1, w.dk, w.dv, w.pool, False)
    for h in range(w.Hv):
        kh = h // G
        r1 = orc.verify(d1, f["q"][:, :, kh:kh + 1], f["k"][:, :, kh:kh + 1], f["v"][:, :, h:h + 1],
                        f["a"][:, :, h:h + 1], f["b"][:, :, h:h + 1], f["A_log"][h:h + 1],
                        f["dt_bias"][h:h + 1], f["pool"][:, h:h + 1], f["idx"], cache_T=w.T)
        assert np.array_equal(r1["o"][:, :, 0], r["o"][:, :, h])


def test_commit_equals_intermediate(orc):
    w = SMALL
    f = _workload_f64(w)
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, True)
    r = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"],
                   f["idx"], cache_T=w.cache_T)
    acc = np.array([1, 4, 0, 3, 6, 2], np.int32)   # 0 and 6 (> cache_T) are skipped
    pool = orc.commit(dims, r["cache"], w.cache_T, f["idx"], acc, f["pool"])
    for row, s in enumerate(f["idx"]):
        n = acc[row]
        if s < 0 or n < 1 or n > w.cache_T:
            continue
        assert np.array_equal(pool[s], r["cache"][row, n - 1])
    touched = {f["idx"][r_] for r_ in range(w.batch) if f["idx"][r_] >= 0 and 1 <= acc[r_] <= w.cache_T}
    for s in range(w.pool):
        if s not in touched:
            assert np.array_equal(pool[s], f["pool"][s])


def test_write_final_equals_last_intermediate(orc):
    w = SMALL
    f = _workload_f64(w)
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, True)
    r = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"],
                   f["idx"], cache_T=w.cache_T, write_final=True)
    valid = f["idx"] >= 0
    assert np.array_equal(r["pool"][f["idx"][valid]], r["cache"][valid, w.T - 1])


def test_fused_commit_equals_commit_then_verify(orc):
    w = workloads.Workload("fused-small", batch=5, T=3, Hk=1, Hv=2, dk=8, dv=8, pool=7,
                           state_dtype="bf16", io_dtype="bf16", mode="verify_fused", cache_T=4, n_pad=1)
    f = _workload_f64(w)
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, True)
    fused = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"],
                       f["idx"], cache_T=w.cache_T, prev_accept=f["prev_accept"], cache_in=f["cache_prev"])
    pool1 = orc.commit(dims, f["cache_prev"], w.cache_T, f["idx"], f["prev_accept"], f["pool"])
    plain = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], pool1,
                       f["idx"], cache_T=w.cache_T, cache_in=f["cache_prev"])
    for key in ("o", "pool", "cache"):
        assert np.array_equal(fused[key], plain[key])
    # the committed slot differs from the original one, so the fused read was not the pool's
    valid = f["idx"] >= 0
    assert not np.array_equal(pool1[f["idx"][valid]], f["pool"][f["idx"][valid]])


@pytest.mark.parametrize("bf16", [False, True])
def test_bf16_mode_stores_bf16_values(orc, bf16):
    w = SMALL
    f = _workload_f64(w)
    dims = orc.make_dims(w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool, bf16)
    r = orc.verify(dims, f["q"], f["k"], f["v"], f["a"], f["b"], f["A_log"], f["dt_bias"], f["pool"],
                   f["idx"], cache_T=w.T)
    valid = f["idx"] >= 0
    c = r["cache"][valid]
    import torch
    rt = torch.from_numpy(c).to(torch.bfloat16).double().numpy()
    if bf16:
        assert np.array_equal(rt, c)
    else:
        assert not np.array_equal(rt, c)


def test_oracle_matches_its_golden_fixture(orc):
    """Regression guard: the oracle still reproduces tests/golden/tiny_verify_oracle.txt."""
    import os
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_golden
    g = _read_golden(os.path.join(os.path.dirname(__file__), "golden", "tiny_verify_oracle.txt"))
    r = make_golden.compute()
    np.testing.assert_allclose(r["o"].ravel(), g["o"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(r["cache"][0, 1, 1].ravel(), g["cache_0_1_1"], rtol=0, atol=1e-15)


def test_l2norm_eps_closed_form(orc):
    """A key of norm 1e-3 with eps = 1e-6 is scaled by 1 / sqrt(|k|^2 + eps) = 1 / sqrt(2e-6),
    so from S0 = 0 one token stores beta k vT / sqrt(2e-6) (a normalised length of 1/sqrt 2,
    not 1); a zero query gives o = 0 and a zero key leaves the decayed state, with no NaN."""
    rng = np.random.default_rng(21)
    dk, dv = 8, 3
    kdir = unit(rng.standard_normal(dk))
    k = (kdir * 1e-3)[None, None]
    q = rng.standard_normal((1, 1, dk))
    v = rng.standard_normal((1, 1, dv))
    b = np.array([[0.2]])
    beta = 1.0 / (1.0 + math.exp(-0.2))
    r = run(orc, S0=np.zeros((1, dk, dv)), q=q, k=k, v=v, a=np.array([[0.1]]), b=b, A_log=np.array([0.0]),
            dt_bias=np.array([0.0]), eps=1e-6)
    np.testing.assert_allclose(r["cache"][0, 0], beta * np.outer(k[0, 0], v[0, 0]) / math.sqrt(2e-6),
                               rtol=1e-13, atol=0)
    # zero query: o = 0 exactly; zero key: S1 = g S0
    S0 = rng.standard_normal((1, dk, dv))
    r = run(orc, S0=S0, q=np.zeros((1, 1, dk)), k=np.zeros((1, 1, dk)), v=v, a=np.array([[0.1]]), b=b,
            A_log=np.array([0.0]), dt_bias=np.array([0.0]), eps=1e-6)
    g = 1.0 / (1.0 + math.exp(0.1))
    assert np.all(r["o"] == 0.0)
    np.testing.assert_allclose(r["cache"][0, 0], g * S0[0], rtol=1e-15, atol=0)
