"""Pins of the oracle's prefill (pooled initial states, fresh mask, variable lengths)
against the already-pinned verify, against splitting a sequence at any token, and an
fp64 check of the chunked decomposition the GPU kernel uses:
    S_t = Gam_t S_0 + sum_{s<=t} (Gam_t / Gam_s) k^_s u_s^T,
    (I + A) U = diag(beta) V - diag(beta Gam) K^ S_0,  A_ts = beta_t (Gam_t/Gam_s) k^_t.k^_s (s < t),
    O = scale (diag(Gam) Q^ S_0 + (M o Q^ K^T) U),  M_ts = Gam_t / Gam_s (s <= t),
    S_C = Gam_C S_0 + K^T diag(Gam_C / Gam) U,
with Gam_t the product of the decays of the chunk's first t tokens."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import PrefillWorkload


def f64(t):
    return t.double().numpy()


def run(w, x, pool=None, fresh="x", idx=None):
    d = oracle.make_dims(w.batch, 1, w.Hk, w.Hv, w.dk, w.dv, w.pool, w.state_dtype == "bf16", scale=w.scale)
    return oracle.prefill(d, x["cu_seqlens"].numpy(), f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["a"]),
                          f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]),
                          f64(x["pool"]) if pool is None else pool, x["idx"].numpy() if idx is None else idx,
                          x["fresh"].numpy() if fresh == "x" else fresh)


SMALL = PrefillWorkload("p", seqlens=(7,), Hk=2, Hv=4, dk=8, dv=12, pool=3, state_dtype="f32", io_dtype="f32")


def test_single_sequence_equals_verify_with_write_back():
    w = SMALL
    x = workloads.make_prefill_inputs(w, seed=1)
    r = run(w, x, fresh=None)
    T = w.tokens
    d = oracle.make_dims(1, T, w.Hk, w.Hv, w.dk, w.dv, w.pool, False, scale=w.scale)
    v = oracle.verify(d, f64(x["q"])[None], f64(x["k"])[None], f64(x["v"])[None], f64(x["a"])[None],
                      f64(x["b"])[None], f64(x["A_log"]), f64(x["dt_bias"]), f64(x["pool"]), x["idx"].numpy(),
                      write_final=True)
    assert np.array_equal(r["o"], v["o"][0]) and np.array_equal(r["pool"], v["pool"])


def test_batch_equals_sequences_one_by_one_and_fresh_is_zero_start():
    w = workloads.PREFILL_WORKLOADS[0]
    x = workloads.make_prefill_inputs(w, seed=2)
    r = run(w, x)
    cu, idx, fresh = x["cu_seqlens"].numpy(), x["idx"].numpy(), x["fresh"].numpy()
    pool = f64(x["pool"])
    for s in range(w.batch):
        one = PrefillWorkload("one", seqlens=(w.seqlens[s],), Hk=w.Hk, Hv=w.Hv, dk=w.dk, dv=w.dv, pool=w.pool,
                              state_dtype=w.state_dtype, io_dtype=w.io_dtype)
        sl = slice(cu[s], cu[s + 1])
        xs = {n: x[n][sl] for n in ("q", "k", "v", "a", "b")}
        xs.update(A_log=x["A_log"], dt_bias=x["dt_bias"])
        xs["cu_seqlens"] = torch.tensor([0, w.seqlens[s]], dtype=torch.int32)
        xs["idx"] = torch.tensor([idx[s]], dtype=torch.int32)
        p0 = pool.copy()
        if fresh[s] and 0 <= idx[s] < w.pool:
            p0[idx[s]] = 0.0                       # fresh == a zeroed slot
        rs = run(one, xs, pool=p0, fresh=None)
        assert np.array_equal(rs["o"], r["o"][sl]), s
        if 0 <= idx[s] < w.pool:
            assert np.array_equal(rs["pool"][idx[s]], r["pool"][idx[s]]), s
    pad = idx < 0
    for s in np.nonzero(pad)[0]:
        assert np.all(r["o"][cu[s]:cu[s + 1]] == 0.0)
    touched = np.zeros(w.pool, bool); touched[idx[~pad]] = True
    assert np.array_equal(r["pool"][~touched], pool[~touched])


@pytest.mark.parametrize("cut", [1, 8, 16, 23])
def test_split_at_any_token_continues_from_the_pool(cut):
    """A sequence prefilled in two calls, the second starting from the state the first
    stored (a chunked prefill across scheduler steps), equals one call (fp32 state)."""
    w = PrefillWorkload("s", seqlens=(24,), Hk=1, Hv=2, dk=16, dv=8, pool=2, state_dtype="f32", io_dtype="f32")
    x = workloads.make_prefill_inputs(w, seed=3)
    whole = run(w, x, fresh=None)
    parts = []
    pool = f64(x["pool"])
    for sl in (slice(0, cut), slice(cut, 24)):
        xs = {n: x[n][sl] for n in ("q", "k", "v", "a", "b")}
        xs.update(A_log=x["A_log"], dt_bias=x["dt_bias"], idx=x["idx"],
                  cu_seqlens=torch.tensor([0, sl.stop - sl.start], dtype=torch.int32))
        wp = PrefillWorkload("p", seqlens=(sl.stop - sl.start,), Hk=1, Hv=2, dk=16, dv=8, pool=2,
                             state_dtype="f32", io_dtype="f32")
        r = run(wp, xs, pool=pool, fresh=None)
        parts.append(r["o"]); pool = r["pool"]
    assert np.array_equal(np.concatenate(parts), whole["o"]) and np.array_equal(pool, whole["pool"])


def test_bf16_pool_rounds_only_the_stored_state():
    w = PrefillWorkload("b", seqlens=(9, 4), Hk=1, Hv=2, dk=16, dv=16, pool=4, state_dtype="bf16", io_dtype="bf16")
    x = workloads.make_prefill_inputs(w, seed=4)
    rb = run(w, x)
    wf = PrefillWorkload("b", seqlens=(9, 4), Hk=1, Hv=2, dk=16, dv=16, pool=4, state_dtype="f32", io_dtype="bf16")
    rf = run(wf, x)                                  # the same bf16 start values, fp64 throughout
    assert np.array_equal(rb["o"], rf["o"])
    touched = x["idx"].numpy()
    rounded = np.vectorize(oracle.round_bf16)(rf["pool"][touched])
    assert np.array_equal(rb["pool"][touched], rounded)


def chunked_reference(q, k, v, a, b, A_log, dt_bias, S0, scale, C, eps=1e-6):
    """The chunked form of one (sequence, head) in fp64, written from the decomposition in
    the module docstring (not from the oracle)."""
    qh = q / np.sqrt((q * q).sum(-1, keepdims=True) + eps)
    kh = k / np.sqrt((k * k).sum(-1, keepdims=True) + eps)
    sp = np.maximum(a + dt_bias, 0) + np.log1p(np.exp(-np.abs(a + dt_bias)))
    logg = -np.exp(A_log) * sp
    beta = 1.0 / (1.0 + np.exp(-b))
    S = S0.copy()
    out = []
    for c0 in range(0, len(q), C):
        sl = slice(c0, min(c0 + C, len(q)))
        Q, K, V, lg, be = qh[sl], kh[sl], v[sl], logg[sl], beta[sl]
        G = np.cumsum(lg)
        ratio = np.exp(G[:, None] - G[None, :])
        KK = K @ K.T
        A = np.tril(be[:, None] * ratio * KK, -1)
        Tm = np.linalg.inv(np.eye(len(G)) + A)
        U = Tm @ (be[:, None] * V) - Tm @ ((be * np.exp(G))[:, None] * K) @ S
        M = np.tril(ratio)
        O = scale * (np.exp(G)[:, None] * (Q @ S) + (M * (Q @ K.T)) @ U)
        S = np.exp(G[-1]) * S + K.T @ (np.exp(G[-1] - G)[:, None] * U)
        out.append(O)
    return np.concatenate(out), S


@pytest.mark.parametrize("C", [1, 4, 16, 32])
def test_chunked_decomposition_equals_the_recurrence(C):
    w = PrefillWorkload("c", seqlens=(45,), Hk=1, Hv=1, dk=16, dv=8, pool=1, state_dtype="f32", io_dtype="f32")
    x = workloads.make_prefill_inputs(w, seed=5)
    r = run(w, x, fresh=None)
    o, S = chunked_reference(f64(x["q"])[:, 0], f64(x["k"])[:, 0], f64(x["v"])[:, 0], f64(x["a"])[:, 0],
                             f64(x["b"])[:, 0], f64(x["A_log"])[0], f64(x["dt_bias"])[0], f64(x["pool"])[0, 0],
                             w.scale, C)
    np.testing.assert_allclose(o, r["o"][:, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, r["pool"][0, 0], rtol=0, atol=1e-12)
