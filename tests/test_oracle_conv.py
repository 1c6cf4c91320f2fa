"""Pins of the short-convolution oracle (conv_update, conv_commit) against facts that do
not come from it: numpy's convolution for the identity activation, closed forms of SiLU,
array slicing for the state after a commit, and the equivalences a speculative verify
and commit must keep (verify + commit of n == n decodes, fused == commit then verify)."""
import math

import numpy as np
import pytest

import oracle
import workloads


def rand_case(rng, B=4, T=3, D=8, K=4, P=6, pad=(1,)):
    idx = rng.permutation(P)[:B].astype(np.int32)
    for r in pad:
        idx[r] = -1
    return dict(x=rng.standard_normal((B, T, D)), w=rng.standard_normal((K, D)), bias=rng.standard_normal(D),
                pool=rng.standard_normal((P, K - 1, D)), idx=idx)


@pytest.mark.parametrize("K", [2, 3, 4, 6])
def test_identity_activation_is_numpy_convolution(K):
    rng = np.random.default_rng(K)
    c = rand_case(rng, K=K)
    B, T, D = c["x"].shape
    d = oracle.make_conv_dims(B, T, D, K, c["pool"].shape[0], activation="none")
    y = oracle.conv_update(d, c["x"], c["w"], None, c["pool"], c["idx"])["y"]
    for r in range(B):
        s = c["idx"][r]
        for ch in range(D):
            if s < 0:
                assert np.all(y[r, :, ch] == 0.0)
                continue
            seq = np.concatenate([c["pool"][s, :, ch], c["x"][r, :, ch]])
            ref = np.convolve(seq, c["w"][::-1, ch], mode="valid")
            np.testing.assert_allclose(y[r, :, ch], ref, rtol=0, atol=1e-13)


def test_silu_closed_forms():
    # single newest tap: y = silu(x + bias)
    xs = np.array([0.0, 1.0, -1.0, math.log(3.0), 2.5])
    D = len(xs)
    w = np.zeros((4, D)); w[3] = 1.0
    bias = np.array([0.0, 0.0, 0.0, 0.0, -2.5])
    d = oracle.make_conv_dims(1, 1, D, 4, 1)
    y = oracle.conv_update(d, xs.reshape(1, 1, D), w, bias, np.zeros((1, 3, D)), np.array([0]))["y"][0, 0]
    e = math.e
    expect = [0.0, e / (1.0 + e), -1.0 / (1.0 + e), 0.75 * math.log(3.0), 0.0]
    np.testing.assert_allclose(y, expect, rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("K", [2, 4, 5])
def test_commit_keeps_the_last_inputs(K):
    rng = np.random.default_rng(10 + K)
    c = rand_case(rng, B=5, T=4, K=K, P=7, pad=(2,))
    B, T, D = c["x"].shape
    d = oracle.make_conv_dims(B, T, D, K, 7)
    acc = np.array([1, 4, 3, 0, 6], np.int32)            # 0 and 6 (> T) are skipped
    new = oracle.conv_commit(d, c["x"], c["pool"], c["idx"], acc)
    ref = c["pool"].copy()
    for r in range(B):
        s, n = c["idx"][r], acc[r]
        if s < 0 or not 1 <= n <= T:
            continue
        ref[s] = np.concatenate([c["pool"][s], c["x"][r, :n]], axis=0)[-(K - 1):]
    assert np.array_equal(new, ref)


@pytest.mark.parametrize("act", ["none", "silu"])
def test_verify_then_commit_equals_decodes(act):
    rng = np.random.default_rng(3)
    c = rand_case(rng, B=4, T=5, D=8, K=4, P=6, pad=(0,))
    B, T, D = c["x"].shape
    dv = oracle.make_conv_dims(B, T, D, 4, 6, act)
    ver = oracle.conv_update(dv, c["x"], c["w"], c["bias"], c["pool"], c["idx"])
    assert np.array_equal(ver["pool"], c["pool"])       # verify leaves the state alone
    d1 = oracle.make_conv_dims(B, 1, D, 4, 6, act)
    pool = c["pool"].copy()
    for t in range(T):
        step = oracle.conv_update(d1, c["x"][:, t:t + 1], c["w"], c["bias"], pool, c["idx"], write_back=True)
        assert np.array_equal(step["y"][:, 0], ver["y"][:, t])
        pool = step["pool"]
        n = np.full(B, t + 1, np.int32)
        assert np.array_equal(oracle.conv_commit(dv, c["x"], c["pool"], c["idx"], n), pool)
    wb = oracle.conv_update(dv, c["x"], c["w"], c["bias"], c["pool"], c["idx"], write_back=True)
    assert np.array_equal(wb["pool"], pool)
    assert np.array_equal(wb["y"], ver["y"])


def test_fused_commit_equals_commit_then_verify():
    rng = np.random.default_rng(4)
    c = rand_case(rng, B=5, T=3, D=8, K=4, P=7, pad=(4,))
    prev = rng.standard_normal((5, 6, 8))                # previous step had 6 tokens
    plen = np.array([2, 0, 6, 7, 1], np.int32)           # 0 and 7 (> 6) commit nothing
    d = oracle.make_conv_dims(5, 3, 8, 4, 7)
    fused = oracle.conv_update(d, c["x"], c["w"], c["bias"], c["pool"], c["idx"], prev_x=prev, prev_len=plen)
    d6 = oracle.make_conv_dims(5, 6, 8, 4, 7)
    pool1 = oracle.conv_commit(d6, prev, c["pool"], c["idx"], plen)
    plain = oracle.conv_update(d, c["x"], c["w"], c["bias"], pool1, c["idx"])
    assert np.array_equal(fused["pool"], pool1)
    assert np.array_equal(fused["y"], plain["y"])


def test_identity_activation_is_linear():
    rng = np.random.default_rng(5)
    c1, c2 = rand_case(rng, pad=()), rand_case(rng, pad=())
    c2["idx"] = c1["idx"]
    B, T, D = c1["x"].shape
    d = oracle.make_conv_dims(B, T, D, 4, 6, "none")
    y1 = oracle.conv_update(d, c1["x"], c1["w"], None, c1["pool"], c1["idx"])["y"]
    y2 = oracle.conv_update(d, c2["x"], c1["w"], None, c2["pool"], c1["idx"])["y"]
    y3 = oracle.conv_update(d, 2 * c1["x"] - 3 * c2["x"], c1["w"], None, 2 * c1["pool"] - 3 * c2["pool"],
                            c1["idx"])["y"]
    np.testing.assert_allclose(y3, 2 * y1 - 3 * y2, rtol=0, atol=1e-12)


def test_padding_and_out_of_range_slots():
    rng = np.random.default_rng(6)
    c = rand_case(rng, B=4, T=2, D=8, K=3, P=5, pad=())
    c["idx"] = np.array([-1, 5, 2, 1 << 20], np.int32)  # only row 2 is valid
    d = oracle.make_conv_dims(4, 2, 8, 3, 5)
    r = oracle.conv_update(d, c["x"], c["w"], c["bias"], c["pool"], c["idx"], write_back=True,
                           prev_x=c["x"], prev_len=np.full(4, 2, np.int32))
    assert np.all(r["y"][[0, 1, 3]] == 0.0) and np.any(r["y"][2] != 0.0)
    untouched = [0, 1, 3, 4]
    assert np.array_equal(r["pool"][untouched], c["pool"][untouched])


def test_workload_generator_shapes():
    for w in workloads.CONV_WORKLOADS:
        x = workloads.make_conv_inputs(w, seed=0)
        assert x["x"].shape == (w.batch, w.T, w.channels)
        assert x["pool"].shape == (w.pool, w.width - 1, w.channels)
        assert x["w"].shape == (w.width, w.channels)
        assert int((x["idx"] < 0).sum()) == w.n_pad
