"""GPU tests of the exact parts of the contract (bit for bit) and of self-consistency:
identity gates, untouched memory, commit, padding and out-of-range slots, duplicate
rows, verify(T) == T decodes, fused == commit + verify, determinism, batch split,
a width-changing episode, HIP-graph capture and replay, and edge geometries against
the oracle."""
import numpy as np
import pytest
import torch

import linear_attention_speculative_gdn_amd as gdn
import workloads
from gpu_harness import SENTINEL, f64, gpu_step, max_abs, oracle_step, say, to_gpu, tol
from workloads import Workload, from_device_state, to_device_state

pytestmark = pytest.mark.gpu
DEV = "cuda"


def small(state="bf16", io=None, **kw):
    base = dict(batch=6, T=4, Hk=2, Hv=4, dk=128, dv=128, pool=9, state_dtype=state,
                io_dtype=io or state, mode="verify", cache_T=4, n_pad=1)
    base.update(kw)
    return Workload("small-" + state, **base)


def verify(g, w, cache=None, write_final=False, prev=None, o=None, idx=None, pool=None, sl=slice(None)):
    o = g["o"] if o is None else o
    gdn.gdn_verify(g["q"][sl], g["k"][sl], g["v"][sl], g["a"][sl], g["b"][sl], g["A_log"], g["dt_bias"], o,
                   g["pool"] if pool is None else pool, (g["idx"] if idx is None else idx)[sl], cache, write_final,
                   prev, scale=w.scale)


@pytest.mark.parametrize("state", ["bf16", "f32"])
def test_identity_gates_keep_state_bit_exact(state):
    w = small(state)
    x = workloads.make_inputs(w, seed=3)
    x["a"] = torch.full_like(x["a"], float("-inf"))
    x["b"] = torch.full_like(x["b"], float("-inf"))
    g = to_gpu(w, x)
    pool0 = g["pool"].clone()
    say(f"[bookkeeping] identity gates {state}")
    verify(g, w, g["cache"], write_final=True)
    torch.cuda.synchronize()
    idx = x["idx"].numpy()
    for r in np.nonzero(idx >= 0)[0]:
        for t in range(w.T):
            assert torch.equal(g["cache"][r, t], pool0[idx[r]]), (r, t)
    assert torch.equal(g["pool"], pool0)


@pytest.mark.parametrize("state", ["bf16", "f32"])
def test_untouched_memory_and_padding(state):
    w = small(state, cache_T=6)
    x = workloads.make_inputs(w, seed=4)
    g = to_gpu(w, x)
    pool0 = g["pool"].clone()
    verify(g, w, g["cache"], write_final=False)
    torch.cuda.synchronize()
    idx = x["idx"].numpy()
    pad = idx < 0
    assert torch.equal(g["pool"], pool0), "read-only verify wrote the pool"
    assert bool(torch.all(g["o"][torch.from_numpy(pad)] == 0))
    assert bool(torch.all(g["cache"][torch.from_numpy(pad)] == SENTINEL))
    assert bool(torch.all(g["cache"][:, w.T:] == SENTINEL))
    assert not bool(torch.any(torch.isnan(g["o"])))


@pytest.mark.parametrize("state", ["bf16", "f32"])
def test_commit_bit_exact_and_skips(state):
    w = small(state, batch=8, pool=12, n_pad=0)
    x = workloads.make_inputs(w, seed=5)
    g = to_gpu(w, x)
    verify(g, w, g["cache"])
    torch.cuda.synchronize()
    idx = torch.tensor([3, 7, 0, 11, 5, 12, -3, 9], dtype=torch.int32)   # 12 = P and -3: padding
    acc = torch.tensor([1, 4, 0, 2, 5, 2, 3, 3], dtype=torch.int32)       # 0 and 5 (> cache_T): skipped
    pool0 = g["pool"].clone()
    gdn.gdn_commit(g["cache"], idx.to(DEV), acc.to(DEV), g["pool"])
    torch.cuda.synchronize()
    expect = pool0.clone()
    for r in range(w.batch):
        s, n = int(idx[r]), int(acc[r])
        if 0 <= s < w.pool and 1 <= n <= w.cache_T:
            expect[s] = g["cache"][r, n - 1]
    assert torch.equal(g["pool"], expect)


def test_out_of_range_slots_are_padding():
    w = small("f32", batch=5, pool=7, n_pad=0)
    x = workloads.make_inputs(w, seed=6)
    x["idx"] = torch.tensor([2, 7, -1, -100, 4], dtype=torch.int32)
    g = to_gpu(w, x)
    pool0 = g["pool"].clone()
    verify(g, w, g["cache"], write_final=True)
    torch.cuda.synchronize()
    for r in (1, 2, 3):
        assert bool(torch.all(g["o"][r] == 0)) and bool(torch.all(g["cache"][r] == SENTINEL))
    for s in (0, 1, 3, 5, 6):
        assert torch.equal(g["pool"][s], pool0[s])
    ref = oracle_step(w.replace(write_final=True), x)
    assert max_abs(f64(g["o"]), ref["o"]) <= tol(w)


def test_duplicate_rows_in_read_only_verify():
    w = small("bf16", batch=4, n_pad=0)
    x = workloads.make_inputs(w, seed=7)
    x["idx"] = torch.tensor([5, 2, 5, 5], dtype=torch.int32)
    g = to_gpu(w, x)
    verify(g, w, g["cache"])
    torch.cuda.synchronize()
    for r in range(w.batch):
        o1 = torch.empty_like(g["o"][r:r + 1])
        c1 = torch.full_like(g["cache"][r:r + 1], SENTINEL)
        verify(g, w, c1, o=o1, sl=slice(r, r + 1))
        torch.cuda.synchronize()
        assert torch.equal(o1, g["o"][r:r + 1]) and torch.equal(c1, g["cache"][r:r + 1])


@pytest.mark.parametrize("state", ["bf16", "f32"])
def test_verify_equals_successive_decodes(state):
    w = small(state, n_pad=1)
    x = workloads.make_inputs(w, seed=8)
    g = to_gpu(w, x)
    pool_dec = g["pool"].clone()
    verify(g, w, g["cache"], write_final=True)
    idx = x["idx"].numpy()
    valid = torch.from_numpy(idx >= 0)
    for t in range(w.T):
        o1 = torch.empty_like(g["o"][:, t:t + 1])
        s = slice(t, t + 1)
        gdn.gdn_decode(g["q"][:, s].contiguous(), g["k"][:, s].contiguous(), g["v"][:, s].contiguous(),
                       g["a"][:, s].contiguous(), g["b"][:, s].contiguous(), g["A_log"], g["dt_bias"], o1,
                       pool_dec, g["idx"], scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o1[:, 0], g["o"][:, t]), f"o differs at token {t}"
        sl = torch.from_numpy(idx[idx >= 0]).long()
        assert torch.equal(pool_dec[sl], g["cache"][valid, t]), f"state differs at token {t}"
    assert torch.equal(pool_dec, g["pool"])


def test_fused_commit_equals_commit_then_verify():
    w = workloads.Workload("fused-small", batch=7, T=3, Hk=2, Hv=4, dk=128, dv=128, pool=11, state_dtype="bf16",
                           io_dtype="bf16", mode="verify_fused", cache_T=5, n_pad=1)
    x = workloads.make_inputs(w, seed=9)
    x["prev_accept"][0] = 0   # one row with nothing to commit starts from its slot
    ga = to_gpu(w, x)
    gb = to_gpu(w, x)
    verify(ga, w, ga["cache"], prev=ga["prev_accept"])
    gdn.gdn_commit(gb["cache"], gb["idx"], gb["prev_accept"], gb["pool"])
    verify(gb, w, gb["cache"])
    torch.cuda.synchronize()
    for key in ("o", "pool", "cache"):
        assert torch.equal(ga[key], gb[key]), key
    ref = oracle_step(w, x)
    assert max_abs(f64(ga["o"]), ref["o"]) <= tol(w)


def test_repeat_runs_bit_identical():
    w = small("bf16")
    x = workloads.make_inputs(w, seed=10)
    g1, g2 = to_gpu(w, x), to_gpu(w, x)
    verify(g1, w, g1["cache"], write_final=True)
    verify(g2, w, g2["cache"], write_final=True)
    torch.cuda.synchronize()
    for key in ("o", "pool", "cache"):
        assert torch.equal(g1[key], g2[key])


def test_batch_split_equals_one_call():
    w = small("bf16", batch=10, pool=16, n_pad=2)
    x = workloads.make_inputs(w, seed=11)
    g1, g2 = to_gpu(w, x), to_gpu(w, x)
    verify(g1, w, g1["cache"], write_final=True)
    for sl in (slice(0, 3), slice(3, 10)):
        o = torch.empty_like(g2["o"][sl])
        c = g2["cache"][sl]
        gdn.gdn_verify(g2["q"][sl], g2["k"][sl], g2["v"][sl], g2["a"][sl], g2["b"][sl], g2["A_log"], g2["dt_bias"],
                       o, g2["pool"], g2["idx"][sl].contiguous(), c, True, None, scale=w.scale)
        g2["o"][sl] = o
    torch.cuda.synchronize()
    for key in ("o", "pool", "cache"):
        assert torch.equal(g1[key], g2[key]), key


def test_width_episode_matches_sequential_decode():
    """Verify widths 8, 1, 3, 2, 8 with a commit after each equal decoding only the
    accepted tokens one by one (one shared cache of depth 8)."""
    widths, accepts = (8, 1, 3, 2, 8), (5, 1, 3, 1, 8)
    base = Workload("episode", batch=5, T=8, Hk=2, Hv=4, dk=128, dv=128, pool=7, state_dtype="bf16",
                    io_dtype="bf16", mode="verify", cache_T=8, n_pad=1)
    x0 = workloads.make_inputs(base, seed=12)
    pool_v = to_device_state(x0["pool"]).to(DEV)
    pool_d = pool_v.clone()
    idx = x0["idx"].to(DEV)
    cache = torch.zeros((base.batch, 8, base.Hv, base.dv, base.dk), dtype=torch.bfloat16, device=DEV)
    for step, (W, n) in enumerate(zip(widths, accepts)):
        wk = base.replace(T=W)
        x = workloads.make_inputs(wk, seed=100 + step)
        g = {k_: x[k_].to(DEV) for k_ in ("q", "k", "v", "a", "b", "A_log", "dt_bias")}
        o = torch.empty((base.batch, W, base.Hv, base.dv), dtype=torch.bfloat16, device=DEV)
        gdn.gdn_verify(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], o, pool_v, idx, cache,
                       False, None, scale=wk.scale)
        acc = torch.full((base.batch,), n, dtype=torch.int32, device=DEV)
        gdn.gdn_commit(cache, idx, acc, pool_v)
        for t in range(n):
            s = slice(t, t + 1)
            o1 = torch.empty((base.batch, 1, base.Hv, base.dv), dtype=torch.bfloat16, device=DEV)
            gdn.gdn_decode(g["q"][:, s].contiguous(), g["k"][:, s].contiguous(), g["v"][:, s].contiguous(),
                           g["a"][:, s].contiguous(), g["b"][:, s].contiguous(), g["A_log"], g["dt_bias"], o1,
                           pool_d, idx, scale=wk.scale)
        torch.cuda.synchronize()
        assert torch.equal(pool_v, pool_d), f"episode step {step} (width {W}, accept {n})"


def test_graph_capture_and_replay():
    """verify + commit captured once in a HIP graph, replayed with new inputs, slots
    and accept lengths written into the captured buffers; every replay equals eager."""
    w = small("bf16", batch=8, pool=12, n_pad=1, commit=True)
    x = workloads.make_inputs(w, seed=13)
    st = to_gpu(w, x)                       # static buffers
    st["accept"] = x["accept"].to(DEV)
    stream = torch.cuda.Stream()
    verify(st, w, st["cache"])               # load the code objects before capture
    gdn.gdn_commit(st["cache"], st["idx"], st["accept"], st["pool"])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        verify(st, w, st["cache"])
        gdn.gdn_commit(st["cache"], st["idx"], st["accept"], st["pool"])
    for rep in range(4):
        xr = workloads.make_inputs(w, seed=200 + rep)
        xr["accept"] = torch.from_numpy(np.random.default_rng(rep).integers(0, 6, w.batch).astype(np.int32))
        ref = to_gpu(w, xr)
        ref["accept"] = xr["accept"].to(DEV)
        for key in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx", "pool", "accept"):
            st[key].copy_(ref[key])
        st["cache"].fill_(SENTINEL)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        verify(ref, w, ref["cache"])
        gdn.gdn_commit(ref["cache"], ref["idx"], ref["accept"], ref["pool"])
        torch.cuda.synchronize()
        for key in ("o", "cache", "pool"):
            assert torch.equal(st[key], ref[key]), (rep, key)


EDGE = [
    dict(dk=16, dv=16, Hk=1, Hv=1, T=1),
    dict(dk=32, dv=48, Hk=2, Hv=2, T=3),
    dict(dk=64, dv=128, Hk=1, Hv=3, T=5),
    dict(dk=128, dv=64, Hk=2, Hv=4, T=2),
    dict(dk=128, dv=80, Hk=1, Hv=2, T=4),
    dict(dk=256, dv=256, Hk=1, Hv=2, T=2),
    dict(dk=128, dv=128, Hk=2, Hv=2, T=16),
    dict(dk=128, dv=80, Hk=1, Hv=2, T=1),     # single token: a whole head per workgroup, rows past d_v masked
    dict(dk=128, dv=256, Hk=2, Hv=4, T=1),    # single token: two workgroups per head
]


@pytest.mark.parametrize("variant", ["as-drawn", "rawqk-weakdecay"])
@pytest.mark.parametrize("geo", EDGE, ids=[f"dk{e['dk']}-dv{e['dv']}-T{e['T']}" for e in EDGE])
@pytest.mark.parametrize("state,io", [("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16"), ("bf16", "f32")])
def test_edge_geometries_against_oracle(geo, state, io, variant):
    """Every supported d_k, ragged d_v, 1-16 tokens and all four dtype pairs against the
    oracle; the second variant stores q and k unnormalised (norms 0.05-20, a zero vector,
    a vector of norm 1e-3) and draws weak decays, so the in-kernel L2 normalisation (its
    eps and its sums over the lanes of every d_k) and the carried state are what is
    checked."""
    w = Workload("edge", batch=5, pool=8, state_dtype=state, io_dtype=io, mode="verify", cache_T=geo["T"] + 1,
                 write_final=True, n_pad=1, **geo)
    if variant != "as-drawn":
        w = w.replace(qk="raw", decay="weak")
    x = workloads.make_inputs(w, seed=14)
    g = to_gpu(w, x)
    say(f"[edge] {geo} state={state} io={io} {variant}")
    gpu_step(w, g)
    torch.cuda.synchronize()
    ref = oracle_step(w, x)
    idx = x["idx"].numpy()
    valid = idx >= 0
    t_o = tol(w) if io == "f32" else max(tol(w), 2e-2)
    assert max_abs(f64(g["o"]), ref["o"]) <= t_o
    gc = from_device_state(g["cache"].cpu()).double().numpy()
    assert max_abs(gc[valid, :w.T], ref["cache"][valid, :w.T]) <= tol(w)
    gp = from_device_state(g["pool"].cpu()).double().numpy()
    assert max_abs(gp, ref["pool"]) <= tol(w)


def test_empty_batch_is_a_no_op():
    w = small("bf16", batch=0, n_pad=0)
    e = lambda *s, dt=torch.bfloat16: torch.empty(s, dtype=dt, device=DEV)
    pool = torch.randn(3, 4, 128, 128, device=DEV).to(torch.bfloat16)
    p0 = pool.clone()
    gdn.gdn_verify(e(0, 4, 2, 128), e(0, 4, 2, 128), e(0, 4, 4, 128), e(0, 4, 4), e(0, 4, 4),
                   torch.zeros(4, device=DEV), torch.zeros(4, device=DEV), e(0, 4, 4, 128), pool,
                   torch.empty(0, dtype=torch.int32, device=DEV), None, True, None)
    torch.cuda.synchronize()
    assert torch.equal(pool, p0)
    assert w.batch == 0
