"""GPU tests of the chunked prefill (gdn_prefill) through the C ABI, against the float64
oracle that runs the recurrence token by token.

The kernel evaluates the chunked form on bf16 matrix cores: every product takes bf16
operands (the stored keys, queries and values exactly; the state, the triangular inverse,
W, U and the output mask rounded to nearest even, at most 2^-9 relative each) and
accumulates in fp32. Errors are therefore measured relative to the scale of the result:
per (sequence, v-head), max |o_gpu - o_ref| <= TOL_O * max |o_ref| and, for the stored
state, max |S_gpu - S_ref| <= TOL_S * max |S_ref| (plus bf16 rounding of a bf16 pool).
The bound: one chunk chains three rounded products into U (Tm, W S_0, then U itself in
P U and in the state update), about 3 * 2^-8 relative to the magnitudes involved; the
decays and the delta rule keep the state bounded, so the error does not grow with the
number of chunks beyond that of one chunk's contributions. TOL_O = TOL_S = 2^-5 leaves a
factor of about 2.5 over 3 * 2^-8 for the sums of a few such terms.
"""
import numpy as np
import pytest
import torch

import linear_attention_speculative_gdn_amd as gdn
import oracle
import workloads
from gpu_harness import say
from workloads import PrefillWorkload, from_device_state, to_device_state

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_O = 2.0 ** -5
TOL_S = 2.0 ** -5


def f64(t):
    return t.detach().to("cpu").double().numpy()


def run_gpu(w, x):
    g = {n: x[n].to(DEV) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx", "fresh", "cu_seqlens")}
    g["pool"] = to_device_state(x["pool"]).to(DEV)
    pool0 = g["pool"].clone()
    o = torch.full((w.tokens, w.Hv, w.dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_prefill(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], o, g["pool"], g["idx"],
                    g["cu_seqlens"], g["fresh"], scale=w.scale)
    torch.cuda.synchronize()
    return o, g["pool"], pool0


def run_oracle(w, x):
    d = oracle.make_dims(w.batch, 1, w.Hk, w.Hv, w.dk, w.dv, w.pool, w.state_dtype == "bf16", scale=w.scale)
    return oracle.prefill(d, x["cu_seqlens"].numpy(), f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["a"]),
                          f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]), f64(x["pool"]), x["idx"].numpy(),
                          x["fresh"].numpy())


def check(w, x, label, seed=0):
    o, pool, pool0 = run_gpu(w, x)
    ref = run_oracle(w, x)
    og, cu, idx = f64(o), x["cu_seqlens"].numpy(), x["idx"].numpy()
    pg = from_device_state(pool.cpu()).double().numpy()
    worst_o = worst_s = 0.0
    for r in range(w.batch):
        sl = slice(cu[r], cu[r + 1])
        if not 0 <= idx[r] < w.pool:
            assert np.all(og[sl] == 0.0), f"{label}: padding row {r} has o != 0"
            continue
        for h in range(w.Hv):
            if cu[r + 1] > cu[r]:
                scale_o = max(np.abs(ref["o"][sl, h]).max(), 1e-30)
                worst_o = max(worst_o, np.abs(og[sl, h] - ref["o"][sl, h]).max() / scale_o)
            Sr = ref["pool"][idx[r], h]
            scale_s = max(np.abs(Sr).max(), 1e-30)
            round_s = 2.0 ** -8 if w.state_dtype == "bf16" else 0.0
            worst_s = max(worst_s, (np.abs(pg[idx[r], h] - Sr).max() - round_s * scale_s) / scale_s)
    say(f"[prefill] {label}: o err {worst_o:.2e}, state err {worst_s:.2e} (relative to the per-head max)")
    assert worst_o <= TOL_O and worst_s <= TOL_S
    touched = np.zeros(w.pool, bool)
    touched[idx[(idx >= 0) & (idx < w.pool)]] = True
    ut = torch.from_numpy(np.nonzero(~touched)[0])
    assert torch.equal(pool.cpu()[ut], pool0.cpu()[ut]), f"{label}: an untouched slot changed"


@pytest.mark.parametrize("wi", [1, 2, 3, 4], ids=[workloads.PREFILL_WORKLOADS[i].name for i in (1, 2, 3, 4)])
def test_prefill_parity(wi):
    w = workloads.PREFILL_WORKLOADS[wi]
    check(w, workloads.make_prefill_inputs(w, seed=0), w.name)


@pytest.mark.parametrize("wi", [1, 2, 3, 4], ids=[workloads.PREFILL_WORKLOADS[i].name for i in (1, 2, 3, 4)])
def test_prefill_parity_unnormalised_qk_weak_decay(wi):
    """The prefill workloads (mixed lengths; 8 x 2048; 4 x 4096 with 32 heads on two-column-
    tile waves; one 16384-token prompt in composed segments) with q and k stored
    unnormalised (norms 0.05-20, a zero vector and one of norm 1e-3 each) and weak decays:
    the norms then enter the chunked form as the diagonal factors that scale the key and
    query products, the masks and the records, and hundreds of tokens stay in the state."""
    w = workloads.PREFILL_WORKLOADS[wi]
    w = w.replace(name=w.name + "-rawqk-weakdecay", qk="raw", decay="weak")
    x = workloads.make_prefill_inputs(w, seed=0)
    n = x["k"].double().norm(dim=-1)
    assert float(n.max()) > 10 and int((n == 0).sum()) == 1
    check(w, x, w.name)


GEOM = [
    PrefillWorkload("edges-dv32-f32", seqlens=(0, 1, 15, 16, 17, 33, 48), Hk=1, Hv=2, dk=128, dv=32, pool=9,
                    state_dtype="f32", io_dtype="bf16", n_fresh=2, n_pad=1),
    PrefillWorkload("dv64-g4-bf16", seqlens=(70, 5, 129), Hk=1, Hv=4, dk=128, dv=64, pool=4,
                    state_dtype="bf16", io_dtype="bf16", n_fresh=1),
    PrefillWorkload("dv256-f32", seqlens=(40, 97), Hk=2, Hv=2, dk=128, dv=256, pool=3,
                    state_dtype="f32", io_dtype="bf16"),
    PrefillWorkload("long-3000-bf16", seqlens=(3000,), Hk=1, Hv=1, dk=128, dv=128, pool=2,
                    state_dtype="bf16", io_dtype="bf16"),
]


@pytest.mark.parametrize("variant", ["as-drawn", "rawqk-weakdecay"])
@pytest.mark.parametrize("w", GEOM, ids=[w.name for w in GEOM])
def test_prefill_geometries(w, variant):
    if variant != "as-drawn":
        w = w.replace(qk="raw", decay="weak")
    check(w, workloads.make_prefill_inputs(w, seed=1), w.name)


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_prefill_slow_decay_long_memory(state):
    """Weak decay (exp(A_log) = 0.02, g ~ 0.99 per token) keeps hundreds of tokens in the
    state, so errors carried across chunks would show; the workloads' own decays forget
    within a few tokens."""
    w = PrefillWorkload(f"slow-{state}", seqlens=(2048, 333), Hk=2, Hv=4, dk=128, dv=128, pool=4,
                        state_dtype=state, io_dtype="bf16", n_fresh=1)
    x = workloads.make_prefill_inputs(w, seed=4)
    x["A_log"] = torch.full((w.Hv,), float(np.log(0.02)), dtype=torch.float32)
    check(w, x, w.name)


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_prefill_segment_boundaries(state):
    """The chunk chain runs in segments of 256 tokens whose maps are composed: lengths at
    and around the segment boundaries (one segment, a one-token second segment, two full
    ones, the first composed map, three maps, an empty sequence), a padding row and a fresh
    row, d_v = 64 (map columns past the value columns), and slow decay so that the composed
    maps carry weight."""
    w = PrefillWorkload(f"segments-{state}", seqlens=(256, 257, 0, 512, 513, 769, 300), Hk=1, Hv=2, dk=128, dv=64,
                        pool=8, state_dtype=state, io_dtype="bf16", n_fresh=1, n_pad=1, qk="raw")
    x = workloads.make_prefill_inputs(w, seed=5)
    x["A_log"] = torch.full((w.Hv,), float(np.log(0.02)), dtype=torch.float32)
    check(w, x, w.name)


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_prefill_segments_in_four_chain_groups(state):
    """A long sequence next to short ones, d_v = 64 and 8 v-heads: the chain runs in segments
    whose groups hold four chains (more than one two-chain workgroup per CU), and in the
    first phase the groups past the value columns carry only map columns (their value-column
    waves take part in the barriers alone). A fresh row, a padding row and slow decay, so
    that the composed maps carry weight."""
    w = PrefillWorkload(f"segments-quads-{state}", seqlens=(8000, 0, 37, 300), Hk=4, Hv=8, dk=128, dv=64, pool=6,
                        state_dtype=state, io_dtype="bf16", n_fresh=1, n_pad=1, qk="raw")
    x = workloads.make_prefill_inputs(w, seed=9)
    x["A_log"] = torch.full((w.Hv,), float(np.log(0.02)), dtype=torch.float32)
    check(w, x, w.name)


@pytest.mark.parametrize("Hk,Hv,seqlens", [(1, 2, (1100, 40, 700, 900)), (4, 8, (3000, 40, 1800, 2600))],
                         ids=["two-chain-groups", "four-chain-groups"])
def test_prefill_long_padding_and_fresh_rows_in_segments(Hk, Hv, seqlens):
    """Padding rows long enough to have middle segments, with d_v = 64: the first phase's
    groups of such a row include ones for the map columns past the value columns, and only
    segment 0's groups (of value columns) write its zeros. The first padding row is followed
    by a valid short row, whose outputs must survive; the last row, also padding, ends the
    output buffer. A fresh row of several segments starts its chain from zero and its later
    segments from the composed states. Two- and four-chain groups, slow decay."""
    for state in ("f32", "bf16"):
        w = PrefillWorkload(f"long-padding-{Hv}-{state}", seqlens=seqlens, Hk=Hk, Hv=Hv, dk=128, dv=64, pool=4,
                            state_dtype=state, io_dtype="bf16", qk="raw")
        x = workloads.make_prefill_inputs(w, seed=11)
        x["idx"][0] = -1
        x["idx"][3] = -1
        x["fresh"][:] = 0
        x["fresh"][2] = 1
        x["A_log"] = torch.full((w.Hv,), float(np.log(0.02)), dtype=torch.float32)
        check(w, x, w.name)


@pytest.mark.parametrize("dv,Hk,Hv", [(32, 1, 1), (256, 1, 1), (256, 1, 3)],
                         ids=["dv32", "dv256-two-chain-groups", "dv256-four-chain-groups"])
def test_prefill_segments_narrow_and_wide_dv(dv, Hk, Hv):
    """Segmented chains with d_v = 32 (one group of value columns, the others map columns
    only) and d_v = 256 (twice d_k: groups past the map columns carry value columns only),
    in two- and four-chain groups, ragged lengths of one to six segments, a padding row and
    a fresh row, fp32 and bf16 pools, slow decay."""
    for state in ("f32", "bf16"):
        w = PrefillWorkload(f"segments-dv{dv}-hv{Hv}-{state}", seqlens=(700, 30, 1300, 260), Hk=Hk, Hv=Hv, dk=128,
                            dv=dv, pool=4, state_dtype=state, io_dtype="bf16", qk="raw")
        x = workloads.make_prefill_inputs(w, seed=12)
        x["idx"][3] = -1
        x["fresh"][:] = 0
        x["fresh"][2] = 1
        x["A_log"] = torch.full((w.Hv,), float(np.log(0.02)), dtype=torch.float32)
        check(w, x, w.name)


def test_prefill_two_v_heads_per_pass1_wave_g4():
    """Pass 1 takes two v-heads of a k-head per wave once one wave per (chunk, v-head) would
    exceed the chip (chunk records x v-heads > 4096): here with four v-heads per k-head, so
    each k-head's pair of waves shares its keys and queries, ragged lengths, a fresh row and
    unnormalised q/k with weak decay."""
    w = PrefillWorkload("g4-vh2", seqlens=(2100, 1999, 17, 2048, 2300), Hk=2, Hv=8, dk=128, dv=128, pool=6,
                        state_dtype="bf16", io_dtype="bf16", n_fresh=1, qk="raw", decay="weak")
    assert (w.tokens // 16 + w.batch) * w.Hv > 4096 and (w.Hv // w.Hk) % 2 == 0
    check(w, workloads.make_prefill_inputs(w, seed=10), w.name)


def test_prefill_wide_column_tiles():
    """Batches with two or more chains per SIMD (2 B Hv d_v/16 >= 2048 waves) and a d_v that
    is not a multiple of 64 run the chain on waves of two 16-column tiles: d_v = 96 (three such blocks per head), ragged
    lengths, a padding row and a fresh row, bf16 and fp32 pools."""
    for state in ("bf16", "f32"):
        w = PrefillWorkload(f"wide-dv96-{state}", seqlens=(37, 130, 0, 16, 211, 64, 5, 96), Hk=4, Hv=32, dk=128,
                            dv=96, pool=10, state_dtype=state, io_dtype="bf16", n_fresh=1, n_pad=1)
        assert 2 * w.batch * w.Hv * (w.dv // 16) >= 2048
        check(w, workloads.make_prefill_inputs(w, seed=7), w.name)
        wr = w.replace(name=w.name + "-rawqk-weakdecay", qk="raw", decay="weak")
        check(wr, workloads.make_prefill_inputs(wr, seed=7), wr.name)


@pytest.mark.parametrize("dv,Hv", [(64, 32), (128, 16)])
def test_prefill_four_chain_groups(dv, Hv):
    """Batches with two or more chains per SIMD and d_v a multiple of 64 run four chains per
    workgroup on records staged once in LDS: ragged lengths (an empty sequence, chunk-sized,
    one-token and long ones), a padding row and a fresh row, bf16 and fp32 pools, and the
    unnormalised-q/k, weak-decay variant."""
    for state in ("bf16", "f32"):
        w = PrefillWorkload(f"quad-dv{dv}-{state}", seqlens=(37, 130, 0, 16, 211, 64, 1, 96), Hk=4, Hv=Hv, dk=128,
                            dv=dv, pool=10, state_dtype=state, io_dtype="bf16", n_fresh=1, n_pad=1)
        assert 2 * w.batch * w.Hv * (w.dv // 16) >= 2048 and w.dv % 64 == 0
        check(w, workloads.make_prefill_inputs(w, seed=8), w.name)
        wr = w.replace(name=w.name + "-rawqk-weakdecay", qk="raw", decay="weak")
        check(wr, workloads.make_prefill_inputs(wr, seed=8), wr.name)


def test_prefill_split_continues_from_the_pool():
    """Two calls (a chunked prefill across scheduler steps, cut off a chunk boundary)
    follow the single call to the same tolerance."""
    w = PrefillWorkload("whole", seqlens=(200,), Hk=1, Hv=2, dk=128, dv=128, pool=2, state_dtype="f32",
                        io_dtype="bf16")
    x = workloads.make_prefill_inputs(w, seed=2)
    o_whole, pool_whole, _ = run_gpu(w, x)
    g = {n: x[n].to(DEV) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx")}
    pool = to_device_state(x["pool"]).to(DEV)
    outs = []
    for a_, b_ in ((0, 77), (77, 200)):
        o = torch.empty((b_ - a_, w.Hv, w.dv), dtype=torch.bfloat16, device=DEV)
        gdn.gdn_prefill(g["q"][a_:b_], g["k"][a_:b_], g["v"][a_:b_], g["a"][a_:b_], g["b"][a_:b_], g["A_log"],
                        g["dt_bias"], o, pool, g["idx"], torch.tensor([0, b_ - a_], dtype=torch.int32, device=DEV))
        outs.append(o)
    torch.cuda.synchronize()
    o_split = torch.cat(outs).double()
    err = float((o_split - o_whole.double()).abs().max() / o_whole.double().abs().max())
    serr = float((pool - pool_whole).abs().max() / pool_whole.abs().max())
    say(f"[prefill] split vs whole: o {err:.2e}, state {serr:.2e}")
    assert err <= TOL_O and serr <= TOL_S


def test_prefill_unsupported_and_empty():
    w = PrefillWorkload("e", seqlens=(4,), Hk=1, Hv=1, dk=128, dv=32, pool=1, state_dtype="f32", io_dtype="f32")
    x = workloads.make_prefill_inputs(w)
    g = {n: x[n].to(DEV) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx", "cu_seqlens")}
    pool = to_device_state(x["pool"]).to(DEV)
    o = torch.empty((4, 1, 32), dtype=torch.float32, device=DEV)
    with pytest.raises(gdn.GdnError) as e:      # fp32 tokens: the matrix-core path takes bf16
        gdn.gdn_prefill(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], o, pool, g["idx"],
                        g["cu_seqlens"])
    assert e.value.status == 5
    q0 = torch.empty((0, 1, 128), dtype=torch.bfloat16, device=DEV)
    v0 = torch.empty((0, 1, 32), dtype=torch.bfloat16, device=DEV)
    ab0 = torch.empty((0, 1), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_prefill(q0, q0, v0, ab0, ab0, g["A_log"], g["dt_bias"], v0, pool, torch.empty(0, dtype=torch.int32,
                    device=DEV), torch.zeros(1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()


def test_prefill_caller_workspace_reused_and_graph_replay():
    """A caller-owned workspace serves consecutive calls of different sizes; the two
    launches of one call replay from a HIP graph like the eager call; a workspace one
    byte short is refused before anything runs."""
    w = PrefillWorkload("ws", seqlens=(50, 0, 130, 7), Hk=2, Hv=4, dk=128, dv=64, pool=6, state_dtype="bf16",
                        io_dtype="bf16", n_fresh=1, n_pad=1)
    x = workloads.make_prefill_inputs(w, seed=7)
    need = gdn.gdn_prefill_workspace_bytes(w.batch, w.tokens, w.Hk, w.Hv, w.dk, w.dv, torch.bfloat16)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    g = {n: x[n].to(DEV) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx", "fresh", "cu_seqlens")}

    def call(pool, o, workspace):
        gdn.gdn_prefill(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], o, pool, g["idx"],
                        g["cu_seqlens"], g["fresh"], scale=w.scale, workspace=workspace)

    pool_ref = to_device_state(x["pool"]).to(DEV)
    o_ref = torch.empty((w.tokens, w.Hv, w.dv), dtype=torch.bfloat16, device=DEV)
    call(pool_ref, o_ref, None)                       # per-call workspace
    small = PrefillWorkload("ws-small", seqlens=(20,), Hk=2, Hv=4, dk=128, dv=64, pool=6, state_dtype="bf16",
                            io_dtype="bf16")
    xs = workloads.make_prefill_inputs(small, seed=8)
    gs = {n: xs[n].to(DEV) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx", "cu_seqlens")}
    os_ = torch.empty((small.tokens, small.Hv, small.dv), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_prefill(gs["q"], gs["k"], gs["v"], gs["a"], gs["b"], gs["A_log"], gs["dt_bias"], os_,
                    to_device_state(xs["pool"]).to(DEV), gs["idx"], gs["cu_seqlens"], workspace=ws)
    pool = to_device_state(x["pool"]).to(DEV)
    o = torch.empty_like(o_ref)
    call(pool, o, ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(pool, pool_ref)
    with pytest.raises(gdn.GdnError) as e:
        call(pool, o, ws[: need - 1])
    assert e.value.status == 2

    pool_g = to_device_state(x["pool"]).to(DEV)
    o_g = torch.empty_like(o_ref)
    graph, stream = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=stream):
        call(pool_g, o_g, ws)
    for rep in range(3):
        pool_g.copy_(to_device_state(x["pool"]).to(DEV))
        o_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref) and torch.equal(pool_g, pool_ref), rep


def test_prefill_segmented_graph_replay():
    """A call whose chains run in segments (four launches: segment 0 and the maps, their
    composition, the later segments; the records hold the factor of -W) replays from a HIP
    graph bit for bit like the eager call, three times, with eager work in between."""
    w = PrefillWorkload("seg-graph", seqlens=(1100, 40, 700), Hk=1, Hv=2, dk=128, dv=64, pool=4, state_dtype="f32",
                        io_dtype="bf16", n_fresh=1, qk="raw")
    x = workloads.make_prefill_inputs(w, seed=13)
    g = {n: x[n].to(DEV) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx", "fresh", "cu_seqlens")}
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(w.batch, w.tokens, w.Hk, w.Hv, w.dk, w.dv, torch.float32),
                     dtype=torch.uint8, device=DEV)

    def call(pool, o):
        gdn.gdn_prefill(g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], o, pool, g["idx"],
                        g["cu_seqlens"], g["fresh"], scale=w.scale, workspace=ws)

    pool_ref = to_device_state(x["pool"]).to(DEV)
    o_ref = torch.empty((w.tokens, w.Hv, w.dv), dtype=torch.bfloat16, device=DEV)
    call(pool_ref, o_ref)
    torch.cuda.synchronize()
    pool_g = to_device_state(x["pool"]).to(DEV)
    o_g = torch.empty_like(o_ref)
    graph, stream = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=stream):
        call(pool_g, o_g)
    for rep in range(3):
        pool_g.copy_(to_device_state(x["pool"]).to(DEV))
        o_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref) and torch.equal(pool_g, pool_ref), rep


def test_fp32_grade_prefill_through_verify():
    """The route to an fp32-grade prefill of an fp32 pool: the tokens through gdn_verify with
    write-back, GDN_MAX_T at a time, match the float64 prefill to the recurrent path's fp32
    tolerance (1e-4 absolute on o and the state), where gdn_prefill itself is held to bf16
    grade. Unnormalised q and k, weak decay, sequence lengths across several calls."""
    w = PrefillWorkload("fp32-grade", seqlens=(40, 17, 100), Hk=2, Hv=4, dk=128, dv=128, pool=5,
                        state_dtype="f32", io_dtype="f32", qk="raw", decay="weak")
    x = workloads.make_prefill_inputs(w, seed=11)
    ref = run_oracle(w, x)
    g = {n: x[n].to(DEV) for n in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx")}
    pool = to_device_state(x["pool"]).to(DEV)
    o = torch.full((w.tokens, w.Hv, w.dv), float("nan"), dtype=torch.float32, device=DEV)
    cu = x["cu_seqlens"].numpy()
    for r in range(w.batch):
        for t0 in range(int(cu[r]), int(cu[r + 1]), gdn.GDN_MAX_T):
            t1 = min(t0 + gdn.GDN_MAX_T, int(cu[r + 1]))
            sl = slice(t0, t1)
            ot = torch.empty((1, t1 - t0, w.Hv, w.dv), dtype=torch.float32, device=DEV)
            gdn.gdn_verify(g["q"][sl][None].contiguous(), g["k"][sl][None].contiguous(), g["v"][sl][None].contiguous(),
                           g["a"][sl][None].contiguous(), g["b"][sl][None].contiguous(), g["A_log"], g["dt_bias"], ot,
                           pool, g["idx"][r:r + 1].contiguous(), None, True, None, scale=w.scale)
            o[sl] = ot[0]
    torch.cuda.synchronize()
    o_err = float(np.abs(f64(o) - ref["o"]).max())
    idx = x["idx"].numpy()
    s_err = float(np.abs(from_device_state(pool.cpu()).double().numpy()[idx] - ref["pool"][idx]).max())
    say(f"[prefill] fp32 through verify: o err {o_err:.2e}, state err {s_err:.2e} (absolute)")
    assert o_err <= 1e-4 and s_err <= 1e-4
