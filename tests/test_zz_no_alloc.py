"""gdn_prefill_noalloc through the C ABI: the prefill with its workspace in the library's
fixed per-GPU device array, for callers that cannot allocate. Its results must equal
gdn_prefill's with a caller-owned workspace bit for bit (the same kernels on the same
inputs), on consecutive calls whose sizes shrink, including one whose chunk chain runs in
composed segments; it must replay from a HIP graph like the eager call; and a call that
needs more than the array is refused before anything runs."""
import pytest
import torch

import linear_attention_speculative_gdn_amd as gdn
import workloads
from gpu_harness import say
from workloads import PrefillWorkload, to_device_state

pytestmark = pytest.mark.gpu
DEV = "cuda"
NAMES = ("q", "k", "v", "a", "b", "A_log", "dt_bias", "idx", "fresh", "cu_seqlens")

BIG = PrefillWorkload("noalloc-batch", seqlens=(700, 0, 1500, 33, 300, 16), Hk=4, Hv=8, dk=128, dv=128, pool=9,
                      state_dtype="bf16", io_dtype="bf16", n_fresh=1, n_pad=1, qk="raw", decay="weak")
SEGMENTED = PrefillWorkload("noalloc-segments", seqlens=(1100,), Hk=1, Hv=2, dk=128, dv=64, pool=2,
                            state_dtype="f32", io_dtype="bf16", decay="weak")
SMALL = PrefillWorkload("noalloc-small", seqlens=(17, 90), Hk=2, Hv=4, dk=128, dv=64, pool=3, state_dtype="f32",
                        io_dtype="bf16", n_fresh=1)


def inputs(w, seed):
    x = workloads.make_prefill_inputs(w, seed=seed)
    g = {n: x[n].to(DEV) for n in NAMES}
    g["pool"] = to_device_state(x["pool"]).to(DEV)
    return g


def call(w, g, pool, o, noalloc, ws=None):
    args = (g["q"], g["k"], g["v"], g["a"], g["b"], g["A_log"], g["dt_bias"], o, pool, g["idx"], g["cu_seqlens"],
            g["fresh"])
    if noalloc:
        gdn.gdn_prefill_noalloc(*args, scale=w.scale)
    else:
        gdn.gdn_prefill(*args, scale=w.scale, workspace=ws)


def run(w, g, noalloc):
    pool = g["pool"].clone()
    o = torch.full((w.tokens, w.Hv, w.dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = None
    if not noalloc:
        ws = torch.empty(gdn.gdn_prefill_workspace_bytes(w.batch, w.tokens, w.Hk, w.Hv, w.dk, w.dv,
                                                         workloads.torch_dtype(w.state_dtype)),
                         dtype=torch.uint8, device=DEV)
    call(w, g, pool, o, noalloc, ws)
    torch.cuda.synchronize()
    return o, pool


def test_noalloc_equals_caller_workspace_on_shrinking_calls():
    for w, seed in ((BIG, 1), (SEGMENTED, 2), (SMALL, 3)):
        say(f"[noalloc] {w.name}: {w.tokens} tokens, {w.Hv} v-heads")
        g = inputs(w, seed)
        o_ref, pool_ref = run(w, g, False)
        o, pool = run(w, g, True)
        assert torch.equal(o, o_ref), w.name
        assert torch.equal(pool, pool_ref), w.name


def test_noalloc_graph_replay():
    w = SMALL
    g = inputs(w, 4)
    o_ref, pool_ref = run(w, g, True)            # one call outside the capture resolves the array
    pool = g["pool"].clone()
    o = torch.empty_like(o_ref)
    graph, stream = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=stream):
        call(w, g, pool, o, True)
    for rep in range(3):
        pool.copy_(g["pool"])
        o.fill_(float("nan"))
        run(BIG, inputs(BIG, 10 + rep), True)    # eager work on the same array between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(pool, pool_ref), rep


def test_noalloc_refuses_calls_beyond_the_array():
    w = PrefillWorkload("noalloc-too-large", seqlens=(36000,), Hk=4, Hv=8, dk=128, dv=128, pool=1,
                        state_dtype="bf16", io_dtype="bf16")
    need = gdn.gdn_prefill_workspace_bytes(w.batch, w.tokens, w.Hk, w.Hv, w.dk, w.dv, torch.bfloat16)
    assert need > gdn.GDN_PREFILL_NOALLOC_BYTES
    e = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=DEV)
    q, v, ab = e(w.tokens, w.Hk, w.dk), e(w.tokens, w.Hv, w.dv), e(w.tokens, w.Hv)
    pool = e(1, w.Hv, w.dv, w.dk)
    pool0 = pool.clone()
    with pytest.raises(gdn.GdnError) as err:
        gdn.gdn_prefill_noalloc(q, q, v, ab, ab, torch.zeros(w.Hv, device=DEV), torch.zeros(w.Hv, device=DEV), v,
                                pool, torch.zeros(1, dtype=torch.int32, device=DEV),
                                torch.tensor([0, w.tokens], dtype=torch.int32, device=DEV))
    assert err.value.status == 7
    torch.cuda.synchronize()
    assert torch.equal(pool, pool0)
