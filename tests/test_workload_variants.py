"""The seeded input variants that the GPU parity tests use beside the workloads as
defined: unnormalised q and k, and weak decay. Checked here without a GPU: the draws
have the stated ranges and special vectors, and the default workloads are unchanged."""
import numpy as np
import torch

import workloads


def test_default_draws_unchanged_by_variants():
    w = workloads.WORKLOADS[4]
    a = workloads.make_inputs(w.replace(batch=8, n_pad=1), seed=0)
    b = workloads.make_inputs(w.replace(batch=8, n_pad=1, qk="raw", decay="weak"), seed=0)
    for n in ("idx", "v", "a", "b", "dt_bias", "pool", "prev_accept", "cache_prev"):
        assert torch.equal(a[n], b[n]), n
    # the directions are the same draws; only the norms change
    qa, qb = a["q"].double(), b["q"].double()
    nb = qb.norm(dim=-1, keepdim=True)
    keep = nb[..., 0] > 0
    cos = (qa * qb).sum(-1)[keep] / nb[..., 0][keep]
    assert float(cos.min()) > 0.999


def test_raw_qk_norms_and_special_vectors():
    for st in ("f32", "bf16"):
        w = workloads.WORKLOADS[2].replace(qk="raw", state_dtype=st, io_dtype=st)
        x = workloads.make_inputs(w, seed=3)
        for name in ("q", "k"):
            n = x[name].double().norm(dim=-1).flatten()
            assert int((n == 0).sum()) == 1
            tiny = n[(n > 0) & (n < 0.01)]
            assert tiny.numel() == 1 and abs(float(tiny[0]) - 1e-3) < 1e-5
            rest = n[n >= 0.01]
            assert float(rest.min()) >= 0.05 * 0.99 and float(rest.max()) <= 20.0 * 1.01
            # spread over the whole range (log-uniform)
            assert float(rest.min()) < 0.1 and float(rest.max()) > 10.0


def test_weak_decay_range():
    w = workloads.WORKLOADS[1].replace(decay="weak")
    x = workloads.make_inputs(w, seed=0)
    A = x["A_log"].double().exp()
    assert float(A.min()) >= 0.02 and float(A.max()) < 0.05
    sp = torch.nn.functional.softplus(x["a"].double() + x["dt_bias"].double())
    g = torch.exp(-A * sp)
    assert float(g.median()) > 0.95 and float(g.min()) > 0.8
    strong = workloads.make_inputs(workloads.WORKLOADS[1], seed=0)
    gs = torch.exp(-strong["A_log"].double().exp() * torch.nn.functional.softplus(
        strong["a"].double() + strong["dt_bias"].double()))
    assert float(gs.median()) < 0.05


def test_prefill_variants():
    w = workloads.PREFILL_WORKLOADS[1].replace(qk="raw", decay="weak")
    a = workloads.make_prefill_inputs(workloads.PREFILL_WORKLOADS[1], seed=0)
    b = workloads.make_prefill_inputs(w, seed=0)
    for n in ("idx", "fresh", "cu_seqlens", "v", "a", "b", "dt_bias", "pool"):
        assert torch.equal(a[n], b[n]), n
    n = b["q"].double().norm(dim=-1)
    assert int((n == 0).sum()) == 1 and float(n.max()) > 10
    assert float(b["A_log"].double().exp().max()) < 0.05
