"""Seeded synthetic workloads for the Gated DeltaNet (GDN) decode / speculative-verify path.

This module only draws inputs. It holds none of the method's arithmetic: no gates,
no recurrence, no rounding rule of the state. It serves the float64 oracle and the
HIP path alike, which is the only thing the two share.

Shapes and value distributions follow the serving workloads on the pages:
- "[NVIDIA] [GDN] Enable FlashInfer MTP verify on SM100+ (Blackwell)", Throughput
  Benchmark: 4 verify tokens per MTP step (3 drafts + 1), bf16 SSM state, batches of
  tens to hundreds of running requests;
- the TensorRT-LLM GB300 Qwen3.8-Flash-Next NVFP4 PR (20937), Results / What changes:
  bf16 recurrent pools, MTP3 and MTP7 widths, concurrency 1..256;
- the pool addressing (per-request slot index, -1 for padding) of the first page's
  Summary and Requirements sections.

Recipe (the same for every workload; one ``numpy.random.default_rng(seed)`` each,
draws in this fixed order):
1. slot indices: the first ``batch`` entries of a permutation of the pool, then
   ``n_pad`` distinct rows set to -1 (padding);
2. q, k ~ N(0,1), each (row, token, k-head) vector L2-normalised in float64 (the
   workload is defined on unit-norm inputs); v, a, b ~ N(0,1);
3. A_log = log U[1,16) and dt_bias ~ N(0, 0.1) per v-head (kept fp32);
4. the state pool ~ N(0, 0.1), drawn in float32;
5. accept lengths ~ U{1..T} (commit) and, for the fused-commit workload, the
   previous step's accept lengths ~ U{1..cache_T} plus the previous step's cached
   state at [row, n-1] ~ N(0, 0.1).
Values are stored in the workload's io / state dtype (bf16 by round-to-nearest-even
through torch). The stored values are the inputs; nobody re-derives them.

Two variants exercise what the unit-norm, fast-decay recipe leaves unseen (both drawn
from a second generator, ``numpy.random.default_rng([seed, 1])``, after the draws
above, so the default workloads are unchanged):
- ``qk="raw"``: q and k are NOT normalised before storing. Each (row, token, k-head)
  vector keeps its N(0,1) direction and is rescaled to a norm drawn log-uniformly in
  [0.05, 20]; then one q and one k vector are set to zero and one q and one k vector
  to norm 1e-3 (where eps = 1e-6 in |x|^2 + eps changes the normalised length by
  about 30 %), at random positions. The kernels' own L2 normalisation is then what
  makes the result right.
- ``decay="weak"``: A_log = log U[0.02, 0.05) per v-head, so g = exp(-e^A_log
  softplus(a + dt_bias)) lies around 0.9-0.999 (median about 0.97) instead of a median
  of a few 1e-3: the state carried across tokens dominates each step, and errors in the
  carry, the intermediate cache or the commit show at full weight.

Logical layouts (row-major): q, k [B,T,Hk,dk]; v [B,T,Hv,dv]; a, b [B,T,Hv];
A_log, dt_bias [Hv]; pool [P,Hv,dk,dv] holding S[i][j] (i: key index, j: value
index); cache [B,cache_T,Hv,dk,dv]. The device keeps states transposed
([..., dv, dk]); ``to_device_state`` / ``from_device_state`` convert.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    T: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    pool: int
    state_dtype: str          # "f32" | "bf16"
    io_dtype: str             # "f32" | "bf16"
    mode: str                 # "decode" | "verify" | "verify_fused"
    cache_T: int = 0          # intermediate-state cache depth (0: none)
    write_final: bool = False
    commit: bool = False      # a separate commit follows the verify
    n_pad: int = 0
    fixed_indices: tuple | None = None
    description: str = ""
    qk: str = "unit"          # "unit": q, k normalised before storing | "raw": see the module docstring
    decay: str = "strong"     # "strong": A_log = log U[1,16) | "weak": A_log = log U[0.02, 0.05)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the GDN hot path. Index 2 is the headline (MTP verify, T=4,
# bf16 state); index 0 is small enough for brute force.
WORKLOADS: list[Workload] = [
    Workload("tiny-verify-t2-f32", batch=2, T=2, Hk=1, Hv=2, dk=16, dv=16, pool=4,
             state_dtype="f32", io_dtype="f32", mode="verify", cache_T=2,
             write_final=True, commit=True, fixed_indices=(2, 0),
             description="tiny verify: B=2, Hk=1, Hv=2, d=16, T=2, fp32 state, pool of 4, slots [2,0]"),
    Workload("decode-t1-f32", batch=64, T=1, Hk=4, Hv=8, dk=128, dv=128, pool=256,
             state_dtype="f32", io_dtype="f32", mode="decode", n_pad=8,
             description="single-token decode: B=64 (8 padding rows), Hk=4, Hv=8, d=128, fp32 state, pool of 256"),
    Workload("mtp-verify-t4-bf16", batch=64, T=4, Hk=4, Hv=8, dk=128, dv=128, pool=256,
             state_dtype="bf16", io_dtype="bf16", mode="verify", cache_T=4, commit=True,
             description="MTP verify T=4: B=64, Hk=4, Hv=8, d=128, bf16 state, pool of 256, 4 intermediates + commit"),
    Workload("verify-t4-b256-f32", batch=256, T=4, Hk=16, Hv=32, dk=128, dv=128, pool=512,
             state_dtype="f32", io_dtype="f32", mode="verify", cache_T=4, commit=True,
             description="high-concurrency verify T=4: B=256, Hk=16, Hv=32, d=128, fp32 state, pool of 512, 4 intermediates + commit"),
    Workload("verify-t8-bf16-fused", batch=128, T=8, Hk=16, Hv=32, dk=128, dv=128, pool=1024,
             state_dtype="bf16", io_dtype="bf16", mode="verify_fused", cache_T=8, n_pad=13,
             description="long-draft verify T=8: B=128 (13 padding rows), Hk=16, Hv=32, d=128, bf16 state, pool of 1024, 8 intermediates, fused commit"),
]

HEADLINE = 2


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _store(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float64/float32 draw -> stored tensor of the given dtype (CPU)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch_dtype(dtype))


def _unit(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _raw_qk(q: np.ndarray, k: np.ndarray, rng: np.random.Generator) -> tuple[np.ndarray, np.ndarray]:
    """Unnormalised q and k: each vector along its drawn direction, with a norm drawn
    log-uniformly in [0.05, 20]; one q and one k vector zero, one of each at norm 1e-3."""
    out = []
    for x in (q, k):
        d = _unit(x)
        lead = d.shape[:-1]
        norms = np.exp(rng.uniform(np.log(0.05), np.log(20.0), lead))
        y = d * norms[..., None]
        flat = y.reshape(-1, y.shape[-1])
        if flat.shape[0] >= 2:
            zi, si = rng.choice(flat.shape[0], size=2, replace=False)
            flat[zi] = 0.0
            flat[si] = d.reshape(-1, d.shape[-1])[si] * 1e-3
        out.append(y)
    return out[0], out[1]


def _weak_a_log(Hv: int, rng: np.random.Generator) -> np.ndarray:
    return np.log(rng.uniform(0.02, 0.05, Hv))


def _variant(seed: int) -> np.random.Generator:
    return np.random.default_rng([seed, 1])


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Draw one batch of inputs for workload ``w``. Returns CPU torch tensors."""
    rng = np.random.default_rng(seed)
    B, T, Hk, Hv, dk, dv, P = w.batch, w.T, w.Hk, w.Hv, w.dk, w.dv, w.pool
    # 1. slot indices
    if w.fixed_indices is not None:
        idx = np.asarray(w.fixed_indices, dtype=np.int32)
        assert idx.shape == (B,)
    else:
        assert B <= P, "more rows than pool slots"
        idx = rng.permutation(P)[:B].astype(np.int32)
        if w.n_pad:
            pad = rng.choice(B, size=w.n_pad, replace=False)
            idx[pad] = -1
    # 2. per-token inputs
    q = _unit(rng.standard_normal((B, T, Hk, dk)))
    k = _unit(rng.standard_normal((B, T, Hk, dk)))
    v = rng.standard_normal((B, T, Hv, dv))
    a = rng.standard_normal((B, T, Hv))
    b = rng.standard_normal((B, T, Hv))
    # 3. per-head parameters (fp32)
    A_log = np.log(rng.uniform(1.0, 16.0, Hv))
    dt_bias = rng.normal(0.0, 0.1, Hv)
    # 4. state pool
    pool = rng.standard_normal((P, Hv, dk, dv), dtype=np.float32)
    pool *= np.float32(0.1)
    if w.qk == "raw" or w.decay == "weak":
        vr = _variant(seed)
        if w.qk == "raw":
            q, k = _raw_qk(q, k, vr)
        if w.decay == "weak":
            A_log = _weak_a_log(Hv, vr)
    out = dict(
        idx=torch.from_numpy(idx),
        q=_store(q, w.io_dtype), k=_store(k, w.io_dtype), v=_store(v, w.io_dtype),
        a=_store(a, w.io_dtype), b=_store(b, w.io_dtype),
        A_log=torch.from_numpy(A_log.astype(np.float32)),
        dt_bias=torch.from_numpy(dt_bias.astype(np.float32)),
        pool=_store(pool, w.state_dtype),
    )
    del pool
    # 5. accept lengths and, for the fused commit, the previous step's cache
    if w.commit:
        out["accept"] = torch.from_numpy(rng.integers(1, T + 1, B).astype(np.int32))
    if w.mode == "verify_fused":
        prev = rng.integers(1, w.cache_T + 1, B).astype(np.int32)
        out["prev_accept"] = torch.from_numpy(prev)
        cache = torch.zeros((B, w.cache_T, Hv, dk, dv), dtype=torch_dtype(w.state_dtype))
        for r in range(B):
            if 0 <= idx[r] < P:
                s = rng.standard_normal((Hv, dk, dv), dtype=np.float32) * np.float32(0.1)
                cache[r, prev[r] - 1] = _store(s, w.state_dtype)
        out["cache_prev"] = cache
    return out


def to_device_state(s: torch.Tensor) -> torch.Tensor:
    """[..., dk, dv] logical state -> [..., dv, dk] device layout (contiguous)."""
    return s.transpose(-1, -2).contiguous()


def from_device_state(s: torch.Tensor) -> torch.Tensor:
    """[..., dv, dk] device layout -> [..., dk, dv] logical state."""
    return s.transpose(-1, -2)


def state_read_bytes(w: Workload, idx: np.ndarray) -> int:
    """Bytes of state one call reads (one tile per valid row and v-head)."""
    ssz = 4 if w.state_dtype == "f32" else 2
    valid = int(np.sum((idx >= 0) & (idx < w.pool)))
    return valid * w.Hv * w.dk * w.dv * ssz


def replay_bytes(w: Workload, idx: np.ndarray, rlen: np.ndarray, commit: bool = True) -> int:
    """Bytes one cached-replay verify must move: each valid tile read once, written once
    more if its row commits a replayed prefix, the new tokens' io and o, and the
    replayed tokens' k, v, a, b."""
    ssz = 4 if w.state_dtype == "f32" else 2
    isz = 4 if w.io_dtype == "f32" else 2
    valid = (idx >= 0) & (idx < w.pool)
    n = np.where(valid & (rlen >= 0) & (rlen <= w.T), rlen, 0)
    tile = w.dk * w.dv * ssz
    state = int(valid.sum()) * w.Hv * tile + (int(np.sum(valid & (n >= 1))) * w.Hv * tile if commit else 0)
    per_tok = (2 * w.Hk * w.dk + w.Hv * w.dv + 2 * w.Hv) * isz
    io = int(valid.sum()) * w.T * per_tok + w.batch * w.T * w.Hv * w.dv * isz
    io += int(n.sum()) * (w.Hk * w.dk + w.Hv * w.dv + 2 * w.Hv) * isz
    return state + io + w.batch * 8 + 2 * w.Hv * 4


def algorithmic_bytes(w: Workload, idx: np.ndarray, kind: str) -> int:
    """Bytes the method must move for one call: each valid (row, v-head) state tile
    read once and written once per stored state, plus the per-token io.

    kind: "verify" (this workload's verify/decode call) or "commit".
    """
    ssz = 4 if w.state_dtype == "f32" else 2
    isz = 4 if w.io_dtype == "f32" else 2
    valid = int(np.sum((idx >= 0) & (idx < w.pool)))
    tile = w.dk * w.dv * ssz
    tiles = valid * w.Hv
    if kind == "commit":
        return tiles * tile * 2 + valid * 4 * 2
    writes = 0
    if w.mode == "decode":
        writes = 1
    else:
        writes = (w.T if w.cache_T else 0) + (1 if w.write_final else 0)
        if w.mode == "verify_fused":
            writes += 1
    state = tiles * tile * (1 + writes)
    B, T = w.batch, w.T
    io = valid * T * (2 * w.Hk * w.dk + w.Hv * w.dv + 2 * w.Hv) * isz  # q, k, v, a, b of valid rows
    io += B * T * w.Hv * w.dv * isz                                     # o, every row
    io += B * 4 + 2 * w.Hv * 4                                          # indices, A_log, dt_bias
    if w.mode == "verify_fused":
        io += B * 4
    return state + io


# ---------------------------------------------------------------- short convolution
# The short causal convolution over the mixed q/k/v channels whose state sits in a pool
# next to the GDN state (TensorRT-LLM PR 20937, What changes: the in_proj GEMV's fused
# conv1d epilogue for verify and decode rows; Per-File QA Perspective: convolution state
# staged and committed per accepted prefix). Its channels are D = 2*Hk*dk + Hv*dv of
# the GDN layer it feeds; width K = 4.
#
# Recipe (one ``numpy.random.default_rng(seed)``, in this order): slot indices as for
# the GDN workloads; x ~ N(0,1) [B,T,D]; taps w ~ N(0, 1/K) [K,D] and bias ~ N(0, 0.1)
# [D] (fp32); the state pool ~ N(0,1) [P,K-1,D] (earlier inputs); accept lengths
# ~ U{1..T}; the previous step's inputs ~ N(0,1) [B,T,D] and accept lengths ~ U{1..T}.
# x, the pool and the previous inputs are stored in the workload's dtype.


@dataclasses.dataclass(frozen=True)
class ConvWorkload:
    name: str
    batch: int
    T: int
    channels: int
    width: int
    pool: int
    dtype: str                # "f32" | "bf16"
    mode: str                 # "verify" (read-only) | "fused" (commit of the previous step, then verify) | "decode"
    activation: str = "silu"
    n_pad: int = 0
    description: str = ""

    def replace(self, **kw) -> "ConvWorkload":
        return dataclasses.replace(self, **kw)


def conv_channels(Hk: int, Hv: int, dk: int, dv: int) -> int:
    return 2 * Hk * dk + Hv * dv


CONV_WORKLOADS: list[ConvWorkload] = [
    ConvWorkload("conv-tiny-f32", batch=3, T=2, channels=16, width=4, pool=5, dtype="f32", mode="fused", n_pad=1,
                 description="tiny: B=3 (1 padding), T=2, D=16, K=4, fp32, fused commit"),
    ConvWorkload("conv-mtp-t4-bf16", batch=64, T=4, channels=conv_channels(4, 8, 128, 128), width=4, pool=256,
                 dtype="bf16", mode="fused",
                 description="MTP verify T=4 of the headline GDN layer: B=64, D=2048, K=4, bf16, fused commit"),
    ConvWorkload("conv-decode-f32", batch=64, T=1, channels=conv_channels(4, 8, 128, 128), width=4, pool=256,
                 dtype="f32", mode="decode", n_pad=8,
                 description="decode: B=64 (8 padding), D=2048, K=4, fp32, state written back"),
    ConvWorkload("conv-t8-bf16", batch=128, T=8, channels=conv_channels(16, 32, 128, 128), width=4, pool=1024,
                 dtype="bf16", mode="fused", n_pad=13,
                 description="verify T=8: B=128 (13 padding), D=8192, K=4, bf16, fused commit"),
]
CONV_HEADLINE = 1


def make_conv_inputs(w: ConvWorkload, seed: int = 0) -> dict:
    """Draw one batch of short-convolution inputs. Returns CPU torch tensors."""
    rng = np.random.default_rng(seed)
    B, T, D, K, P = w.batch, w.T, w.channels, w.width, w.pool
    assert B <= P, "more rows than pool slots"
    idx = rng.permutation(P)[:B].astype(np.int32)
    if w.n_pad:
        idx[rng.choice(B, size=w.n_pad, replace=False)] = -1
    x = rng.standard_normal((B, T, D))
    taps = rng.normal(0.0, 1.0 / math.sqrt(K), (K, D))
    bias = rng.normal(0.0, 0.1, D)
    pool = rng.standard_normal((P, K - 1, D), dtype=np.float32)
    accept = rng.integers(1, T + 1, B).astype(np.int32)
    prev_x = rng.standard_normal((B, T, D))
    prev_len = rng.integers(1, T + 1, B).astype(np.int32)
    return dict(idx=torch.from_numpy(idx), x=_store(x, w.dtype),
                w=torch.from_numpy(taps.astype(np.float32)), bias=torch.from_numpy(bias.astype(np.float32)),
                pool=_store(pool, w.dtype), accept=torch.from_numpy(accept),
                prev_x=_store(prev_x, w.dtype), prev_len=torch.from_numpy(prev_len))


def conv_bytes(w: ConvWorkload, idx: np.ndarray, prev_len: np.ndarray | None = None) -> int:
    """Bytes one convolution update must move: x of valid rows, y of all rows, taps and
    bias, the K-1 history rows of each valid row read once (a fused commit of n tokens
    takes min(n, K-1) of them from the previous step's inputs and the rest from the
    state), the state written once when the row commits (fused commit with
    1 <= prev_len <= T, or write-back), and the slot indices and commit lengths."""
    esz = 4 if w.dtype == "f32" else 2
    B, T, D, H = w.batch, w.T, w.channels, w.width - 1
    valid = (idx >= 0) & (idx < w.pool)
    nv = int(valid.sum())
    total = nv * T * D * esz + B * T * D * esz + (H + 2) * D * 4 + B * 4 + nv * H * D * esz
    if w.mode == "decode":
        total += nv * H * D * esz
    elif w.mode == "fused" and prev_len is not None:
        n = np.where(valid & (prev_len >= 1) & (prev_len <= T), prev_len, 0)
        total += int(np.sum(n >= 1)) * H * D * esz + B * 4
    return total


def make_gate_inputs(w: Workload, seed: int = 0) -> dict:
    """Inputs of the gated RMS normalisation of the output: the gate z ~ N(0,1) shaped like
    v (io dtype) and the norm weight ~ U[0.5, 1.5) over d_v (fp32), from their own
    ``numpy.random.default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((w.batch, w.T, w.Hv, w.dv))
    weight = rng.uniform(0.5, 1.5, w.dv)
    return dict(z=_store(z, w.io_dtype), norm_weight=torch.from_numpy(weight.astype(np.float32)))


# ---------------------------------------------------------------- chunked prefill
# Prefill of variable-length sequences from pooled initial states, with a mask that zeroes
# fresh states (TensorRT-LLM PR 20937, Per-File QA Perspective: the chunked gated delta
# rule prefill with a bf16 state and an initial-state mask). Tokens of all sequences are
# packed along the first axis (q, k [N,Hk,dk], v [N,Hv,dv], a, b [N,Hv]); cu_seqlens
# [B+1] are the offsets.
#
# Recipe (one ``numpy.random.default_rng(seed)``, in this order): slot indices as for the
# GDN workloads (n_pad rows set to -1); fresh flags: n_fresh distinct rows; q, k ~ N(0,1)
# L2-normalised per vector; v, a, b ~ N(0,1); A_log = log U[1,16), dt_bias ~ N(0, 0.1);
# the pool ~ N(0, 0.1) in float32. The "raw" q/k and "weak" decay variants are those of
# the module docstring, drawn the same way.


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    seqlens: tuple
    Hk: int
    Hv: int
    dk: int
    dv: int
    pool: int
    state_dtype: str
    io_dtype: str
    n_fresh: int = 0
    n_pad: int = 0
    description: str = ""
    qk: str = "unit"          # as for Workload: "raw" keeps q, k unnormalised
    decay: str = "strong"     # as for Workload: "weak" draws A_log = log U[0.02, 0.05)

    def replace(self, **kw) -> "PrefillWorkload":
        return dataclasses.replace(self, **kw)

    @property
    def batch(self) -> int:
        return len(self.seqlens)

    @property
    def tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def scale(self) -> float:
        return self.dk ** -0.5


PREFILL_WORKLOADS: list[PrefillWorkload] = [
    PrefillWorkload("prefill-tiny-f32", seqlens=(5, 0, 19, 16), Hk=1, Hv=2, dk=16, dv=16, pool=6,
                    state_dtype="f32", io_dtype="f32", n_fresh=1, n_pad=1,
                    description="tiny: 4 sequences (one empty, one padding, one fresh), d=16"),
    PrefillWorkload("prefill-mixed-bf16", seqlens=(1, 17, 64, 300, 1000, 16, 555, 33), Hk=4, Hv=8, dk=128, dv=128,
                    pool=32, state_dtype="bf16", io_dtype="bf16", n_fresh=2, n_pad=1,
                    description="mixed lengths 1..1000, Hk=4, Hv=8, d=128, bf16, 2 fresh, 1 padding"),
    PrefillWorkload("prefill-8x2048-bf16", seqlens=(2048,) * 8, Hk=4, Hv=8, dk=128, dv=128, pool=64,
                    state_dtype="bf16", io_dtype="bf16", n_fresh=4,
                    description="8 sequences x 2048 tokens, Hk=4, Hv=8 (one GPU's share at TP=4), d=128, bf16"),
    PrefillWorkload("prefill-4x4096-f32", seqlens=(4096,) * 4, Hk=16, Hv=32, dk=128, dv=128, pool=16,
                    state_dtype="f32", io_dtype="bf16", n_fresh=2,
                    description="4 sequences x 4096 tokens, Hk=16, Hv=32, d=128, fp32 state, bf16 io"),
    PrefillWorkload("prefill-1x16384-bf16", seqlens=(16384,), Hk=4, Hv=8, dk=128, dv=128, pool=2,
                    state_dtype="bf16", io_dtype="bf16",
                    description="one long prompt of 16384 tokens, Hk=4, Hv=8, d=128, bf16"),
]
PREFILL_HEADLINE = 2


def make_prefill_inputs(w: PrefillWorkload, seed: int = 0) -> dict:
    """Draw one prefill batch. Returns CPU torch tensors."""
    rng = np.random.default_rng(seed)
    B, N, Hk, Hv, dk, dv, P = w.batch, w.tokens, w.Hk, w.Hv, w.dk, w.dv, w.pool
    assert B <= P, "more sequences than pool slots"
    idx = rng.permutation(P)[:B].astype(np.int32)
    if w.n_pad:
        idx[rng.choice(B, size=w.n_pad, replace=False)] = -1
    fresh = np.zeros(B, np.int32)
    if w.n_fresh:
        fresh[rng.choice(B, size=w.n_fresh, replace=False)] = 1
    cu = np.concatenate([[0], np.cumsum(w.seqlens)]).astype(np.int32)
    q = _unit(rng.standard_normal((N, Hk, dk)))
    k = _unit(rng.standard_normal((N, Hk, dk)))
    v = rng.standard_normal((N, Hv, dv))
    a = rng.standard_normal((N, Hv))
    b = rng.standard_normal((N, Hv))
    A_log = np.log(rng.uniform(1.0, 16.0, Hv))
    dt_bias = rng.normal(0.0, 0.1, Hv)
    pool = rng.standard_normal((P, Hv, dk, dv), dtype=np.float32) * np.float32(0.1)
    if w.qk == "raw" or w.decay == "weak":
        vr = _variant(seed)
        if w.qk == "raw":
            q, k = _raw_qk(q, k, vr)
        if w.decay == "weak":
            A_log = _weak_a_log(Hv, vr)
    return dict(idx=torch.from_numpy(idx), fresh=torch.from_numpy(fresh), cu_seqlens=torch.from_numpy(cu),
                q=_store(q, w.io_dtype), k=_store(k, w.io_dtype), v=_store(v, w.io_dtype),
                a=_store(a, w.io_dtype), b=_store(b, w.io_dtype),
                A_log=torch.from_numpy(A_log.astype(np.float32)), dt_bias=torch.from_numpy(dt_bias.astype(np.float32)),
                pool=_store(pool, w.state_dtype))


def prefill_flops(w: PrefillWorkload, chunk: int = 16) -> int:
    """Flops of the chunked form per call (each product counted once, 2 flop per
    multiply-add): per chunk of C tokens and v-head, K K^T, Q K^T and W (2 C^2 d_k each),
    U~ and P U (2 C^2 d_v each), W S_0, Q S_0 and the state update (2 C d_k d_v each).
    Padding rows count nothing."""
    per_chunk = 3 * 2 * chunk * chunk * w.dk + 2 * 2 * chunk * chunk * w.dv + 3 * 2 * chunk * w.dk * w.dv
    chunks = sum((L + chunk - 1) // chunk for L in w.seqlens)
    return per_chunk * chunks * w.Hv


def prefill_bytes(w: PrefillWorkload) -> int:
    """Bytes one prefill must move: q, k (per k-head), v, a, b and o of every token, and
    each valid sequence's state tiles read once and written once (bf16 io)."""
    esz = 2
    ssz = 4 if w.state_dtype == "f32" else 2
    tok = w.tokens * (2 * w.Hk * w.dk + 2 * w.Hv * w.dv + 2 * w.Hv) * esz
    return tok + 2 * w.batch * w.Hv * w.dk * w.dv * ssz
