"""ctypes wrapper of the float64 GDN oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``. The HIP library never imports or links it, and it
imports nothing from the HIP library.

All functions take and return NumPy arrays in the logical layouts of
``gdn_oracle.h`` (states as S[i][j], key index first). Inputs are the stored values
(bf16 / fp32 widened exactly to float64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "gdn_oracle.c"), os.path.join(_HERE, "conv_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict IEEE float64, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, *_SRCS, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("T", ctypes.c_int32),
                ("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("pool_slots", ctypes.c_int32), ("state_bf16", ctypes.c_int32),
                ("scale", ctypes.c_double), ("eps", ctypes.c_double)]


class ConvDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("T", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("width", ctypes.c_int32), ("pool_slots", ctypes.c_int32), ("activation", ctypes.c_int32)]


_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int32)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_softplus.argtypes = [ctypes.c_double]
        L.oracle_softplus.restype = ctypes.c_double
        L.oracle_gates.argtypes = [ctypes.c_double] * 4 + [_D, _D]
        L.oracle_gates.restype = None
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_round_bf16.restype = ctypes.c_double
        L.oracle_round_bf16_f32bits.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32]
        L.oracle_round_bf16_f32bits.restype = None
        L.oracle_verify.argtypes = [ctypes.POINTER(Dims)] + [_D] * 7 + [_D, _I, _D, ctypes.c_int32,
                                                                         ctypes.c_int32, _I, _D, ctypes.c_int32]
        L.oracle_verify.restype = ctypes.c_int32
        L.oracle_decode.argtypes = [ctypes.POINTER(Dims)] + [_D] * 7 + [_D, _I, _D, ctypes.c_int32]
        L.oracle_decode.restype = ctypes.c_int32
        L.oracle_commit.argtypes = [ctypes.POINTER(Dims), _D, ctypes.c_int32, _I, _I, _D, ctypes.c_int32]
        L.oracle_commit.restype = ctypes.c_int32
        L.oracle_verify_replay.argtypes = ([ctypes.POINTER(Dims)] + [_D] * 7 + [_D, _I] + [_D] * 4 +
                                           [ctypes.c_int32, _I, ctypes.c_int32, _D, ctypes.c_int32])
        L.oracle_verify_replay.restype = ctypes.c_int32
        L.oracle_commit_replay.argtypes = ([ctypes.POINTER(Dims), _D, _D, _D, _I] + [_D] * 4 +
                                           [ctypes.c_int32, _I, ctypes.c_int32])
        L.oracle_commit_replay.restype = ctypes.c_int32
        L.oracle_prefill.argtypes = [ctypes.POINTER(Dims), _I] + [_D] * 7 + [_D, _I, _I, _D, ctypes.c_int32]
        L.oracle_prefill.restype = ctypes.c_int32
        L.oracle_gated_norm.argtypes = [ctypes.c_int64, ctypes.c_int32, _D, _D, _D, ctypes.c_double, _D]
        L.oracle_gated_norm.restype = None
        CD = ctypes.POINTER(ConvDims)
        L.oracle_conv_update.argtypes = [CD, _D, _D, _D, _D, _I, _D, ctypes.c_int32, _I, _D, ctypes.c_int32]
        L.oracle_conv_update.restype = ctypes.c_int32
        L.oracle_conv_commit.argtypes = [CD, _D, _D, _I, _I]
        L.oracle_conv_commit.restype = ctypes.c_int32
        _lib = L
    return _lib


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.int32)


def _p(x: np.ndarray | None, t=_D):
    return None if x is None else x.ctypes.data_as(t)


def host_threads() -> int:
    """Threads the oracle uses by default: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when that is set (a machine that shares its host between GPUs grants
    each job a share through it)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def _nthreads(n):
    return int(n) if n else host_threads()


def softplus(x: float) -> float:
    return lib().oracle_softplus(float(x))


def gates(a: float, b: float, A_log: float, dt_bias: float) -> tuple[float, float]:
    g, beta = ctypes.c_double(), ctypes.c_double()
    lib().oracle_gates(float(a), float(b), float(A_log), float(dt_bias), ctypes.byref(g), ctypes.byref(beta))
    return g.value, beta.value


def round_bf16(x: float) -> float:
    return lib().oracle_round_bf16(float(x))


def round_bf16_f32bits(bits: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    out = np.empty(bits.shape, dtype=np.uint16)
    lib().oracle_round_bf16_f32bits(bits.ctypes.data, out.ctypes.data, bits.size, _nthreads(nthreads))
    return out


def make_dims(batch, T, Hk, Hv, dk, dv, pool, state_bf16, scale=None, eps=1e-6) -> Dims:
    return Dims(batch, T, Hk, Hv, dk, dv, pool, int(bool(state_bf16)),
                float(dk ** -0.5 if scale is None else scale), float(eps))


def verify(dims: Dims, q, k, v, a, b, A_log, dt_bias, pool, idx, *, cache_T: int = 0,
           write_final: bool = False, prev_accept=None, cache_in=None,
           nthreads: int | None = None) -> dict:
    """Run T verify tokens per row. Returns dict(o, pool, cache) (new arrays).

    ``cache_in`` is the cache content before the call (the previous step's
    intermediates for a fused commit); rows the call does not write keep it.
    """
    B, T, Hv, dk, dv = dims.batch, dims.T, dims.num_v_heads, dims.d_k, dims.d_v
    q, k, v, a, b = map(_f64, (q, k, v, a, b))
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    pool = _f64(pool).copy()
    idx = _i32(idx)
    o = np.zeros((B, T, Hv, dv), dtype=np.float64)
    cache = None
    if cache_T:
        cache = (_f64(cache_in).copy() if cache_in is not None
                 else np.zeros((B, cache_T, Hv, dk, dv), dtype=np.float64))
    pa = None if prev_accept is None else _i32(prev_accept)
    rc = lib().oracle_verify(ctypes.byref(dims), _p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log),
                             _p(dt_bias), _p(pool), _p(idx, _I), _p(cache), int(cache_T),
                             int(bool(write_final)), _p(pa, _I), _p(o), _nthreads(nthreads))
    if rc:
        raise ValueError("oracle_verify: invalid dimensions")
    return dict(o=o, pool=pool, cache=cache)


def decode(dims: Dims, q, k, v, a, b, A_log, dt_bias, pool, idx, *, nthreads: int | None = None) -> dict:
    """One token per row; the state is updated in its pool slot. Returns dict(o, pool)."""
    B, Hv, dv = dims.batch, dims.num_v_heads, dims.d_v
    q, k, v, a, b = map(_f64, (q, k, v, a, b))
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    pool = _f64(pool).copy()
    idx = _i32(idx)
    o = np.zeros((B, 1, Hv, dv), dtype=np.float64)
    rc = lib().oracle_decode(ctypes.byref(dims), _p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log),
                             _p(dt_bias), _p(pool), _p(idx, _I), _p(o), _nthreads(nthreads))
    if rc:
        raise ValueError("oracle_decode: invalid dimensions")
    return dict(o=o, pool=pool)


def commit(dims: Dims, cache, cache_T: int, idx, accept, pool, *, nthreads: int | None = None) -> np.ndarray:
    """Accepted-prefix commit. Returns the new pool."""
    cache = _f64(cache)
    pool = _f64(pool).copy()
    rc = lib().oracle_commit(ctypes.byref(dims), _p(cache), int(cache_T), _p(_i32(idx), _I),
                             _p(_i32(accept), _I), _p(pool), _nthreads(nthreads))
    if rc:
        raise ValueError("oracle_commit: invalid dimensions")
    return pool


def verify_replay(dims: Dims, q, k, v, a, b, A_log, dt_bias, pool, idx, rk, rv, ra, rb, rlen, *,
                  commit: bool = True, nthreads: int | None = None) -> dict:
    """Replay rlen[r] cached tokens (rk, rv, ra, rb: [B, rT, ...]) from each row's slot,
    commit the result to the slot if asked, then run this call's T tokens.
    Returns dict(o, pool)."""
    B, T, Hv, dv = dims.batch, dims.T, dims.num_v_heads, dims.d_v
    q, k, v, a, b, rk, rv, ra, rb = map(_f64, (q, k, v, a, b, rk, rv, ra, rb))
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    pool = _f64(pool).copy()
    o = np.zeros((B, T, Hv, dv), dtype=np.float64)
    rT = rk.shape[1]
    rc = lib().oracle_verify_replay(ctypes.byref(dims), _p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log),
                                    _p(dt_bias), _p(pool), _p(_i32(idx), _I), _p(rk), _p(rv), _p(ra), _p(rb),
                                    int(rT), _p(_i32(rlen), _I), int(bool(commit)), _p(o), _nthreads(nthreads))
    if rc:
        raise ValueError("oracle_verify_replay: invalid dimensions")
    return dict(o=o, pool=pool)


def commit_replay(dims: Dims, A_log, dt_bias, pool, idx, rk, rv, ra, rb, rlen, *,
                  nthreads: int | None = None) -> np.ndarray:
    """Separate replay commit. Returns the new pool."""
    rk, rv, ra, rb = map(_f64, (rk, rv, ra, rb))
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    pool = _f64(pool).copy()
    rc = lib().oracle_commit_replay(ctypes.byref(dims), _p(A_log), _p(dt_bias), _p(pool), _p(_i32(idx), _I),
                                    _p(rk), _p(rv), _p(ra), _p(rb), int(rk.shape[1]), _p(_i32(rlen), _I),
                                    _nthreads(nthreads))
    if rc:
        raise ValueError("oracle_commit_replay: invalid dimensions")
    return pool


def prefill(dims: Dims, cu_seqlens, q, k, v, a, b, A_log, dt_bias, pool, idx, fresh=None, *,
            nthreads: int | None = None) -> dict:
    """Prefill of variable-length sequences packed along the first axis (q, k [N,Hk,dk],
    v [N,Hv,dv], a, b [N,Hv]; cu_seqlens [B+1]) from pooled initial states (zero where
    fresh[r] != 0). Returns dict(o [N,Hv,dv], pool)."""
    q, k, v, a, b = map(_f64, (q, k, v, a, b))
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    pool = _f64(pool).copy()
    cu = _i32(cu_seqlens)
    N = int(cu[-1])
    o = np.zeros((N, dims.num_v_heads, dims.d_v), dtype=np.float64)
    fr = None if fresh is None else _i32(fresh)
    rc = lib().oracle_prefill(ctypes.byref(dims), _p(cu, _I), _p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log),
                              _p(dt_bias), _p(pool), _p(_i32(idx), _I), _p(fr, _I), _p(o), _nthreads(nthreads))
    if rc:
        raise ValueError("oracle_prefill: invalid dimensions")
    return dict(o=o, pool=pool)


def gated_norm(o, z, weight, eps: float = 1e-6) -> np.ndarray:
    """y = weight * o / sqrt(mean(o^2) + eps) * silu(z) over the last axis (d_v)."""
    o, z, w = _f64(o), _f64(z), _f64(weight)
    if z.shape != o.shape or w.shape != (o.shape[-1],):
        raise ValueError("gated_norm: z must match o and weight must be [d_v]")
    y = np.empty_like(o)
    lib().oracle_gated_norm(int(o.size // o.shape[-1]), int(o.shape[-1]), _p(o), _p(z), _p(w), float(eps), _p(y))
    return y


def make_conv_dims(batch, T, channels, width, pool, activation="silu") -> ConvDims:
    return ConvDims(batch, T, channels, width, pool, {"none": 0, "silu": 1}[activation])


def conv_update(dims: ConvDims, x, w, bias, pool, idx, *, prev_x=None, prev_len=None,
                write_back: bool = False) -> dict:
    """Short causal convolution of this call's tokens (x [B, T, D]) from each valid row's
    slot state (pool [P, K-1, D]); optional fused commit of prev_x's first prev_len[r]
    tokens before, optional write-back of the advanced state after. Returns dict(y, pool)."""
    B, T, D = dims.batch, dims.T, dims.channels
    x, w = _f64(x), _f64(w)
    b = None if bias is None else _f64(bias)
    pool = _f64(pool).copy()
    y = np.zeros((B, T, D), dtype=np.float64)
    px = None if prev_x is None else _f64(prev_x)
    T_prev = 0 if px is None else px.shape[1]
    pl = None if px is None else _i32(prev_len)
    rc = lib().oracle_conv_update(ctypes.byref(dims), _p(x), _p(w), _p(b), _p(pool), _p(_i32(idx), _I), _p(px),
                                  int(T_prev), _p(pl, _I), _p(y), int(bool(write_back)))
    if rc:
        raise ValueError("oracle_conv_update: invalid dimensions")
    return dict(y=y, pool=pool)


def conv_commit(dims: ConvDims, x, pool, idx, accept) -> np.ndarray:
    """Accepted-prefix commit of the convolution state. Returns the new pool."""
    pool = _f64(pool).copy()
    rc = lib().oracle_conv_commit(ctypes.byref(dims), _p(_f64(x)), _p(pool), _p(_i32(idx), _I),
                                  _p(_i32(accept), _I))
    if rc:
        raise ValueError("oracle_conv_commit: invalid dimensions")
    return pool


def verify_commit_inplace(dims: Dims, q, k, v, a, b, A_log, dt_bias, pool, idx, cache, cache_T: int, accept, *,
                          nthreads: int | None = None) -> None:
    """One verify (every intermediate into ``cache``) then the commit of ``accept``, on
    float64 arrays prepared by the caller and updated in place: the same two oracle
    functions as ``verify`` and ``commit``, without their input conversions and copies, so
    that a timing of this call covers the oracle's own arithmetic only (the CPU baseline)."""
    for x in (q, k, v, a, b, A_log, dt_bias, pool, cache):
        assert x.dtype == np.float64 and x.flags.c_contiguous
    assert idx.dtype == np.int32 and accept.dtype == np.int32
    B, T, Hv, dv = dims.batch, dims.T, dims.num_v_heads, dims.d_v
    o = np.empty((B, T, Hv, dv), dtype=np.float64)
    n = _nthreads(nthreads)
    rc = lib().oracle_verify(ctypes.byref(dims), _p(q), _p(k), _p(v), _p(a), _p(b), _p(A_log), _p(dt_bias),
                             _p(pool), _p(idx, _I), _p(cache), int(cache_T), 0, None, _p(o), n)
    rc = rc or lib().oracle_commit(ctypes.byref(dims), _p(cache), int(cache_T), _p(idx, _I), _p(accept, _I),
                                   _p(pool), n)
    if rc:
        raise ValueError("oracle verify/commit: invalid dimensions")
