"""Python binding of libgdn.so, the gfx950 Gated DeltaNet state-update library.

Argument marshalling only: shapes, dtypes, devices and contiguity of torch tensors
are turned into the plain pointers and sizes of ``include/gdn.h``, and the calls go
through ctypes on the current HIP stream. Every step of decode, verify and commit
runs in the HIP kernels; there is no other code path. If the library has not been
built, importing works but the first call raises.

Layouts (see include/gdn.h): q, k [B,T,Hk,dk]; v, o [B,T,Hv,dv]; a, b [B,T,Hv];
A_log, dt_bias [Hv] fp32; state_pool [P,Hv,dv,dk]; inter_cache [B,cache_T,Hv,dv,dk];
state_indices, accept lengths [B] int32.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_DTYPE_F32, GDN_DTYPE_BF16 = 0, 1
STATUS = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_DTYPE", 4: "GDN_ERR_ALIGN",
          5: "GDN_ERR_UNSUPPORTED", 6: "GDN_ERR_LAUNCH", 7: "GDN_ERR_TOO_LARGE"}
EXPORTED = ("gdn_decode", "gdn_verify", "gdn_verify_gated", "gdn_prefill", "gdn_prefill_noalloc",
            "gdn_prefill_workspace_bytes", "gdn_commit", "gdn_verify_replay", "gdn_commit_replay", "gdn_conv_update",
            "gdn_conv_commit", "gdn_status_string", "gdn_abi_version")
GDN_PREFILL_NOALLOC_BYTES = 128 << 20
GDN_CONV_MAX_WIDTH = 8
GDN_MAX_T = 16


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class GdnDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("T", ctypes.c_int32), ("num_k_heads", ctypes.c_int32),
                ("num_v_heads", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("pool_slots", ctypes.c_int32), ("state_dtype", ctypes.c_int), ("io_dtype", ctypes.c_int),
                ("scale", ctypes.c_float), ("l2norm_eps", ctypes.c_float)]


class GdnIo(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("o", ctypes.c_void_p)]


class GdnOutGate(ctypes.Structure):
    _fields_ = [("z", ctypes.c_void_p), ("weight", ctypes.c_void_p), ("eps", ctypes.c_float)]


class GdnTokens(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("a", ctypes.c_void_p), ("b", ctypes.c_void_p),
                ("T_src", ctypes.c_int32)]


class GdnConvDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("T", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("width", ctypes.c_int32), ("pool_slots", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("activation", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library with its C signatures. Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        D, I = ctypes.POINTER(GdnDims), ctypes.POINTER(GdnIo)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.gdn_decode.argtypes = [D, I, vp, vp, vp]
        L.gdn_verify.argtypes = [D, I, vp, vp, vp, i32, i32, vp, vp]
        L.gdn_commit.argtypes = [D, vp, i32, vp, vp, vp, vp]
        L.gdn_verify_gated.argtypes = [D, I, ctypes.POINTER(GdnOutGate), vp, vp, vp, i32, i32, vp, vp]
        L.gdn_prefill.argtypes = [D, I, vp, vp, vp, vp, ctypes.c_int64, vp, ctypes.c_size_t, vp]
        L.gdn_prefill_noalloc.argtypes = [D, I, vp, vp, vp, vp, ctypes.c_int64, vp]
        L.gdn_prefill_workspace_bytes.argtypes = [D, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
        TK = ctypes.POINTER(GdnTokens)
        L.gdn_verify_replay.argtypes = [D, I, vp, vp, TK, vp, i32, vp]
        L.gdn_commit_replay.argtypes = [D, vp, vp, vp, vp, TK, vp, vp]
        CD = ctypes.POINTER(GdnConvDims)
        L.gdn_conv_update.argtypes = [CD, vp, vp, vp, vp, vp, vp, i32, vp, vp, i32, vp]
        L.gdn_conv_commit.argtypes = [CD, vp, vp, vp, vp, vp]
        for f in ("gdn_decode", "gdn_verify", "gdn_verify_gated", "gdn_prefill", "gdn_prefill_noalloc",
                  "gdn_prefill_workspace_bytes", "gdn_commit", "gdn_verify_replay", "gdn_commit_replay",
                  "gdn_conv_update", "gdn_conv_commit"):
            getattr(L, f).restype = ctypes.c_int
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def _raise(status: int, what: str):
    if status != 0:
        raise GdnError(status, f"{what}: {status_string(status)}")


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GDN_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, ndim: int, device: torch.device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, has {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device: torch.device, stream) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dims_io(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, scale, l2norm_eps):
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    _need(q, "q", 4, dev); _need(k, "k", 4, dev); _need(v, "v", 4, dev); _need(o, "o", 4, dev)
    _need(a, "a", 3, dev); _need(b, "b", 3, dev); _need(A_log, "A_log", 1, dev); _need(dt_bias, "dt_bias", 1, dev)
    _need(state_pool, "state_pool", 4, dev); _need(state_indices, "state_indices", 1, dev)
    B, T, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    P = state_pool.shape[0]
    if k.shape != q.shape or v.shape != (B, T, Hv, dv) or o.shape != v.shape:
        raise ValueError("q/k/v/o shapes disagree")
    if a.shape != (B, T, Hv) or b.shape != (B, T, Hv):
        raise ValueError("a and b must be [B, T, Hv]")
    if A_log.shape != (Hv,) or dt_bias.shape != (Hv,):
        raise ValueError("A_log and dt_bias must be [Hv]")
    if A_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
        raise TypeError("A_log and dt_bias must be float32")
    if state_pool.shape[1:] != (Hv, dv, dk):
        raise ValueError(f"state_pool must be [P, Hv, dv, dk] = [P, {Hv}, {dv}, {dk}]")
    if state_indices.shape != (B,) or state_indices.dtype != torch.int32:
        raise ValueError("state_indices must be int32 [B]")
    io_dt = _dt(q)
    for name, t in (("k", k), ("v", v), ("a", a), ("b", b), ("o", o)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} must have the io dtype {q.dtype}")
    dims = GdnDims(B, T, Hk, Hv, dk, dv, P, _dt(state_pool), io_dt,
                   float(dk ** -0.5 if scale is None else scale), float(l2norm_eps))
    io = GdnIo(q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(), A_log.data_ptr(),
               dt_bias.data_ptr(), o.data_ptr())
    return dims, io


def gdn_decode(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, *, scale=None,
               l2norm_eps=1e-6, stream=None) -> None:
    """One token per row; the state of each valid slot is updated in place; o is written."""
    dims, io = _dims_io(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, scale, l2norm_eps)
    st = lib().gdn_decode(ctypes.byref(dims), ctypes.byref(io), _ptr(state_pool), _ptr(state_indices),
                          _stream(q.device, stream))
    _raise(st, "gdn_decode")


def _cache_prev(dims, state_pool, inter_cache, prev_accept_len, device) -> int:
    cache_T = 0
    if inter_cache is not None:
        _need(inter_cache, "inter_cache", 5, device)
        if inter_cache.shape[0] != dims.batch or inter_cache.shape[2:] != state_pool.shape[1:]:
            raise ValueError("inter_cache must be [B, cache_T, Hv, dv, dk]")
        if inter_cache.dtype != state_pool.dtype:
            raise TypeError("inter_cache must have the state dtype")
        cache_T = inter_cache.shape[1]
    if prev_accept_len is not None:
        _need(prev_accept_len, "prev_accept_len", 1, device)
        if prev_accept_len.shape != (dims.batch,) or prev_accept_len.dtype != torch.int32:
            raise ValueError("prev_accept_len must be int32 [B]")
    return cache_T


def gdn_verify(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, inter_cache=None,
               write_final=False, prev_accept_len=None, *, scale=None, l2norm_eps=1e-6, stream=None) -> None:
    """T tokens per row from its pool slot; see include/gdn.h for the cache, write_final
    and fused-commit (prev_accept_len) semantics."""
    dims, io = _dims_io(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, scale, l2norm_eps)
    cache_T = _cache_prev(dims, state_pool, inter_cache, prev_accept_len, q.device)
    st = lib().gdn_verify(ctypes.byref(dims), ctypes.byref(io), _ptr(state_pool), _ptr(state_indices),
                          _ptr(inter_cache), cache_T, int(bool(write_final)), _ptr(prev_accept_len),
                          _stream(q.device, stream))
    _raise(st, "gdn_verify")


def gdn_verify_gated(q, k, v, a, b, A_log, dt_bias, z, norm_weight, y, state_pool, state_indices,
                     inter_cache=None, write_final=False, prev_accept_len=None, *, norm_eps=1e-6, scale=None,
                     l2norm_eps=1e-6, stream=None) -> None:
    """gdn_verify whose output y [B,T,Hv,dv] is the gated RMS normalisation
    norm_weight * o / sqrt(mean(o^2) + norm_eps) * silu(z) of each (row, token, v-head)
    vector, z [B,T,Hv,dv] in the io dtype, norm_weight [dv] fp32."""
    dims, io = _dims_io(q, k, v, a, b, A_log, dt_bias, y, state_pool, state_indices, scale, l2norm_eps)
    _need(z, "z", 4, q.device); _need(norm_weight, "norm_weight", 1, q.device)
    if z.shape != v.shape or z.dtype != v.dtype:
        raise ValueError("z must match v in shape and dtype")
    if norm_weight.shape != (dims.d_v,) or norm_weight.dtype != torch.float32:
        raise ValueError("norm_weight must be float32 [dv]")
    cache_T = _cache_prev(dims, state_pool, inter_cache, prev_accept_len, q.device)
    gate = GdnOutGate(z.data_ptr(), norm_weight.data_ptr(), float(norm_eps))
    st = lib().gdn_verify_gated(ctypes.byref(dims), ctypes.byref(io), ctypes.byref(gate), _ptr(state_pool),
                                _ptr(state_indices), _ptr(inter_cache), cache_T, int(bool(write_final)),
                                _ptr(prev_accept_len), _stream(q.device, stream))
    _raise(st, "gdn_verify_gated")


def gdn_commit(inter_cache, state_indices, accept_len, state_pool, *, stream=None) -> None:
    """state_pool[idx[r]] <- inter_cache[r, n-1] for rows with a valid slot and 1 <= n <= cache_T."""
    dev = inter_cache.device
    _need(inter_cache, "inter_cache", 5, dev); _need(state_indices, "state_indices", 1, dev)
    _need(accept_len, "accept_len", 1, dev); _need(state_pool, "state_pool", 4, dev)
    B, cache_T, Hv, dv, dk = inter_cache.shape
    if state_pool.shape[1:] != (Hv, dv, dk) or state_pool.dtype != inter_cache.dtype:
        raise ValueError("state_pool must be [P, Hv, dv, dk] in the cache's dtype")
    for name, t in (("state_indices", state_indices), ("accept_len", accept_len)):
        if t.shape != (B,) or t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32 [B]")
    dims = GdnDims(B, 1, 1, Hv, dk, dv, state_pool.shape[0], _dt(state_pool), _dt(state_pool), 1.0, 0.0)
    st = lib().gdn_commit(ctypes.byref(dims), _ptr(inter_cache), cache_T, _ptr(state_indices), _ptr(accept_len),
                          _ptr(state_pool), _stream(dev, stream))
    _raise(st, "gdn_commit")


def _tokens(rk, rv, ra, rb, B, Hk, Hv, dk, dv, io_dtype, device) -> GdnTokens:
    _need(rk, "replay_k", 4, device); _need(rv, "replay_v", 4, device)
    _need(ra, "replay_a", 3, device); _need(rb, "replay_b", 3, device)
    Ts = rk.shape[1]
    if rk.shape != (B, Ts, Hk, dk) or rv.shape != (B, Ts, Hv, dv) or ra.shape != (B, Ts, Hv) or rb.shape != (B, Ts, Hv):
        raise ValueError("replay arrays must be k [B,T_src,Hk,dk], v [B,T_src,Hv,dv], a and b [B,T_src,Hv]")
    for name, t in (("replay_k", rk), ("replay_v", rv), ("replay_a", ra), ("replay_b", rb)):
        if t.dtype != io_dtype:
            raise TypeError(f"{name} must have the io dtype {io_dtype}")
    return GdnTokens(rk.data_ptr(), rv.data_ptr(), ra.data_ptr(), rb.data_ptr(), Ts)


def _need_len(t, B, device, name="replay_len"):
    _need(t, name, 1, device)
    if t.shape != (B,) or t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32 [B]")


def gdn_verify_replay(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, replay_k, replay_v,
                      replay_a, replay_b, replay_len, commit=True, *, scale=None, l2norm_eps=1e-6,
                      stream=None) -> None:
    """Replay replay_len[r] tokens of an earlier verify (replay_* arrays) from each row's
    slot, commit the result to the slot if asked, then run this call's T tokens."""
    dims, io = _dims_io(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, scale, l2norm_eps)
    rep = _tokens(replay_k, replay_v, replay_a, replay_b, dims.batch, dims.num_k_heads, dims.num_v_heads,
                  dims.d_k, dims.d_v, q.dtype, q.device)
    _need_len(replay_len, dims.batch, q.device)
    st = lib().gdn_verify_replay(ctypes.byref(dims), ctypes.byref(io), _ptr(state_pool), _ptr(state_indices),
                                 ctypes.byref(rep), _ptr(replay_len), int(bool(commit)), _stream(q.device, stream))
    _raise(st, "gdn_verify_replay")


def gdn_commit_replay(A_log, dt_bias, state_pool, state_indices, replay_k, replay_v, replay_a, replay_b,
                      replay_len, *, l2norm_eps=1e-6, stream=None) -> None:
    """Separate replay commit: each valid row's slot advances through its replay_len[r]
    replayed tokens and is written back."""
    dev = state_pool.device
    _need(state_pool, "state_pool", 4, dev); _need(state_indices, "state_indices", 1, dev)
    _need(A_log, "A_log", 1, dev); _need(dt_bias, "dt_bias", 1, dev)
    B, Ts, Hk, dk = replay_k.shape
    P, Hv, dv, dk2 = state_pool.shape
    if dk2 != dk:
        raise ValueError("state_pool must be [P, Hv, dv, dk] with the replay arrays' dk")
    if A_log.shape != (Hv,) or dt_bias.shape != (Hv,) or A_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
        raise ValueError("A_log and dt_bias must be float32 [Hv]")
    if state_indices.shape != (B,) or state_indices.dtype != torch.int32:
        raise ValueError("state_indices must be int32 [B]")
    rep = _tokens(replay_k, replay_v, replay_a, replay_b, B, Hk, Hv, dk, dv, replay_k.dtype, dev)
    _need_len(replay_len, B, dev)
    dims = GdnDims(B, 1, Hk, Hv, dk, dv, P, _dt(state_pool), _dt(replay_k), 1.0, float(l2norm_eps))
    st = lib().gdn_commit_replay(ctypes.byref(dims), _ptr(A_log), _ptr(dt_bias), _ptr(state_pool),
                                 _ptr(state_indices), ctypes.byref(rep), _ptr(replay_len), _stream(dev, stream))
    _raise(st, "gdn_commit_replay")


# ---------------------------------------------------------------- short convolution
# Layouts: x, y [B,T,D]; prev_x [B,T_prev,D]; conv_pool [P,K-1,D] (x's dtype); weight
# [K,D] fp32; bias [D] fp32 or None; state_indices, prev_len, accept_len [B] int32.

_ACT = {"none": 0, "silu": 1}


def _conv_dims(x, conv_pool, state_indices, activation="silu") -> GdnConvDims:
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    _need(x, "x", 3, dev); _need(conv_pool, "conv_pool", 3, dev); _need(state_indices, "state_indices", 1, dev)
    B, T, D = x.shape
    P, H = conv_pool.shape[0], conv_pool.shape[1]
    if conv_pool.shape[2] != D or conv_pool.dtype != x.dtype:
        raise ValueError(f"conv_pool must be [P, K-1, {D}] of x's dtype")
    if state_indices.shape != (B,) or state_indices.dtype != torch.int32:
        raise ValueError("state_indices must be int32 [B]")
    return GdnConvDims(B, T, D, H + 1, P, _dt(x), _ACT[activation])


def gdn_conv_update(x, weight, bias, conv_pool, state_indices, y, *, prev_x=None, prev_len=None,
                    write_back=False, activation="silu", stream=None) -> None:
    """Short causal convolution of this call's tokens from each valid row's slot state:
    optional fused commit of prev_x's first prev_len[r] tokens before, optional
    write-back of the state advanced over all tokens after (decode)."""
    dims = _conv_dims(x, conv_pool, state_indices, activation)
    dev = x.device
    _need(weight, "weight", 2, dev); _need(y, "y", 3, dev)
    if weight.shape != (dims.width, dims.channels) or weight.dtype != torch.float32:
        raise ValueError(f"weight must be float32 [K, D] = [{dims.width}, {dims.channels}]")
    if bias is not None:
        _need(bias, "bias", 1, dev)
        if bias.shape != (dims.channels,) or bias.dtype != torch.float32:
            raise ValueError("bias must be float32 [D]")
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("y must match x")
    T_prev = 0
    if prev_x is not None:
        _need(prev_x, "prev_x", 3, dev); _need(prev_len, "prev_len", 1, dev)
        if prev_x.shape[0] != dims.batch or prev_x.shape[2] != dims.channels or prev_x.dtype != x.dtype:
            raise ValueError("prev_x must be [B, T_prev, D] of x's dtype")
        if prev_len.shape != (dims.batch,) or prev_len.dtype != torch.int32:
            raise ValueError("prev_len must be int32 [B]")
        T_prev = prev_x.shape[1]
    st = lib().gdn_conv_update(ctypes.byref(dims), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_pool),
                               _ptr(state_indices), _ptr(prev_x), int(T_prev),
                               _ptr(prev_len) if prev_x is not None else None, _ptr(y), int(bool(write_back)),
                               _stream(dev, stream))
    _raise(st, "gdn_conv_update")


def gdn_conv_commit(x, conv_pool, state_indices, accept_len, *, stream=None) -> None:
    """Accepted-prefix commit of the convolution state: each valid slot advances over the
    first accept_len[r] tokens of x (1 <= accept_len[r] <= T; other rows untouched)."""
    dims = _conv_dims(x, conv_pool, state_indices)
    _need(accept_len, "accept_len", 1, x.device)
    if accept_len.shape != (dims.batch,) or accept_len.dtype != torch.int32:
        raise ValueError("accept_len must be int32 [B]")
    st = lib().gdn_conv_commit(ctypes.byref(dims), _ptr(x), _ptr(conv_pool), _ptr(state_indices),
                               _ptr(accept_len), _stream(x.device, stream))
    _raise(st, "gdn_conv_commit")


# ---------------------------------------------------------------- chunked prefill
# Tokens of all sequences packed along the first axis: q, k [N,Hk,dk], v, o [N,Hv,dv],
# a, b [N,Hv]; cu_seqlens [B+1] int32 offsets; state_indices, fresh [B] int32.

def _prefill_dims(B, N, Hk, Hv, dk, dv, P, state_dt, io_dt, scale, eps):
    return GdnDims(B, 1, Hk, Hv, dk, dv, P, state_dt, io_dt, float(dk ** -0.5 if scale is None else scale),
                   float(eps))


def gdn_prefill_workspace_bytes(batch, num_tokens, num_k_heads, num_v_heads, d_k, d_v, state_dtype=torch.float32,
                                io_dtype=torch.bfloat16) -> int:
    """Bytes of the device workspace gdn_prefill needs for `batch` sequences with
    `num_tokens` packed tokens."""
    dims = _prefill_dims(batch, num_tokens, num_k_heads, num_v_heads, d_k, d_v, 0,
                         GDN_DTYPE_F32 if state_dtype == torch.float32 else GDN_DTYPE_BF16,
                         GDN_DTYPE_F32 if io_dtype == torch.float32 else GDN_DTYPE_BF16, None, 1e-6)
    out = ctypes.c_size_t(0)
    _raise(lib().gdn_prefill_workspace_bytes(ctypes.byref(dims), int(num_tokens), ctypes.byref(out)),
           "gdn_prefill_workspace_bytes")
    return int(out.value)


def _prefill_args(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, cu_seqlens, fresh, scale,
                  l2norm_eps):
    """Checks of the prefill tensors; returns (dims, io, N)."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    for n_, t_, nd in (("q", q, 3), ("k", k, 3), ("v", v, 3), ("o", o, 3), ("a", a, 2), ("b", b, 2),
                       ("A_log", A_log, 1), ("dt_bias", dt_bias, 1), ("state_pool", state_pool, 4),
                       ("state_indices", state_indices, 1), ("cu_seqlens", cu_seqlens, 1)):
        _need(t_, n_, nd, dev)
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    B = state_indices.shape[0]
    if k.shape != q.shape or v.shape != (N, Hv, dv) or o.shape != v.shape or a.shape != (N, Hv) or b.shape != (N, Hv):
        raise ValueError("q/k [N,Hk,dk], v/o [N,Hv,dv], a/b [N,Hv] disagree")
    if state_pool.shape[1:] != (Hv, dv, dk):
        raise ValueError(f"state_pool must be [P, {Hv}, {dv}, {dk}]")
    if cu_seqlens.shape != (B + 1,) or cu_seqlens.dtype != torch.int32 or state_indices.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32 [B+1], state_indices int32 [B]")
    if fresh is not None:
        _need(fresh, "fresh", 1, dev)
        if fresh.shape != (B,) or fresh.dtype != torch.int32:
            raise ValueError("fresh must be int32 [B]")
    for n_, t_ in (("k", k), ("v", v), ("o", o), ("a", a), ("b", b)):
        if t_.dtype != q.dtype:
            raise TypeError(f"{n_} must have q's dtype")
    if A_log.dtype != torch.float32 or dt_bias.dtype != torch.float32:
        raise TypeError("A_log and dt_bias must be float32")
    dims = _prefill_dims(B, N, Hk, Hv, dk, dv, state_pool.shape[0], _dt(state_pool), _dt(q), scale, l2norm_eps)
    io = GdnIo(q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(), A_log.data_ptr(),
               dt_bias.data_ptr(), o.data_ptr())
    return dims, io, N


def gdn_prefill(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, cu_seqlens, fresh=None, *,
                scale=None, l2norm_eps=1e-6, workspace=None, stream=None) -> None:
    """Prefill of variable-length sequences from pooled initial states (zero where fresh[r]);
    o for every token, the final state back to each valid slot. `workspace` is a device
    uint8 tensor of at least gdn_prefill_workspace_bytes(...) bytes; when it is omitted one
    is allocated for the call, which a call under HIP graph capture must not do (it raises
    then: pass a workspace, or use gdn_prefill_noalloc). cu_seqlens[-1] must not exceed
    q.shape[0]."""
    dims, io, N = _prefill_args(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, cu_seqlens, fresh,
                                scale, l2norm_eps)
    dev = q.device
    if workspace is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("gdn_prefill: no workspace given under HIP graph capture; pass a workspace of "
                               "gdn_prefill_workspace_bytes(...) bytes or call gdn_prefill_noalloc")
        need = ctypes.c_size_t(0)
        _raise(lib().gdn_prefill_workspace_bytes(ctypes.byref(dims), N, ctypes.byref(need)), "gdn_prefill")
        workspace = torch.empty(max(int(need.value), 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", 1, dev)
    if workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 tensor")
    st = lib().gdn_prefill(ctypes.byref(dims), ctypes.byref(io), _ptr(state_pool), _ptr(state_indices),
                           _ptr(cu_seqlens), _ptr(fresh), N, _ptr(workspace), workspace.numel(),
                           _stream(dev, stream))
    _raise(st, "gdn_prefill")


def gdn_prefill_noalloc(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, cu_seqlens, fresh=None, *,
                        scale=None, l2norm_eps=1e-6, stream=None) -> None:
    """gdn_prefill with its workspace in the library's fixed per-GPU device array
    (GDN_PREFILL_NOALLOC_BYTES): nothing is allocated, so it may run under HIP graph
    capture once one call has run on the GPU outside it. Raises GdnError with
    GDN_ERR_TOO_LARGE when the call needs more than the array. Calls on one GPU share the
    array: overlapping calls race."""
    dims, io, N = _prefill_args(q, k, v, a, b, A_log, dt_bias, o, state_pool, state_indices, cu_seqlens, fresh,
                                scale, l2norm_eps)
    st = lib().gdn_prefill_noalloc(ctypes.byref(dims), ctypes.byref(io), _ptr(state_pool), _ptr(state_indices),
                                   _ptr(cu_seqlens), _ptr(fresh), N, _stream(q.device, stream))
    _raise(st, "gdn_prefill_noalloc")
