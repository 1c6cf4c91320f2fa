"""The C ABI without a GPU: the library loads, exports every declared symbol, and the
host-side validation returns the documented status before any launch."""
import ctypes
import os
import re

import pytest

import linear_attention_speculative_gdn_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn.so is not built (run __graft_entry__.build())")
    return gdn.lib()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^GDN_API\s+[\w\s\*]+?\b(gdn_\w+)\s*\(", text, flags=re.M)


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(gdn.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_only_abi_symbols_exported(L):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert {s for s in syms if not s.startswith("_")} == set(gdn.EXPORTED)


def test_abi_version_and_limits(L):
    text = open(HEADER).read()
    ver = int(re.search(r"#define GDN_ABI_VERSION (\d+)", text).group(1))
    assert L.gdn_abi_version() == ver
    assert int(re.search(r"#define GDN_MAX_T (\d+)", text).group(1)) == gdn.GDN_MAX_T


def test_status_strings(L):
    for code, name in gdn.STATUS.items():
        assert gdn.status_string(code).startswith(name)
    assert "unknown" in gdn.status_string(99)


# Fake device addresses: validation never dereferences them and returns before launch.
A16 = 0x10000


def dims(**kw):
    base = dict(batch=4, T=4, num_k_heads=2, num_v_heads=4, d_k=128, d_v=128, pool_slots=8,
                state_dtype=gdn.GDN_DTYPE_BF16, io_dtype=gdn.GDN_DTYPE_BF16, scale=128 ** -0.5, l2norm_eps=1e-6)
    base.update(kw)
    return gdn.GdnDims(**base)


def io(**kw):
    base = dict(q=A16, k=A16 * 2, v=A16 * 3, a=A16 * 4, b=A16 * 5, A_log=A16 * 6, dt_bias=A16 * 7, o=A16 * 8)
    base.update(kw)
    return gdn.GdnIo(**base)


def verify(L, d, i, pool=A16 * 9, idx=A16 * 10, cache=A16 * 11, cache_T=4, wf=0, prev=None):
    return L.gdn_verify(ctypes.byref(d) if d is not None else None, ctypes.byref(i) if i is not None else None,
                        pool, idx, cache, cache_T, wf, prev, None)


def test_verify_validation(L):
    # sizes and dtypes first; a valid empty batch is a no-op whatever the pointers
    assert verify(L, dims(batch=0), io()) == 0
    assert verify(L, dims(batch=0), io(q=None), pool=None, idx=None) == 0
    assert verify(L, None, io()) == 1
    assert verify(L, dims(batch=-1), io()) == 2
    assert verify(L, dims(T=0), io()) == 2
    assert verify(L, dims(num_v_heads=3), io()) == 2                 # Hv % Hk != 0
    assert verify(L, dims(state_dtype=7), io()) == 3
    assert verify(L, dims(io_dtype=-1), io()) == 3
    assert verify(L, dims(d_k=96), io()) == 5
    assert verify(L, dims(d_v=120), io()) == 5
    assert verify(L, dims(d_v=512), io()) == 5
    assert verify(L, dims(T=gdn.GDN_MAX_T + 1), io(), cache_T=64) == 5
    assert verify(L, dims(batch=70000), io()) == 5
    # with rows to process (these all return before any launch)
    assert verify(L, dims(), None) == 1
    assert verify(L, dims(), io(q=None)) == 1
    assert verify(L, dims(), io(dt_bias=None)) == 1
    assert verify(L, dims(), io(), pool=None) == 1
    assert verify(L, dims(), io(), idx=None) == 1
    assert verify(L, dims(), io(), cache=None, prev=A16 * 12) == 1   # fused commit needs a cache
    assert verify(L, dims(), io(), cache_T=3) == 2                   # cache shallower than T
    assert verify(L, dims(), io(q=A16 + 8)) == 4
    assert verify(L, dims(), io(o=A16 * 8 + 4)) == 4
    assert verify(L, dims(), io(), pool=A16 * 9 + 4) == 4
    assert verify(L, dims(), io(), cache=A16 * 11 + 2) == 4
    assert verify(L, dims(), io(a=A16 * 4 + 1)) == 4
    assert verify(L, dims(io_dtype=gdn.GDN_DTYPE_F32), io(a=A16 * 4 + 2)) == 4
    assert verify(L, dims(), io(A_log=A16 * 6 + 2)) == 4
    assert verify(L, dims(), io(), idx=A16 * 10 + 2) == 4
    assert verify(L, dims(), io(), prev=A16 * 12 + 1) == 4


def test_decode_validation(L):
    def dec(d, i, pool=A16 * 9, idx=A16 * 10):
        return L.gdn_decode(ctypes.byref(d), ctypes.byref(i), pool, idx, None)
    assert dec(dims(batch=0, T=1), io()) == 0
    assert dec(dims(batch=0, T=2), io()) == 2                        # decode is one token
    assert dec(dims(T=1), io(), idx=None) == 1
    assert dec(dims(T=1), io(v=A16 * 3 + 8)) == 4
    assert dec(dims(batch=0, T=1, d_k=48), io()) == 5


def test_commit_validation(L):
    def com(d, cache=A16, cache_T=4, idx=A16 * 2, acc=A16 * 3, pool=A16 * 4):
        return L.gdn_commit(ctypes.byref(d), cache, cache_T, idx, acc, pool, None)
    assert com(dims(batch=0)) == 0
    assert com(dims(batch=0), cache=None) == 0
    assert com(dims(batch=0), cache_T=0) == 2
    assert com(dims(), cache=None) == 1
    assert com(dims(), acc=None) == 1
    assert com(dims(), cache_T=0) == 2
    assert com(dims(), pool=A16 * 4 + 8) == 4
    assert com(dims(), acc=A16 * 3 + 2) == 4
    assert com(dims(batch=0, d_v=8)) == 5


def test_verify_gated_validation(L):
    def vg(d, gate="ok", i=None, pool=A16 * 9, idx=A16 * 10, cache=None, cache_T=0):
        i = io() if i is None else i
        g = gdn.GdnOutGate(A16 * 20, A16 * 21, 1e-6) if gate == "ok" else gate
        return L.gdn_verify_gated(ctypes.byref(d), ctypes.byref(i), ctypes.byref(g) if g is not None else None,
                                  pool, idx, cache, cache_T, 0, None, None)
    assert vg(dims(batch=0)) == 0
    assert vg(dims(), gate=None) == 1
    assert vg(dims(), gate=gdn.GdnOutGate(None, A16 * 21, 1e-6)) == 1
    assert vg(dims(), gate=gdn.GdnOutGate(A16 * 20, None, 1e-6)) == 1
    assert vg(dims(batch=0), gate=gdn.GdnOutGate(A16 * 20, A16 * 21, -1.0)) == 2
    assert vg(dims(), gate=gdn.GdnOutGate(A16 * 20 + 8, A16 * 21, 1e-6)) == 4
    assert vg(dims(), gate=gdn.GdnOutGate(A16 * 20, A16 * 21 + 4, 1e-6)) == 4
    assert vg(dims(batch=0, d_k=128, d_v=256)) == 5        # a head's d_v must fit one workgroup
    assert vg(dims(), i=io(q=None)) == 1


def prefill_ws(L, d, n):
    out = ctypes.c_size_t(0)
    st = L.gdn_prefill_workspace_bytes(ctypes.byref(d), n, ctypes.byref(out))
    return st, out.value


def test_prefill_workspace_size(L):
    """Per 16-token chunk (floor(N/16) + B of them) a 5376-byte record per v-head and a
    4096-byte one per k-head; then, per segment of the chunk chain (floor(N / 2^s) + B of
    them, 2^s tokens each), a 4-byte table entry (the table padded to 256 bytes) and per
    v-head a slot of a 128 x d_v fp32 state and a 128 x 128 bf16 map. The segment length:
    longer than N (one segment per sequence) when the chains (2 B Hv d_v/16 waves) number
    at least 512, else the power of two >= 256 nearest above N Hv (d_v/16) 2 / 2048."""
    def shift(B, Hv, dv, N):
        whole = 8
        while (1 << whole) <= N:
            whole += 1
        if B * Hv * (dv // 16) * 2 >= 512:
            return whole
        s_ = 8
        while (1 << s_) < N * Hv * (dv // 16) * 2 // 2048:
            s_ += 1
        return min(s_, whole)

    def size(B, Hk, Hv, dv, N):
        segs = (N >> shift(B, Hv, dv, N)) + B
        table = (segs * 4 + 255) // 256 * 256
        return (N // 16 + B) * (Hv * 5376 + Hk * 4096) + table + segs * Hv * (128 * dv * 4 + 128 * 128 * 2)

    assert shift(4, 4, 128, 64) == 8 and shift(3, 32, 64, 16399) == 15 and shift(1, 8, 128, 16384) == 10
    assert prefill_ws(L, dims(batch=4, num_v_heads=4), 64) == (0, size(4, 2, 4, 128, 64))
    assert prefill_ws(L, dims(batch=4, num_v_heads=4), 64)[1] == (
        (4 + 4) * (4 * 5376 + 2 * 4096) + 256 + 4 * 4 * (128 * 128 * 4 + 128 * 128 * 2))
    assert prefill_ws(L, dims(batch=3, num_v_heads=32, d_v=64), 16384 + 15) == (0, size(3, 2, 32, 64, 16399))
    assert prefill_ws(L, dims(batch=1, num_k_heads=4, num_v_heads=8), 16384) == (0, size(1, 4, 8, 128, 16384))
    assert prefill_ws(L, dims(batch=1, num_k_heads=4, num_v_heads=8), 16384)[1] == (
        (1024 + 1) * (8 * 5376 + 4 * 4096) + 256 + 17 * 8 * (128 * 128 * 4 + 128 * 128 * 2))
    assert prefill_ws(L, dims(batch=0), 0) == (0, 0)
    assert prefill_ws(L, dims(), -1)[0] == 2
    assert prefill_ws(L, dims(d_k=64), 16)[0] == 5
    assert prefill_ws(L, dims(io_dtype=gdn.GDN_DTYPE_F32), 16)[0] == 5
    assert L.gdn_prefill_workspace_bytes(ctypes.byref(dims()), 16, None) == 1


def test_prefill_validation(L):
    need = prefill_ws(L, dims(), 64)[1]

    def pf(d, i=None, pool=A16 * 9, idx=A16 * 10, cu=A16 * 11, fresh=None, n=64, ws=A16 * 20, wsb=need):
        i = io() if i is None else i
        return L.gdn_prefill(ctypes.byref(d), ctypes.byref(i), pool, idx, cu, fresh, n, ws, wsb, None)
    assert pf(dims(batch=0), ws=None, wsb=0) == 0
    assert pf(dims(batch=0, T=0)) == 0                       # T is not used
    assert pf(dims(io_dtype=gdn.GDN_DTYPE_F32)) == 5         # the matrix-core path takes bf16 tokens
    assert pf(dims(batch=0, d_k=64)) == 5
    assert pf(dims(batch=0, d_v=48)) == 5                    # d_v a multiple of 32
    assert pf(dims(), n=-1) == 2
    assert pf(dims(), n=1 << 24) == 5                        # 32-bit offsets: N * Hv * d_v < 2^30
    assert pf(dims(), wsb=need - 1) == 2                     # workspace too small
    assert pf(dims(), n=80) == 2                             # ... for more tokens
    assert pf(dims(), ws=None) == 1
    assert pf(dims(), ws=A16 * 20 + 128) == 4                # 256-byte aligned
    assert pf(dims(), cu=None) == 1
    assert pf(dims(), i=io(v=None)) == 1
    assert pf(dims(), cu=A16 * 11 + 2) == 4
    assert pf(dims(), fresh=A16 * 12 + 1) == 4
    assert pf(dims(), i=io(q=A16 + 8)) == 4


def test_prefill_noalloc_validation(L):
    """The fixed-array prefill refuses, before touching a GPU, a call whose workspace
    exceeds the array (GDN_ERR_TOO_LARGE), and checks sizes and pointers like gdn_prefill."""
    def pf(d, i=None, pool=A16 * 9, idx=A16 * 10, cu=A16 * 11, fresh=None, n=64):
        i = io() if i is None else i
        return L.gdn_prefill_noalloc(ctypes.byref(d), ctypes.byref(i), pool, idx, cu, fresh, n, None)
    big = dims(batch=1, num_k_heads=4, num_v_heads=8)
    fits = max(n for n in range(0, 40000, 16) if prefill_ws(L, big, n)[1] <= gdn.GDN_PREFILL_NOALLOC_BYTES)
    assert 33000 <= fits <= 35000                             # about 34,000 tokens at Hk = 4, Hv = 8, d_v = 128
    assert pf(big, n=fits + 16) == 7 and pf(dims(batch=0), n=1 << 19) == 7
    assert pf(dims(batch=0)) == 0
    assert pf(dims(io_dtype=gdn.GDN_DTYPE_F32)) == 5
    assert pf(dims(), n=-1) == 2
    assert pf(dims(), cu=None) == 1
    assert pf(dims(), i=io(k=None)) == 1
    assert pf(dims(), i=io(o=A16 + 8)) == 4
    assert pf(dims(), fresh=A16 * 12 + 2) == 4


def tokens(**kw):
    base = dict(k=A16 * 13, v=A16 * 14, a=A16 * 15, b=A16 * 16, T_src=4)
    base.update(kw)
    return gdn.GdnTokens(**base)


def test_verify_replay_validation(L):
    def vr(d, i=None, rep=None, rlen=A16 * 17, pool=A16 * 9, idx=A16 * 10, commit=1):
        i = io() if i is None else i
        rep = tokens() if rep is None else rep
        return L.gdn_verify_replay(ctypes.byref(d), ctypes.byref(i), pool, idx,
                                   ctypes.byref(rep) if rep != "null" else None, rlen, commit, None)
    assert vr(dims(batch=0)) == 0
    assert vr(dims(batch=0), rep=tokens(T_src=0)) == 2
    assert vr(dims(batch=0, T=12), rep=tokens(T_src=5)) == 5          # T + T_src > GDN_MAX_T
    assert vr(dims(), rep="null") == 1
    assert vr(dims(), rep=tokens(v=None)) == 1
    assert vr(dims(), rlen=None) == 1
    assert vr(dims(), i=io(o=None)) == 1
    assert vr(dims(), rep=tokens(k=A16 * 13 + 8)) == 4
    assert vr(dims(), rep=tokens(a=A16 * 15 + 1)) == 4
    assert vr(dims(), rlen=A16 * 17 + 2) == 4
    assert vr(dims(), pool=A16 * 9 + 4) == 4


def test_commit_replay_validation(L):
    def cr(d, rep=None, rlen=A16 * 17, pool=A16 * 9, idx=A16 * 10, A=A16 * 6, dt=A16 * 7):
        rep = tokens() if rep is None else rep
        return L.gdn_commit_replay(ctypes.byref(d), A, dt, pool, idx, ctypes.byref(rep), rlen, None)
    assert cr(dims(batch=0)) == 0
    assert cr(dims(batch=0), rep=tokens(T_src=0)) == 2
    assert cr(dims(batch=0), rep=tokens(T_src=gdn.GDN_MAX_T + 1)) == 5
    assert cr(dims(), A=None) == 1
    assert cr(dims(), rlen=None) == 1
    assert cr(dims(), rep=tokens(b=None)) == 1
    assert cr(dims(), rep=tokens(v=A16 * 14 + 4)) == 4
    assert cr(dims(), dt=A16 * 7 + 2) == 4
    assert cr(dims(d_k=48)) == 5


def cdims(**kw):
    base = dict(batch=4, T=4, channels=2048, width=4, pool_slots=8, dtype=gdn.GDN_DTYPE_BF16, activation=1)
    base.update(kw)
    return gdn.GdnConvDims(**base)


def test_conv_update_validation(L):
    def cu(d, x=A16, w=A16 * 2, b=A16 * 3, pool=A16 * 4, idx=A16 * 5, px=None, T_prev=0, plen=None,
           y=A16 * 6, wb=0):
        return L.gdn_conv_update(ctypes.byref(d), x, w, b, pool, idx, px, T_prev, plen, y, wb, None)
    assert cu(cdims(batch=0)) == 0
    assert cu(cdims(batch=0), x=None, y=None) == 0
    assert L.gdn_conv_update(None, A16, A16, A16, A16, A16, None, 0, None, A16, 0, None) == 1
    assert cu(cdims(batch=-1)) == 2
    assert cu(cdims(T=0)) == 2
    assert cu(cdims(width=1)) == 2
    assert cu(cdims(batch=0), px=A16 * 7, T_prev=0, plen=A16 * 8) == 2    # prev_x needs 1 <= T_prev
    assert cu(cdims(dtype=7)) == 3
    assert cu(cdims(activation=2)) == 5
    assert cu(cdims(channels=2044)) == 5                                  # not a multiple of 8 bf16
    assert cu(cdims(width=gdn.GDN_CONV_MAX_WIDTH + 1)) == 5
    assert cu(cdims(T=gdn.GDN_MAX_T + 1)) == 5
    assert cu(cdims(batch=65536, pool_slots=70000)) == 5
    assert cu(cdims(), x=None) == 1
    assert cu(cdims(), w=None) == 1
    assert cu(cdims(), y=None) == 1
    assert cu(cdims(), px=A16 * 7, T_prev=4, plen=None) == 1
    assert cu(cdims(), x=A16 + 8) == 4
    assert cu(cdims(), b=A16 * 3 + 4) == 4
    assert cu(cdims(), pool=A16 * 4 + 2) == 4
    assert cu(cdims(), px=A16 * 7 + 8, T_prev=4, plen=A16 * 8) == 4
    assert cu(cdims(), px=A16 * 7, T_prev=4, plen=A16 * 8 + 2) == 4


def test_conv_commit_validation(L):
    def cc(d, x=A16, pool=A16 * 4, idx=A16 * 5, acc=A16 * 6):
        return L.gdn_conv_commit(ctypes.byref(d), x, pool, idx, acc, None)
    assert cc(cdims(batch=0)) == 0
    assert cc(cdims(batch=0), acc=None) == 0
    assert cc(cdims(T=0)) == 2
    assert cc(cdims(), acc=None) == 1
    assert cc(cdims(), x=None) == 1
    assert cc(cdims(), x=A16 + 4) == 4
    assert cc(cdims(), acc=A16 * 6 + 1) == 4
    assert cc(cdims(width=9)) == 5


STREAM_HEADER = os.path.join(ROOT, "include", "gdn_stream.h")
STREAM_LIB = os.path.join(os.path.dirname(gdn.LIB_PATH), "libgdn_stream.so")


def test_stream_library_exports_and_validates():
    """The measurement library (a streaming copy bench.py times as the practical HBM
    ceiling) loads, exports what its header declares, and refuses bad arguments before any
    launch."""
    import subprocess
    if not os.path.exists(STREAM_LIB):
        pytest.fail("libgdn_stream.so is not built (run __graft_entry__.build())")
    declared = set(re.findall(r'visibility\("default"\)\)\)\s+[\w\s\*]+?\b(gdn_\w+)\s*\(',
                              open(STREAM_HEADER).read()))
    assert declared == {"gdn_stream_copy", "gdn_stream_wait"}
    out = subprocess.run(["nm", "-D", "--defined-only", STREAM_LIB], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert {s for s in syms if not s.startswith("_")} == declared
    S = ctypes.CDLL(STREAM_LIB)
    S.gdn_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_int32] * 4 + [
        ctypes.c_void_p]
    S.gdn_stream_copy.restype = ctypes.c_int32
    S.gdn_stream_wait.argtypes = [ctypes.c_int64, ctypes.c_void_p]
    S.gdn_stream_wait.restype = ctypes.c_int32
    blk = 256 * 2 * 16
    assert S.gdn_stream_copy(A16, A16 * 2, 0, 4, 256, 2, 7, None) == 0        # nothing to do
    assert S.gdn_stream_copy(A16, A16 * 2, -blk, 4, 256, 2, 7, None) == 2
    assert S.gdn_stream_copy(A16, A16 * 2, blk + 16, 4, 256, 2, 7, None) == 2  # not whole blocks
    assert S.gdn_stream_copy(A16, A16 * 2, blk, 0, 256, 2, 7, None) == 2
    assert S.gdn_stream_copy(A16, A16 * 2, blk, 17, 256, 2, 7, None) == 2
    assert S.gdn_stream_copy(A16, A16 * 2, blk, 4, 128, 2, 7, None) == 2      # threads 64 or 256
    assert S.gdn_stream_copy(A16, A16 * 2, blk, 4, 256, 4, 7, None) == 2      # chunks 1, 2 or 8
    assert S.gdn_stream_copy(A16, A16 * 2, blk, 4, 256, 2, 8, None) == 2
    assert S.gdn_stream_copy(None, A16 * 2, blk, 4, 256, 2, 7, None) == 1
    assert S.gdn_stream_copy(A16 + 4, A16 * 2, blk, 4, 256, 2, 7, None) == 4
    assert S.gdn_stream_wait(-1, None) == 2 and S.gdn_stream_wait(10 ** 8, None) == 2


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 1, 16)
    with pytest.raises(ValueError):
        gdn.gdn_verify(x, x, x, torch.zeros(1, 1, 1), torch.zeros(1, 1, 1), torch.zeros(1), torch.zeros(1), x,
                       torch.zeros(1, 1, 16, 16), torch.zeros(1, dtype=torch.int32))
