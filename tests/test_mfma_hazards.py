"""The prefill kernels never feed one matrix-core product into a product of another shape
through its accumulator operand (srcC).

AMD's CDNA3 and CDNA4 instruction-set references (the MFMA dependency-resolution rules:
required independent instructions between dependent matrix-core instructions) leave the
ordering of such dependencies to software: the hardware forwards an accumulator from one
product to the next only for chains of the same instruction, and a product of another
shape or opcode that reads it as srcC needs independent instructions in between, more the
more passes the first product takes. A build of the chunk chain in which the compiler had
scheduled a v_mfma_f32_16x16x32_bf16 reading the accumulator of a
v_mfma_f32_16x16x16_bf16 a few instructions earlier gave wrong prefill outputs (a term of U
lost for some chunk counts). The kernels therefore combine products of different shapes
through vector adds only, and this test compiles the prefill source to gfx950 assembly with
the library's flags (and with accumulation registers) and requires that no such dependency
exists at all, whatever the number of instructions in between: no threshold from the
tables is needed.
"""
import os
import re
import subprocess

import pytest

from linear_attention_speculative_gdn_amd import _build

SRC = os.path.join(_build.CSRC, "gdn_prefill.hip")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok) or re.match(r"v(\d+)$", tok)
    if not m:
        return set()
    lo = int(m.group(1))
    hi = int(m.group(2)) if m.lastindex == 2 else lo
    return set(range(lo, hi + 1))


def cross_shape_srcc(asm: str):
    """(wait states, writer, reader line) for every MFMA whose srcC register was last
    written by an MFMA of another opcode. Wait states count the instructions in between,
    s_nop N counting N + 1; labels do not reset the tracking (fall-through order)."""
    last = {}  # vgpr -> (opcode, position)
    pos = 0
    found = []
    for raw in asm.splitlines():
        ln = raw.split(";")[0].strip()
        if not ln or ln.startswith(".") or ln.endswith(":"):
            if re.match(r"^_Z\w*:", ln):
                last.clear()  # a new function
            continue
        op, _, rest = ln.partition(" ")
        if op == "s_nop":
            pos += int(rest.strip(), 0) + 1
            continue
        args = [a.strip() for a in rest.split(",")] if rest else []
        if op.startswith("v_mfma") and len(args) >= 4:
            writers = {last[r] for r in _regs(args[3]) if r in last}
            for wop, wpos in writers:
                if wop != op:
                    found.append((pos - wpos - 1, wop, ln))
            for r in _regs(args[0]):
                last[r] = (op, pos)
        elif args:
            for r in _regs(args[0]):
                last.pop(r, None)
        pos += 1
    return found


def test_scanner_flags_a_short_cross_shape_chain():
    bad = """
_Zk:
  v_mfma_f32_16x16x16_bf16 v[4:7], v[0:1], v[2:3], 0
  s_nop 2
  v_mfma_f32_16x16x32_bf16 v[8:11], v[12:15], v[16:19], v[4:7]
"""
    ok = bad.replace("s_nop 2", "s_nop 4")
    same = bad.replace("v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16").replace("v[12:15], v[16:19]", "v[0:1], v[2:3]")
    assert [f[0] for f in cross_shape_srcc(bad)] == [3]
    assert [f[0] for f in cross_shape_srcc(ok)] == [5]
    assert cross_shape_srcc(same) == []          # same opcode: the chained form is not checked
    partial = bad.replace("  s_nop 2\n", "  v_mov_b32 v4, 0\n")
    assert [f[0] for f in cross_shape_srcc(partial)] == [1]   # v5..v7 still hold the product
    reset = bad.replace("  s_nop 2\n", "".join(f"  v_mov_b32 v{r}, 0\n" for r in range(4, 8)))
    assert cross_shape_srcc(reset) == []         # srcC rewritten by vector ops in between


@pytest.mark.parametrize("form", ["vgpr", "agpr"])
def test_prefill_has_no_cross_shape_srcc_dependency(tmp_path, form):
    flags = [f for f in _build.HIPCC_FLAGS if f not in ("-shared",)]
    if form == "agpr":
        flags = [f for f in flags if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form")]
    out = tmp_path / "prefill.s"
    cmd = [_build.hipcc(), *flags, "--cuda-device-only", "-S", "-o", str(out), SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    asm = out.read_text()
    assert "v_mfma_f32_16x16x32_bf16" in asm and "v_mfma_f32_16x16x16_bf16" in asm
    found = cross_shape_srcc(asm)
    assert not found, "\n".join(f"{w} wait states after {op}: {ln}" for w, op, ln in found)
