"""The kernels read some LDS operands (the gfx950 transposing reads
ds_read_b64_tr_b16) in inline assembly and wait for them later, so that the
reads overlap the MFMA work before them.  The compiler takes an inline-asm
result as written when the instruction issues; if it copies, spills or
overwrites such a register before the data has landed, the kernel computes
with stale values (a development form of the prefill kernel did exactly
that: its carried V operands were spilled to scratch right after the reads
were issued).  This test compiles the attention library for gfx950 on the
CPU, walks every kernel's code in order and checks that no register written
by an outstanding LDS read is read or written before an s_waitcnt that
covers it (lgkmcnt(N) retires all but the N most recent LDS/scalar-memory
operations).  The walk is linear: a wait anywhere before a use in the text
counts, which is how the kernels are written (each read and its wait sit in
one straight-line page step)."""
import os
import re
import shutil
import subprocess

import pytest

from paged_gqa_decode_attn_amd import _build

SRC = os.path.join(_build.PKG, "csrc", "pgqa.hip")

pytestmark = pytest.mark.skipif(shutil.which(_build.HIPCC) is None and not os.path.exists(_build.HIPCC),
                                reason="hipcc not available")


def device_asm(tmp_path):
    out = str(tmp_path / "pgqa_gfx950.s")
    flags = [f for f in _build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [_build.HIPCC] + flags + ["-I", _build.INCLUDE, "--cuda-device-only", "-S", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().split("\n")


def vregs(text):
    regs = set()
    for a, b in re.findall(r"v\[(\d+):(\d+)\]", text):
        regs.update(range(int(a), int(b) + 1))
    regs.update(int(a) for a in re.findall(r"\bv(\d+)\b", text))
    return regs


def early_uses(lines):
    """(kernel, line, instruction) for every touch of a register that an
    outstanding LDS read still has to write, and the number of transposing
    reads seen."""
    found, reads = [], 0
    queue = []  # outstanding LGKM operations, oldest first: (opcode, registers they write)
    kernel = ""
    for n, line in enumerate(lines, 1):
        t = line.split(";")[0].strip()
        if re.match(r"^_Z\S+:$", t):
            kernel, queue = t[:-1], []
            continue
        if not t or t.startswith("."):
            continue
        op, _, rest = t.partition(" ")
        if op.startswith("s_waitcnt"):
            m = re.search(r"lgkmcnt\((\d+)\)", t)
            if m:
                keep = int(m.group(1))
                queue = queue[len(queue) - keep:] if keep else []
            continue
        parts = [p.strip() for p in rest.split(",")] if rest else []
        pending = set().union(*[r for _, r in queue]) if queue else set()
        if pending and parts:
            store = op.startswith(("global_store", "buffer_store", "ds_write", "scratch_store", "flat_store"))
            touched = set().union(*[vregs(p) for p in parts]) if store else \
                vregs(parts[0]) | set().union(*[vregs(p) for p in parts[1:]] or [set()])
            if touched & pending:
                found.append((kernel, n, t))
        if op.startswith(("ds_", "s_load", "s_buffer_load")):
            writes = vregs(parts[0]) if op.startswith(("ds_read", "ds_load")) and parts else set()
            queue.append((op, writes))
            reads += op == "ds_read_b64_tr_b16"
    return found, reads


def test_no_lds_result_is_used_before_its_wait(tmp_path):
    found, reads = early_uses(device_asm(tmp_path))
    assert reads > 0, "no transposing LDS reads found: the check would be vacuous"
    assert not found, "LDS results touched before their wait:\n" + "\n".join(
        f"{k}:{n}: {t}" for k, n, t in found[:10])


def test_the_check_sees_a_spilled_read():
    """The walk flags a result copied out before its wait, and accepts the
    same code with the wait first."""
    bad = ["_Zk:", "ds_read_b64_tr_b16 v[4:5], v21 offset:512", "scratch_store_dwordx2 off, v[4:5], off",
           "s_waitcnt lgkmcnt(0)"]
    good = ["_Zk:", "ds_read_b64_tr_b16 v[4:5], v21 offset:512", "ds_read_b64_tr_b16 v[6:7], v21",
            "s_waitcnt lgkmcnt(1)", "v_mov_b32 v9, v4", "s_waitcnt lgkmcnt(0)", "v_mov_b32 v8, v6"]
    assert len(early_uses(bad)[0]) == 1
    assert early_uses(good)[0] == []
