"""The library's own device assembly (CPU only: hipcc -S of the sources, no GPU):
no 12- or 16-byte vector store may leave its data registers to be rewritten by
the very next vector instruction.

gfx950 needs one wait state between such a store and a write of its data
registers. The compiler inserts it only for buffer stores whose scalar offset
is not a register, so every buffer store here passes a literal zero scalar
offset; when a persistent kernel still passed the member's column offset there,
a move into a store's first data register right after the store changed the
layer_input it wrote in some lanes (seen as differences between identical calls
in the graph-replay test). This test rebuilds the assembly and checks both the
rule and its purpose."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from decode_mhc_pre_amd import build as B

WIDE_STORE = re.compile(r"^(buffer|global|flat)_store_dwordx[34]\s+(.*)$")
REG = re.compile(r"v\[(\d+):(\d+)\]|v(\d+)$")


def _regs(tok):
    m = REG.match(tok.strip())
    if not m:
        return set()
    if m.group(1):
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return {int(m.group(3))}


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "mhc.s")
        flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
        subprocess.run([B.HIPCC, *flags, "--offload-device-only", "-S", "-o", out, *B.SOURCES],
                       check=True, capture_output=True, timeout=600)
        with open(out) as f:
            return [ln.strip() for ln in f]


def _instructions(lines):
    for i, ln in enumerate(lines):
        if ln and not ln.startswith((";", ".")) and not ln.endswith(":"):
            yield i, ln


def test_wide_buffer_stores_have_no_scalar_offset_register(asm):
    bad = []
    for i, ln in _instructions(asm):
        m = WIDE_STORE.match(ln)
        if m and m.group(1) == "buffer":
            ops = [o.strip() for o in m.group(2).split(",")]
            # data, vaddr, rsrc, soffset [modifiers]
            soff = ops[3].split()[0]
            if re.match(r"^s\d+$|^s\[\d+:\d+\]$|^m0$|^vcc", soff):
                bad.append(ln)
    assert not bad, bad[:5]


def test_no_write_of_store_data_in_the_next_instruction(asm):
    ins = list(_instructions(asm))
    bad = []
    for n, (i, ln) in enumerate(ins[:-1]):
        m = WIDE_STORE.match(ln)
        if not m:
            continue
        ops = [o.strip() for o in m.group(2).split(",")]
        data = _regs(ops[0] if m.group(1) == "buffer" else ops[1])
        nxt = ins[n + 1][1]
        op = nxt.split()[0]
        if op.startswith("v_") and not op.startswith(("v_readlane", "v_readfirstlane", "v_cmp")):
            dst = _regs(nxt.split(None, 1)[1].split(",")[0])
            if dst & data and not op.startswith("v_mfma"):
                bad.append((ln, nxt))
    assert not bad, bad[:5]
