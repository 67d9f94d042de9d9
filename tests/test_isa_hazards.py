"""Inline-asm LDS reads in the HIP kernels must be retired before use.

The attention kernels read LDS with inline-asm ds_read_* instructions and
retire them with explicit s_waitcnt lgkmcnt(N).  The compiler does not know
these results arrive asynchronously, so if it ever moved or copied such a
register before its wait, the kernel would read stale data.  This test
compiles each kernel source for gfx950 to assembly (host-only, no GPU) and
scans every kernel in program order: a queue of in-flight LDS operations,
retired by s_waitcnt lgkmcnt(N) (LDS operations complete in order), and no
instruction may touch a VGPR written by an in-flight asm read.
"""

import os
import re
import shutil
import subprocess

import pytest

from block_sparse_attention_strided_amd import build as xbuild

CSRC = os.path.join(os.path.dirname(xbuild.__file__), "csrc")


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _operands(line):
    parts = line.split(None, 1)
    if len(parts) < 2:
        return parts[0], []
    return parts[0], [o.strip() for o in re.split(r",\s*", parts[1].split(";")[0])]


def scan_function(text):
    """Return a list of (line, message) hazards in one function's assembly."""
    hazards = []
    in_asm = False
    pending = []  # in issue order: set of destination VGPRs (asm reads) or None
    for i, raw in enumerate(text.split("\n")):
        line = raw.strip()
        if line.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if line.startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not line or line.startswith((".", ";")) or line.endswith(":"):
            continue
        op, ops = _operands(line)
        if op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", line)
            if m:
                n = int(m.group(1))
                pending = pending[len(pending) - n:] if 0 < n < len(pending) else ([] if n == 0 else pending)
            continue
        used = set()
        for o in ops[1:] if op.startswith("ds_") else ops:
            used |= _vregs(o)
        for dst, at in pending:
            if dst and used & dst:
                hazards.append((i, "v%s of the asm LDS read at line %d used before its wait: %s"
                                % (sorted(used & dst), at, line)))
        if op.startswith("ds_"):
            dst = _vregs(ops[0]) if (in_asm and op.startswith("ds_read") and ops) else None
            pending.append((dst, i))
        elif op.startswith(("s_memtime", "s_load", "s_buffer_load")):
            pending.append((None, i))
    return hazards


def scan_assembly(asm):
    out = {}
    for m in re.finditer(r"^(_Z\S+):(?:[ \t]*;.*)?$", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        out[m.group(1)] = scan_function(asm[m.end():end])
    return out


def test_scanner_catches_a_planted_copy():
    asm = """_Zkernel:
\t;;#ASMSTART
\tds_read_b128 v[4:7], v1 offset:16
\t;;#ASMEND
\tv_mov_b32_e32 v20, v5
\t;;#ASMSTART
\ts_waitcnt lgkmcnt(0)
\t;;#ASMEND
\tv_mov_b32_e32 v21, v6
.Lfunc_end0:
"""
    res = scan_assembly(asm)
    assert len(res["_Zkernel"]) == 1 and "v[5]" in res["_Zkernel"][0][1]


def test_scanner_respects_partial_waits():
    asm = """_Zkernel:
\t;;#ASMSTART
\tds_read_b128 v[4:7], v1
\t;;#ASMEND
\t;;#ASMSTART
\tds_read_b128 v[8:11], v1 offset:64
\t;;#ASMEND
\t;;#ASMSTART
\ts_waitcnt lgkmcnt(1)
\t;;#ASMEND
\tv_mov_b32_e32 v20, v5
\tv_mov_b32_e32 v21, v9
.Lfunc_end0:
"""
    res = scan_assembly(asm)
    assert len(res["_Zkernel"]) == 1 and "v[9]" in res["_Zkernel"][0][1]


@pytest.mark.skipif(shutil.which(xbuild._hipcc()) is None and not os.path.exists(xbuild._hipcc()),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", ["attention.hip", "estimate.hip"])
def test_no_asm_lds_result_used_before_its_wait(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [xbuild._hipcc(), "-x", "hip", "-S", "--cuda-device-only", os.path.join(CSRC, src), "-o", str(out)]
    cmd += [f for f in xbuild.FLAGS if f != "-fPIC"]
    subprocess.run(cmd, check=True, capture_output=True)
    res = scan_assembly(out.read_text())
    assert res, "no kernels found in the assembly"
    bad = {k: v for k, v in res.items() if v}
    assert not bad, "\n".join("%s: %s" % (k[:60], msg) for k, v in bad.items() for _, msg in v[:5])
