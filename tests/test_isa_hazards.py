"""CPU: the gfx950 assembly of every library source, scanned for one hazard
the compiler cannot guard against.

The pipelined GEMMs issue their direct-to-LDS loads (and some stores) from
inline assembly.  A VMEM instruction that reads an SGPR written by a VALU
instruction (v_readlane, v_readfirstlane, v_cmp with a scalar destination,
...) needs five wait states in between; the compiler inserts them for its own
instructions but cannot see into inline assembly, and when it restores a
spilled scalar with v_readlane right before such a load, the load reads a
stale value (this happened once: a load's scalar offset came out of a VGPR
lane in the previous instruction).  The device code is compiled to assembly
here with the library's own flags and every inline-assembly VMEM instruction
is checked against the instructions before it."""
import concurrent.futures as cf
import os
import re
import subprocess
import tempfile

import pytest

from dora_adapter_amd import build as B

WAIT_STATES = 5
VMEM = re.compile(r"^(buffer_|global_|scratch_|flat_)")
SREG = re.compile(r"\bs\[(\d+):(\d+)\]|\bs(\d+)\b|\b(vcc)\b")


def _sregs(text):
    out = set()
    for a, b, c, v in SREG.findall(text):
        if v:
            out.update(("vcc_lo", "vcc_hi"))
        elif c:
            out.add(f"s{c}")
        else:
            out.update(f"s{i}" for i in range(int(a), int(b) + 1))
    return out


def _instructions(asm):
    """(text, in inline asm) for every instruction, labels and comments dropped."""
    inside = False
    for raw in asm.splitlines():
        line = raw.strip()
        if line.startswith(";;#ASMSTART"):
            inside = True
            continue
        if line.startswith(";;#ASMEND"):
            inside = False
            continue
        line = line.split(";")[0].strip()
        if not line or line.endswith(":") or line.startswith("."):
            continue
        yield line, inside


def hazards(asm):
    """Inline-asm VMEM instructions that read an SGPR a VALU instruction wrote
    fewer than WAIT_STATES wait states earlier."""
    found = []
    window = []  # (wait states taken, sgprs written by VALU)
    for text, inline in _instructions(asm):
        op, _, args = text.partition(" ")
        if inline and VMEM.match(op):
            reads = _sregs(args)
            taken = 0
            for states, written in reversed(window):
                if taken >= WAIT_STATES:
                    break
                if written & reads:
                    found.append(text)
                    break
                taken += states
        if op.startswith("s_nop"):
            n = int(args.strip() or "0", 0)
            states, written = n + 1, set()
        elif op.startswith("v_"):
            ops = [a.strip() for a in args.split(",")] if args else []
            # the destination; VOP3 forms with a scalar carry / condition
            # destination name it second
            wide = any(k in op for k in ("_co_", "div_scale", "mad_u64", "mad_i64"))
            dst = ops[:2] if wide else ops[:1]
            states, written = 1, _sregs(" ".join(dst))
        else:
            states, written = 1, set()
        window.append((states, written))
        window = window[-16:]
    return found


def test_scanner_finds_the_pattern():
    bad = """
        v_readlane_b32 s9, v220, 43
        ;;#ASMSTART
        buffer_load_dwordx4 v64, s[52:55], s9 offen offset:0 lds
        ;;#ASMEND
    """
    ok = """
        v_readlane_b32 s9, v220, 43
        ;;#ASMSTART
        s_nop 4
        buffer_load_dwordx4 v64, s[52:55], s9 offen offset:0 lds
        ;;#ASMEND
    """
    compiler_own = """
        v_readfirstlane_b32 s4, v1
        buffer_load_dword v2, v3, s[4:7], 0 offen
    """
    assert hazards(bad) and not hazards(ok) and not hazards(compiler_own)


def _device_asm(unit, out_dir):
    src, defines, name = unit
    out = os.path.join(out_dir, name + ".s")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [B.HIPCC, *B.COMMON, *defines, *lang, "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as fh:
        return name, fh.read()


@pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not available")
def test_library_assembly_has_no_inline_vmem_sgpr_hazard():
    units = [u for u in B.SOURCES if u[0].endswith(".hip")]
    with tempfile.TemporaryDirectory() as d, cf.ThreadPoolExecutor(min(8, len(units))) as ex:
        results = list(ex.map(lambda u: _device_asm(u, d), units))
    bad = {name: hazards(asm) for name, asm in results}
    assert all("buffer_load_dwordx4" in asm for name, asm in results if name.startswith("gemm_dma"))
    assert not any(bad.values()), {k: v[:3] for k, v in bad.items() if v}
