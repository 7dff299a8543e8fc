"""Check of the built gfx950 assembly for one hazard the compiler cannot see.

gfx950 needs two wait states between a vector instruction that writes an
SGPR pair (a compare or a carry-out) and a vector instruction that reads it
as a lane mask or carry-in.  The compiler inserts them before instructions it
emits, but not before inline asm, and several kernels read compare masks in
asm (bit pushes with add-with-carry, selects on a mask).  This module
compiles a source to assembly and reports every such read whose pair was
last written by a vector instruction fewer than two instructions earlier.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

from quantization_aware_amd import build

_PAIR = re.compile(r"s\[(\d+):(\d+)\]|\b(vcc)\b")
_FUNC = re.compile(r"^(_Z\S+):")
_NO_DEST = ("s_waitcnt", "s_nop", "s_cbranch", "s_branch", "s_barrier", "s_setprio", "s_endpgm", "s_sleep")


def _pairs(operands: str) -> list[str]:
    return ["vcc" if m.group(3) else f"s[{m.group(1)}:{m.group(2)}]" for m in _PAIR.finditer(operands)]


def close_mask_reads(asm: str, min_distance: int = 2) -> list[tuple[str, str, int]]:
    """(function, instruction, distance) for every v_cndmask / v_addc that reads an SGPR
    pair last written by a vector instruction fewer than min_distance instructions before."""
    found = []
    func = None
    hist: list[tuple[str, str | None]] = []  # (kind, pair written) per issued instruction slot
    for line in asm.split("\n"):
        m = _FUNC.match(line)
        if m:
            func, hist = m.group(1), []
            continue
        if func is None:
            continue
        t = line.strip()
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        ins = t.split()[0]
        ops = t[len(ins):].split(";")[0]
        pairs = _pairs(ops)
        if ins.startswith(("v_cndmask_b32", "v_addc_co_u32")) and pairs:
            src = pairs[-1]
            for d, (kind, wrote) in enumerate(reversed(hist)):
                if wrote == src:
                    if kind == "valu" and d < min_distance:
                        found.append((func, t, d))
                    break
        if ins.startswith("s_nop"):
            hist.extend([("nop", None)] * (int(t.split()[1], 0) + 1))
            continue
        if ins.startswith("s_"):
            wrote = pairs[0] if pairs and not ins.startswith(_NO_DEST) and re.match(r"\s*(s\[|vcc)", ops) else None
            hist.append(("salu", wrote))
            continue
        wrote = None
        if ins.startswith("v_cmp"):
            wrote = pairs[0] if "_e64" in ins and pairs else "vcc"
        elif ins.startswith(("v_addc_co_u32_e64", "v_add_co_u32_e64", "v_sub_co_u32_e64", "v_subb_co_u32_e64")):
            wrote = pairs[0] if pairs else None
        hist.append(("valu", wrote))
    return found


def compile_asm(source: str) -> str:
    """gfx950 device assembly of one source under the library's own flags."""
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "out.s")
        cmd = [build.hipcc_path(), *build.compile_flags(source), "--cuda-device-only", "-S",
               os.path.join(build.CSRC, source), "-o", out]
        subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        with open(out) as f:
            return f.read()
