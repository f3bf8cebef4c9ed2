"""Post-build checks of the gfx950 machine code: wide-store data hazards
(run by the build) and the kernels' resource metadata (LDS, VGPRs).

A vector-memory store of more than 64 bits of data (dwordx3 / dwordx4) reads
its data VGPRs after it issues, so a VALU instruction may overwrite those
VGPRs only after some wait states (LLVM's gfx950 hazard model inserts two).
LLVM waives the wait states for buffer stores whose scalar offset operand is
an SGPR, and a build of the step kernel in which the next instruction after
a commit store overwrote that store's data (scalar row offset, zero wait
states) wrote wrong values for exactly the rows of that store.  The kernels
now pass store offsets through the vector operand, which the hazard model
covers; this check keeps any later build from reintroducing the pattern: it
disassembles the device code of every object file and fails if a VALU
instruction writes a data VGPR of a >64-bit store within two wait states of
it, whatever the store's offset operands.

    python -m state_space_recurrence_amd.isa_check [object files...]
"""
from __future__ import annotations

import glob
import os
import re
import subprocess
import sys
import tempfile

LLVM = "/opt/rocm/llvm/bin"
WAIT_STATES = 2   # required between a >64-bit store and a VALU write of its data

_WIDE_STORE = re.compile(r"^(buffer|global|flat|scratch)_store_(dwordx3|dwordx4|b96|b128|format_xyz|format_xyzw)\b")
_VREG = re.compile(r"^v\[(\d+):(\d+)\]$|^v(\d+)$")


def _vregs(tok: str) -> set:
    m = _VREG.match(tok.strip())
    if not m:
        return set()
    if m.group(1) is not None:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    return {int(m.group(3))}


def _instructions(text: str):
    """(function, line number, instruction text) in program order.  Accepts
    compiler assembly (';' comments, '.L' labels) and llvm-objdump output
    ('//' comments, '<symbol>:' headers)."""
    fn = None
    for n, line in enumerate(text.splitlines(), 1):
        head = re.match(r"^[0-9a-fA-F]+ <(\S+)>:\s*$", line)
        if head:
            fn = head.group(1)
            continue
        s = line.split("//")[0].split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            if not s.startswith(".L"):
                fn = s[:-1]
            continue
        if s.startswith("."):
            continue
        yield fn, n, s


def scan(text: str, wait_states: int = WAIT_STATES):
    """Hazards in one disassembly: list of (function, line, store, offender)."""
    insts = list(_instructions(text))
    hits = []
    for i, (fn, n, s) in enumerate(insts):
        m = _WIDE_STORE.match(s)
        if not m:
            continue
        ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
        data = ops[0] if m.group(1) in ("buffer", "scratch") else ops[1]
        dregs = _vregs(data)
        ws = 0
        for _, _, nxt in insts[i + 1:i + 1 + wait_states]:
            op = nxt.split()[0]
            parts = nxt.split(None, 1)
            if op.startswith("v_") and len(parts) > 1 and _vregs(parts[1].split(",")[0]) & dregs:
                hits.append((fn, n, s, nxt))
                break
            ws += int(parts[1], 0) + 1 if op == "s_nop" else 1
            if ws >= wait_states:
                break
    return hits


def _device_object(obj: str, td: str, arch: str) -> str:
    """Extract the gfx950 code object embedded in a hipcc object file."""
    fb, co = os.path.join(td, "fatbin"), os.path.join(td, "dev.co")
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fb}", obj, os.path.join(td, "host.o")],
                   check=True, capture_output=True)
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fb}",
                    f"--targets=hipv4-amdgcn-amd-amdhsa--{arch}", f"--output={co}"],
                   check=True, capture_output=True)
    return co


def disassemble(obj: str, arch: str = "gfx950") -> str:
    """Device-code disassembly of a hipcc object file."""
    with tempfile.TemporaryDirectory() as td:
        co = _device_object(obj, td, arch)
        return subprocess.run([f"{LLVM}/llvm-objdump", "-d", f"--mcpu={arch}", co], check=True,
                              capture_output=True, text=True).stdout


def kernel_resources(obj: str, arch: str = "gfx950") -> dict:
    """Per-kernel resources from the code object's metadata note:
    {symbol: {"lds": bytes, "vgpr": count, "scratch": bytes}}."""
    import yaml
    with tempfile.TemporaryDirectory() as td:
        co = _device_object(obj, td, arch)
        notes = subprocess.run([f"{LLVM}/llvm-readelf", "--notes", co], check=True, capture_output=True,
                               text=True).stdout
    start = notes.index("---")
    meta = yaml.safe_load(notes[start:notes.index("...", start) + 3])
    return {k[".name"]: {"lds": k[".group_segment_fixed_size"], "vgpr": k[".vgpr_count"],
                         "scratch": k[".private_segment_fixed_size"]} for k in meta["amdhsa.kernels"]}


def check_objects(objs, arch: str = "gfx950") -> int:
    """Raise if any object's device code has a wide-store data hazard;
    returns the number of wide stores seen (for the caller's log)."""
    bad, seen = [], 0
    for obj in objs:
        text = disassemble(obj, arch)
        seen += sum(1 for _, _, s in _instructions(text) if _WIDE_STORE.match(s))
        bad += [(os.path.basename(obj),) + h for h in scan(text)]
    if bad:
        lines = "\n".join(f"  {o}: {fn}: {s}  ->  {v}" for o, fn, _, s, v in bad[:20])
        raise RuntimeError(f"{len(bad)} wide-store data hazard(s) in the device code:\n{lines}")
    return seen


if __name__ == "__main__":
    objs = sys.argv[1:] or sorted(glob.glob(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                        "_build", "*.hip.o")))
    print(f"{check_objects(objs)} wide stores in {len(objs)} objects, no data hazards")
