"""Build libreplayssm.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m state_space_recurrence_amd.build [-v]

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 VALU forms are
disabled for device code (`-packed-fp32-ops`): the kernels are written with
scalar fp32 arithmetic and must not be lowered to v_pk_*_f32.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libreplayssm.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = os.environ.get("RSSM_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libreplayssm)")


# -ffp-contract=on: a*b+c is fused only inside one expression, never across
# statements, so the same source arithmetic compiles to the same roundings in
# every kernel that inlines it (results do not depend on the calling kernel).
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=on", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # matrix-core accumulators in ordinary VGPRs (no AGPR copies around each MFMA)
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-Wno-unused-command-line-argument"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + sorted(glob.glob(os.path.join(CSRC, "*.cpp")))
    objs, procs = [], []
    t0 = time.time()
    for src in srcs:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        objs.append(obj)
        lang = ["-x", "hip", f"--offload-arch={ARCH}"] if src.endswith(".hip") else [
            "-x", "hip", f"--offload-arch={ARCH}"]
        cmd = [cc, *COMMON, *lang, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            time.sleep(0.05)
    for cmd, p in procs:
        out = p.communicate()[0]
        out = "\n".join(l for l in out.splitlines()
                        if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
        if p.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
        if verbose and out.strip():
            print(out, flush=True)
    # refuse device code in which a VALU op overwrites the data of a wide
    # store before the store has read it (see isa_check)
    from . import isa_check
    nst = isa_check.check_objects([o for o in objs if o.endswith(".hip.o")], ARCH)
    if verbose:
        print(f"isa check: {nst} wide stores, no data hazards", flush=True)
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"], verbose)
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
