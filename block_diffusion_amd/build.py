"""Build libdbd.so (gfx950) in-tree with hipcc.

    python -m block_diffusion_amd.build

Every source is compiled to an object in parallel (each with its device
assembly kept for the ISA check), then the objects are linked into one
shared library.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdbd.so")
ARCH = "gfx950"

# -packed-fp32-ops off: keep the compiler from emitting packed fp32 VALU
# instructions; the kernels use plain fp32 arithmetic.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libdbd)")


def check_isa(asm_dir: str, verbose: bool = False) -> None:
    """Scans the kept gfx950 assembly for LDS-DMA wait-state hazards
    (isa_check); raises if any is found."""
    from block_diffusion_amd import isa_check
    found, n = [], 0
    for f in sorted(glob.glob(os.path.join(asm_dir, "**", f"*-hip-amdgcn-amd-amdhsa-{ARCH}.s"),
                              recursive=True)):
        with open(f) as fh:
            k, h = isa_check.scan(fh.read())
        n += k
        found += [(os.path.basename(f),) + x for x in h]
    if found:
        msg = "\n".join(f"  {f}:{line} {kern}: '{dma}' after '{w}'" for f, kern, line, dma, w in found[:20])
        raise RuntimeError(f"{len(found)} LDS-DMA wait-state hazard(s) in the compiled kernels:\n{msg}")
    if verbose:
        print(f"ISA check: {n} LDS-DMA instructions, no wait-state hazard", flush=True)


def _run(cmd, cwd):
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=cwd)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, err


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    inc = os.path.abspath(os.path.join(HERE, "..", "include"))
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="dbd_build_") as work:
        jobs = []
        for s in srcs:
            d = os.path.join(work, os.path.splitext(os.path.basename(s))[0])
            os.makedirs(d)
            # -save-temps keeps the device assembly that is linked, for check_isa
            jobs.append(([hipcc(), *FLAGS, "-save-temps", "-I", inc, "-c", s, "-o",
                          os.path.join(d, "obj.o")], d))
        if verbose:
            for cmd, _ in jobs:
                print(" ".join(cmd), flush=True)
        nproc = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
        with ThreadPoolExecutor(nproc) as ex:
            res = list(ex.map(lambda j: _run(*j), jobs))
        for (cmd, _), (rc, err) in zip(jobs, res):
            if rc != 0:
                raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-3]}:\n{err}")
            if err.strip() and verbose:
                print(err, file=sys.stderr)
        link = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp,
                *[os.path.join(d, "obj.o") for _, d in jobs]]
        rc, err = _run(link, work)
        if rc != 0:
            raise RuntimeError(f"link failed ({rc}):\n{err}")
        try:
            check_isa(work, verbose)
        except RuntimeError:
            os.remove(tmp)
            raise
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
