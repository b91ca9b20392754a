"""Build libeqlinear.so from csrc/ with hipcc for gfx950 (cross-compiles without a GPU)."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libeqlinear.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")

ARCH = "gfx950"
# Packed-fp32 VALU ops are disabled: the plain scalar forms are used everywhere.
# MFMA results live in ordinary VGPRs (gfx950 allows it): no copies between the
# accumulation registers and the VALU, and fewer registers in all.
# The first 16 dwords of kernel arguments are preloaded into SGPRs at wave
# launch (gfx950 supports it; the code object keeps a loading prologue for
# firmware that does not), instead of scalar loads whose round trips the
# compiler otherwise spreads over the kernel's first instructions.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++20", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libeqlinear")


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + HIPCC_FLAGS + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every csrc/*.hip for gfx950 and link libeqlinear.so (always rebuilds)."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)), 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # a kernel whose host-side stub was not emitted leaves an undefined symbol
    # that only shows when the library is loaded: refuse such a link here
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    stubs = [l.split()[-1] for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if stubs:
        os.remove(tmp)
        raise RuntimeError("kernel stubs missing from the link (host compilation dropped them): "
                           + ", ".join(stubs[:4]))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def stale() -> bool:
    """True if the library is missing or older than any source file."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + glob.glob(os.path.join(CSRC, "*.h")) + [os.path.join(ROOT, "include", "eqlinear.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    build()
