"""Compile the HIP sources into the in-tree shared library ``libsvgear.so`` (gfx950)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsvgear.so")
SOURCES = ["api.hip", "kmeans.hip", "route.hip", "attn.hip", "seed.hip", "quant.hip"]
ARCH = os.environ.get("SVGEAR_ARCH", "gfx950")

# Packed fp32 instructions are kept out of the device code on purpose.
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)


def _check_no_undefined_kernels(lib: str) -> None:
    """A kernel whose host-side stub the compiler silently dropped shows up as
    an undefined symbol of the library's own namespace; refuse such a build."""
    nm = shutil.which("nm")
    if nm is None:
        return
    r = subprocess.run([nm, "-D", "--undefined-only", lib], capture_output=True, text=True)
    bad = [l.split()[-1] for l in r.stdout.splitlines() if "3svg" in l]
    if bad:
        raise RuntimeError("library has undefined kernel symbols (host stub not emitted): " + ", ".join(bad))


def build(verbose: bool = False) -> str:
    """Always recompiles every source and relinks the library; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    jobs = min(len(SOURCES), max(1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose), zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    _check_no_undefined_kernels(tmp)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
