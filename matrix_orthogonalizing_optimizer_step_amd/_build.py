"""Compile the HIP sources of the Muon library into ``libmuon.so`` (gfx950).

``python -m matrix_orthogonalizing_optimizer_step_amd._build`` builds in
place; the shared library sits next to this file so it travels with the
source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmuon.so")
SOURCES = ["muon_gemm_bf16.hip", "muon_gemm_f16.hip", "muon_gemm_f32.hip", "muon_gemm.hip",
           "muon_elementwise.hip", "muon_grasp.hip", "muon_api.hip", "muon_schedule.cpp"]
ARCH = os.environ.get("MUON_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _run(cmd: list[str], verbose: bool) -> subprocess.Popen:
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(proc: subprocess.Popen, what: str, verbose: bool) -> None:
    out, _ = proc.communicate()
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in out.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed on {what} ({proc.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)


def build(verbose: bool = False, csrc: str = CSRC, lib: str = LIB, defines=()) -> str:
    """Always recompiles (one process per source, in parallel); writes the
    library (default libmuon.so next to this file) atomically and returns its
    path.  ``csrc``, ``lib`` and ``defines`` (-D flags) build a variant."""
    objdir = tempfile.mkdtemp(prefix="muon_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            procs.append((src, _run([hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-c", "-o", obj,
                                     os.path.join(csrc, src)], verbose)))
        for src, proc in procs:
            _finish(proc, src, verbose)
        tmp = lib + ".tmp"
        _finish(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose), "link", verbose)
        os.replace(tmp, lib)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
