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
           "muon_elementwise.hip", "muon_grasp.hip", "muon_api.hip", "muon_schedule.cpp", "muon_ceiling.hip"]
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


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (the device code is
# built as usual): for checking the argument checks, workspace planning and
# schedule derivation on the CPU.  Load the result with the clang sanitizer
# runtime preloaded (see sanitizer_runtime()).
SANITIZE_COMPILE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_LINK = ["-fsanitize=address", "-fsanitize=undefined", "-fno-gpu-sanitize", "-shared-libsan"]


def sanitizer_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime that a sanitized build links against."""
    out = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


def build(verbose: bool = False, csrc: str = CSRC, lib: str = LIB, defines=(), sanitize: bool = False) -> str:
    """Always recompiles (one process per source, in parallel); writes the
    library (default libmuon.so next to this file) atomically and returns its
    path.  ``csrc``, ``lib`` and ``defines`` (-D flags) build a variant;
    ``sanitize`` instruments the host code (see SANITIZE_COMPILE)."""
    objdir = tempfile.mkdtemp(prefix="muon_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            san = SANITIZE_COMPILE if sanitize else []
            procs.append((src, _run([hipcc(), *HIPCC_FLAGS, *san, *[f"-D{d}" for d in defines], "-c", "-o", obj,
                                     os.path.join(csrc, src)], verbose)))
        for src, proc in procs:
            _finish(proc, src, verbose)
        tmp = lib + ".tmp"
        _finish(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SANITIZE_LINK if sanitize else []),
                      "-o", tmp, *objs], verbose), "link", verbose)
        os.replace(tmp, lib)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return lib


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        print(build(verbose=True, lib=os.path.join(HERE, "libmuon_sanitized.so"), sanitize=True))
        print("runtime to preload:", sanitizer_runtime())
    else:
        print(build(verbose=True))
