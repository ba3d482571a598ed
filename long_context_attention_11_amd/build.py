"""Build the HIP library ``libcsa.so`` in-tree for gfx950.

Run as ``python -m long_context_attention_11_amd.build`` (or call ``build()``).  Always
recompiles.  The library is placed next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["csa_api.cpp", "compress.hip", "indexer.hip", "topk.hip", "attend.hip", "proj.hip"]
LIB = os.path.join(HERE, "libcsa.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are switched off: hand-free codegen of v_pk_{add,mul,fma}_f32 is
# avoided on this platform.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (device code is unaffected): the
# checks, planning and dispatch code of the C ABI, for the host sanitizer test.
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library needs ROCm's hipcc")


def build(verbose: bool = False, jobs: int = 4, out: str = LIB, host_sanitize: bool = False) -> str:
    """Compile every source for gfx950 and link ``out`` (the in-tree libcsa.so by default).
    host_sanitize builds the host code with the sanitizers (a separate library, for tests)."""
    cc = hipcc()
    extra = HOST_SANITIZE if host_sanitize else []
    tmp = tempfile.mkdtemp(prefix="csa_build_")
    try:
        objs, procs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"]
            cmd = [cc, *HIP_FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0), verbose)
        for p in procs:
            _wait(p, verbose)
        out_tmp = out + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *extra, *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(out_tmp, out)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return out


def _wait(item, verbose):
    src, p = item
    out = p.communicate()[0].decode(errors="replace")
    if p.returncode:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
