"""Build libwmtp.so (the HIP library behind include/wmtp.h) in-tree for gfx950.

    python -m draft_attention_amd.build

hipcc cross-compiles for gfx950 without a GPU. Packed-FP32 instructions are switched off for the
device code (-packed-fp32-ops); the host pass warns that it does not know the feature, which is
harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libwmtp.so")
SOURCES = ["abi.hip", "attn.hip", "ring.hip", "accept.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, out: str = LIB, host_flags=()) -> str:
    """Compile every source to an object (all at once) and link libwmtp.so. Returns its path.

    ``out``: where the library goes (objects beside it in ``_build`` for another path);
    ``host_flags``: extra flags for the host pass only (each passed as -Xarch_host FLAG, at compile
    and link time), e.g. sanitizers for a CPU-side check of the argument validation."""
    objdir = os.path.join(PKG if out == LIB else os.path.dirname(os.path.abspath(out)), "_build")
    os.makedirs(objdir, exist_ok=True)
    host = [x for f in host_flags for x in ("-Xarch_host", f)]
    common = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", INCLUDE, "-I", CSRC] + host
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [hipcc()] + common + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        log, _ = p.communicate()
        text = log.decode(errors="replace")
        noise = "is not a recognized feature for this target"
        shown = "\n".join(l for l in text.splitlines() if noise not in l)
        if shown.strip() and (verbose or p.returncode != 0):
            print(f"--- {src}\n{shown}", file=sys.stderr)
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + host + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
