"""Builds liblacache.so (the HIP library behind include/lacache.h) for gfx950.

Usage: python -m exact_attention_state_amd.build   (or __graft_entry__.build()).
Compiles every csrc/*.hip with hipcc into one shared library placed next to
this file, so it ships with the source tree.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblacache.so")
ARCH = os.environ.get("LACACHE_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: accumulators that VALU code also
    # touches (the online-softmax rescale) are not moved through AGPRs.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    return r.returncode, r.stdout + r.stderr


def build(verbose=False):
    """Compiles each source to an object in parallel, then links the library."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(f)[:-4] + ".o") for f in srcs]
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    cmds = [[hipcc, *compile_flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", f, "-o", o]
            for f, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), 4)) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    log = "\n".join(out for _, out in results)
    if any(rc != 0 for rc, _ in results):
        sys.stderr.write(log)
        raise RuntimeError("hipcc failed building liblacache.so")
    tmp = LIB + ".tmp"
    rc, out = _run([hipcc, *HIPCC_FLAGS, *objs, "-o", tmp], verbose)
    log += "\n" + out
    if rc != 0:
        sys.stderr.write(log)
        raise RuntimeError("hipcc failed linking liblacache.so")
    warn = "\n".join(l for l in log.splitlines() if "packed-fp32-ops" not in l)
    if verbose and warn.strip():
        print(warn)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
