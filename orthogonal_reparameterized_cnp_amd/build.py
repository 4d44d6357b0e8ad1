"""Build libpoetx.so in-tree with hipcc for gfx950.

    python -m orthogonal_reparameterized_cnp_amd.build      (or build() from Python)

The library is one shared object with a plain C ABI (include/poetx.h); the
Python binding loads it with ctypes.
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpoetx.so")
SOURCES = ["poetx_kernels.hip", "poetx_cnp.hip", "poetx_optim.hip", "poetx_api.hip"]

# Packed fp32 instructions are kept out of the device code (-packed-fp32-ops);
# the host pass warns that it does not know the feature, which is harmless.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpoetx)")


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libpoetx.so; returns its path."""
    objs = []
    cc = hipcc()
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [cc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), src))
        objs.append(obj)
    failed = []
    for p, src in procs:
        out, _ = p.communicate()
        noise = [l for l in out.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if p.returncode != 0:
            failed.append((src, "\n".join(noise)))
        elif noise and verbose:
            print("\n".join(noise))
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(f"[{s}]\n{o}" for s, o in failed))
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
