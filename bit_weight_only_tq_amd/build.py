"""Build libtq.so (the HIP kernels and the C ABI) in-tree for gfx950.

Usage: python -m bit_weight_only_tq_amd.build  (or call ``build()``).

Every HIP translation unit is compiled with hipcc for --offload-arch=gfx950
and linked into ``bit_weight_only_tq_amd/libtq.so``.  The prepare kernels
(pack.hip) are compiled with -ffp-contract=off so that their fp64 sums and
divisions are exactly the operations written.  Packed fp32 instructions are
disabled for all device code (-packed-fp32-ops); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtq.so")
ARCH = "gfx950"

SOURCES = {
    "pack.hip": ["-ffp-contract=off"],
    "gemv.hip": [],
    "gemm.hip": [],
    "diag.hip": [],
    "api.cpp": ["-x", "hip"],
}


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile all sources and link libtq.so; returns the library path."""
    hipcc = _hipcc()
    common = [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
    ]
    with tempfile.TemporaryDirectory(prefix="tq_build_") as tmp:
        procs = []
        objs = []
        for src, extra in SOURCES.items():
            obj = os.path.join(tmp, src.replace(".", "_") + ".o")
            cmd = [hipcc] + common + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
            objs.append(obj)
            procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        failed = []
        for src, cmd, p in procs:
            out = p.communicate()[0].decode(errors="replace")
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
            if p.returncode != 0:
                failed.append((src, " ".join(cmd), "\n".join(lines)))
            elif verbose and lines:
                print(f"[{src}]\n" + "\n".join(lines))
        if failed:
            msg = "\n\n".join(f"{s}: {c}\n{o}" for s, c, o in failed)
            raise RuntimeError(f"libtq build failed:\n{msg}")
        tmp_lib = LIB + ".tmp"
        link = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp_lib] + objs
        r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            raise RuntimeError("libtq link failed:\n" + r.stdout.decode(errors="replace"))
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
