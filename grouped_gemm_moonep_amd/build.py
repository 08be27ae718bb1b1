"""Build libmoonep.so for gfx950 with hipcc (in-tree).

    python grouped_gemm_moonep_amd/build.py

Every source under csrc/ is compiled for --offload-arch=gfx950 and linked
into grouped_gemm_moonep_amd/libmoonep.so.  Packed-fp32 instructions are
disabled for all device code; the data-movement file is also compiled without
floating-point contraction (its sums are defined operation by operation).
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoonep.so")
SOURCES = ["api.hip", "plan.hip", "plan_noalloc.hip", "move.hip", "gemm.hip", "gemm_bwd.hip",
           "symbuf.hip"]
ARCH = "gfx950"


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoonep.so)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        "-mcode-object-version=5",
        "-I", os.path.join(REPO, "include"), "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
    ]


def _compile(src):
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    flags = common_flags()
    if src == "move.hip":
        flags.append("-ffp-contract=off")
    cmd = [hipcc()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    return obj, out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, out in results:
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
