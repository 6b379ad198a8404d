"""Build libreplayssm.so (HIP, gfx950) in-tree.

kernels.hip is compiled once per supported state size N (in parallel), api.hip once, and the
objects are linked into hybrid_mamba_decode_amd/libreplayssm.so. Objects go to _build/.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libreplayssm.so")
STATE_SIZES = (16, 32, 64, 128, 256)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU ops are kept out of the device code (plain float code only).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)


def build(verbose: bool = False, jobs: int = 0) -> str:
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(8, (os.cpu_count() or 4))
    steps = []
    for n in STATE_SIZES:
        steps.append([HIPCC, *FLAGS, f"-DRSSM_N={n}", "-c", os.path.join(CSRC, "kernels.hip"),
                      "-o", os.path.join(OBJ, f"kernels_n{n}.o")])
    steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, "api.hip"), "-o", os.path.join(OBJ, "api.o")])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, s, verbose) for s in steps]:
            f.result()
    objs = [os.path.join(OBJ, f"kernels_n{n}.o") for n in STATE_SIZES] + [os.path.join(OBJ, "api.o")]
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs], verbose)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
