"""Build libreplayssm.so (HIP, gfx950) in-tree, and the benchmark's bandwidth probes
(libbwprobe.so).

kernels.hip (Mamba-2) and gdn_kernels.hip (Gated DeltaNet) are compiled once per supported state
/ key size N (in parallel), api.hip and gdn_api.hip once, and the objects are linked into
hybrid_mamba_decode_amd/libreplayssm.so. Objects go to _build/.
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
PROBE_LIB = os.path.join(PKG, "libbwprobe.so")  # bandwidth probes for the benchmark's ceilings
STATE_SIZES = (16, 32, 64, 128, 256)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 VALU ops are kept out of the device code (plain float code only). MFMA
# accumulators are kept in ordinary VGPRs (no copies to and from the accumulation registers).
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form"]


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
    objs = []
    for src in ("kernels", "gdn_kernels"):
        for n in STATE_SIZES:
            obj = os.path.join(OBJ, f"{src}_n{n}.o")
            steps.append([HIPCC, *FLAGS, f"-DRSSM_N={n}", "-c", os.path.join(CSRC, f"{src}.hip"), "-o", obj])
            objs.append(obj)
    for src in ("api", "gdn_api"):
        obj = os.path.join(OBJ, f"{src}.o")
        steps.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, f"{src}.hip"), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, s, verbose) for s in steps]:
            f.result()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs], verbose)
    os.replace(LIB + ".tmp", LIB)
    _run([HIPCC, *FLAGS, "-shared", "-o", PROBE_LIB + ".tmp", os.path.join(CSRC, "bwprobe.hip")], verbose)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
