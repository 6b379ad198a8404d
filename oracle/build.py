"""Build the float64 CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

Plain IEEE float64: no -ffast-math and no FMA contraction, so the oracle's arithmetic is exactly
what its source says.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, f) for f in ("oracle.c", "oracle_gdn.c", "oracle_mixer.c")]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """Compile the oracle into `out`. sanitize: an AddressSanitizer + UndefinedBehaviorSanitizer
    build (host code, gcc) for the tests that run the oracle's pins under the sanitizers."""
    opt = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-Wall", "-Wextra", "-o", out + ".tmp", *SRCS, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
