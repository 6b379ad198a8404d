"""The oracle's pins, rerun against an AddressSanitizer + UndefinedBehaviorSanitizer build of
liboracle.so (gcc, host code): an out-of-bounds access, a use after free or undefined behaviour
(signed overflow, misaligned access, a bad shift) anywhere the pins reach aborts the run. CPU only;
the sanitizer runtime is preloaded into a fresh interpreter."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_recurrence.py", "tests/test_oracle_replay.py", "tests/test_oracle_quant.py",
        "tests/test_oracle_mxfp4.py", "tests/test_oracle_master.py", "tests/test_oracle_gdn.py",
        "tests/test_oracle_mixer.py", "tests/test_pointer_machine_properties.py"]


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    runtime = _asan_runtime()
    if runtime is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from oracle import build as oracle_build
    lib = oracle_build.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    env = dict(os.environ, RSSM_ORACLE_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stdout + r.stderr, tail
    assert "runtime error" not in r.stdout + r.stderr, tail
