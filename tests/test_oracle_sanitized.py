"""The oracle's CPU pin suites once more against an AddressSanitizer + UndefinedBehaviorSanitizer
build of oracle.c: any out-of-bounds access, use after free, signed overflow or other undefined
behaviour in the oracle aborts the child run.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_alg2.py", "tests/test_oracle_int8.py",
              "tests/test_oracle_ccq_encoder.py"]


@pytest.mark.slow
def test_pin_suites_clean_under_asan_ubsan():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("another library is preloaded in this environment; the ASan runtime must come first")
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's ASan runtime is not installed")
    env = dict(os.environ, ORACLE_SANITIZE="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    sys.path.insert(0, ROOT)
    import oracle

    r = subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"], cwd=ROOT,
                       env=dict(os.environ, ORACLE_SANITIZE="1"), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    try:
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *PIN_SUITES],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    finally:
        san = os.path.join(ROOT, "oracle", "liboracle_san.so")
        if os.path.exists(san):
            os.remove(san)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert oracle  # the unsanitized module in this process is untouched
