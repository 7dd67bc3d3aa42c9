"""The oracle's pins once more, against a build of oracle_sdm.c with
AddressSanitizer and UndefinedBehaviorSanitizer (out-of-bounds accesses, use
after free, signed overflow, misaligned loads and the like abort the run).
Runs in a child process that preloads the ASan runtime, since the Python
interpreter itself is not instrumented."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    except OSError:
        return None
    return p if p and os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime() is None, reason="no gcc ASan runtime")
def test_oracle_pins_under_address_and_undefined_behaviour_sanitizers():
    # the ASan runtime must come first among preloaded libraries; keep any others after it
    preload = " ".join(p for p in (_runtime(), os.environ.get("LD_PRELOAD", "")) if p)
    env = dict(os.environ, SDM_ORACLE_SANITIZE="1", LD_PRELOAD=preload,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"], cwd=ROOT, env=env,
                   check=True, timeout=300)
    pins = ["tests/test_oracle_pins.py", "tests/test_oracle_backward_pins.py", "tests/test_oracle_idw_pins.py",
            "tests/test_oracle_bf16_table_pins.py", "tests/test_oracle_glue_pins.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail
