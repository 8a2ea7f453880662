"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a g++ build with both (every finding
fatal) runs the oracle's pins in a child Python process with the sanitizer runtimes preloaded."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_oracle_pins_under_asan_ubsan():
    from oracle.build import build, sanitize_env

    build(sanitize=True)
    env = sanitize_env()
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    tail = (r.stdout[-1500:] + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
