"""The C ABI's host-side validation under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU): the CPU ABI
tests run again, in a child process, against a build whose argument checking is instrumented. A memory error
aborts the child and an undefined-behaviour finding stops it with an illegal instruction, so a clean run means the
validation of every argument set those tests pass (NULL, misaligned, out-of-range, unaddressable sizes, unknown
status codes) stays within defined behaviour."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_is_clean_under_host_sanitizers():
    try:
        from long_context_attention_causal_amd import sanitize
    except ImportError:   # the sanitizer recipe is a CPU-side tool and is not shipped everywhere
        pytest.skip("sanitizer build recipe not present")
    sanitize.build()
    env = sanitize.environment()
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, f"sanitized ABI tests failed (rc {r.returncode}):\n{tail}"
    assert " passed" in r.stdout
