"""The CPU tests of the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

The library is rebuilt with both sanitizers on its host code
(build.build_host_sanitized: device code as usual, never launched here),
then the ABI and host-fuzz tests run in a child Python process that loads it
through PKV_LIBRARY with the sanitizer runtime preloaded.  Any report stops
the child (halt_on_error) and fails this test.
"""

import os
import subprocess
import sys

from paged_kv_cache_mapping_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_address_and_undefined_behaviour_sanitizers():
    lib = build.build_host_sanitized()
    env = dict(os.environ)
    env.update(PKV_LIBRARY=lib, LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a report is written to the child's stderr, not into a capture the
    # halted child never prints
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_abi_cpu.py", "tests/test_host_fuzz_cpu.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
