"""The host-side tests again, on AddressSanitizer + UndefinedBehaviorSanitizer builds of the
oracle, the input generator and libhdt's host code (tests/sanitize.py).

The child run covers the oracle against its pins and planted mistakes, the generator, and
every host check of the C ABI (descriptor, tree, path, order and capacity refusals, the
snapshot header checks, tree metadata).  Any sanitizer report fails it: ASan stops at the
first bad access and UBSan is built not to recover.
"""
import os
import subprocess
import sys

import pytest

from tests import sanitize

HOST_TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_mutants.py", "tests/test_synth.py",
              "tests/test_abi_host.py", "tests/test_price_table.py"]


@pytest.mark.skipif(sanitize.runtime() is None, reason="clang's ASan runtime is not installed")
def test_host_code_under_asan_and_ubsan():
    env = dict(os.environ)
    env.update(sanitize.build())
    env["LD_PRELOAD"] = sanitize.runtime()
    # Python and PyTorch are not instrumented: their allocations are not leaks of ours
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                          "-p", "no:cacheprovider", *HOST_TESTS],
                         cwd=sanitize.ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out, out[-6000:]
    assert "runtime error:" not in out, out[-6000:]
    assert " passed" in out
    # the sanitized builds are the ones a child process maps
    probe = ("import oracle, synth, hybrid_deltanet_tree_amd\n"
             "oracle._load(); synth._load()\n"
             "print(open('/proc/self/maps').read())")
    maps = subprocess.run([sys.executable, "-c", probe], cwd=sanitize.ROOT, env=env,
                          capture_output=True, text=True, timeout=300)
    assert maps.returncode == 0, maps.stderr[-4000:]
    for name in ("liboracle.so", "libsynth.so", "libhdt.so"):
        assert os.path.join(sanitize.OUT, name) in maps.stdout, name
