"""The C ABI without Python: tests/c_abi/verify_round (built by __graft_entry__.build())
creates an engine through include/hdt.h, verifies a 6-node tree through a GDN and an
attention layer, commits a root path, and checks outputs, state and cache rows against the
C oracle."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(__file__), "c_abi", "verify_round")


def test_c_program_verify_round():
    assert os.path.exists(BIN), "build() compiles tests/c_abi/verify_round"
    print("running tests/c_abi/verify_round", flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "PASS" in r.stdout
