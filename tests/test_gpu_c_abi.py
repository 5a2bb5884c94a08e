"""The library used from plain C: tests/c_abi/abi_roundtrip.c (built by __graft_entry__.build())
allocates device buffers with hipMalloc and, on a stream of its own, runs quantize +
dequantize for every rule, three group layouts and both quantize forms, a paged quantize and
gather through a shuffled block table (two rules), RTN INT4 and INT2 round trips, comparing
every output byte with the oracle, and an attention call against the oracle's double
attention (max |err| <= 2e-2, rel RMS <= 1e-2); it also checks host-side argument errors.
It runs as its own process (its own HIP runtime)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_roundtrip")


def test_c_program_round_trip_matches_oracle():
    if not os.path.exists(EXE):
        pytest.fail("tests/c_abi/abi_roundtrip not built (run __graft_entry__.build())")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("OK")
    # 3 layouts x 3 rules x 2 quantize forms, the plain entry point, 2 paged rules, 2 RTN widths
    assert r.stdout.count("bit-exact") == 23
    assert r.stdout.count("within tolerance") == 1
