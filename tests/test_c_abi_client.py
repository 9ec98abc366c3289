"""The library from a plain C program (tests/c_abi/mla_c_abi.c): no Python or
torch between the caller and include/pkv.h.  The program compares its result
with the CPU oracle itself and exits 0 on agreement."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_abi", "mla_c_abi")


@pytest.mark.gpu
def test_c_client_matches_oracle():
    assert os.path.exists(BIN), "tests/c_abi/mla_c_abi is not built (run __graft_entry__.build())"
    print("[c-abi] running", BIN, flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "PASS" in r.stdout


def test_c_client_builds():
    """The C client compiles as C99 against the public header (CPU check)."""
    subprocess.run(["make", "-s", "-C", os.path.join(HERE, "c_abi")], check=True)
    assert os.path.exists(BIN)
