"""The C ABI used from a host program with no Python or torch in it
(tests/c_abi/moe_abi_check.cpp, built by __graft_entry__.build() or
`python -m combine_moe_layout_06_amd.build`): a small layer and the
hierarchical pass, checked against the invariants the method fixes."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "moe_abi_check")


def test_host_program_through_the_c_abi():
    assert os.path.exists(BIN), "build it first: python -m combine_moe_layout_06_amd.build"
    print("running", BIN, flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert "c-abi check ok" in r.stdout
