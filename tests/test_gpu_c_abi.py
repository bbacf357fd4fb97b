"""The library driven from a plain C program through its C ABI alone: the
HIP runtime for device memory and the stream, no Python and no torch in
that process (tests/c_abi/step_from_c.c, built by __graft_entry__.build()).
The program runs the clipped step, the no-alloc clipped step and the
three-call step on ragged lists and checks every element against the
oracle it links; this test runs it and reads its result."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "step_from_c")


def test_c_program_steps_match_the_oracle():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build it with __graft_entry__.build()")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    print(r.stderr)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().endswith("c abi ok"), r.stdout
