"""The library from C alone: tests/c_abi/sq_c_pipeline.c includes include/sq.h,
allocates device buffers with hipMalloc, runs the five calls and compares every
output bit for bit with the oracle's C functions (no Python or torch in the
loop).  The program is compiled by __graft_entry__.build()."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "sq_c_pipeline")


def _program():
    if not os.path.exists(BIN):
        import __graft_entry__
        __graft_entry__.build_c_pipeline()
    return BIN


def test_c_program_host_checks():
    """Argument checks, workspace sizes and status strings from C; no GPU call."""
    r = subprocess.run([_program(), "host"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "host checks ok" in r.stdout


@pytest.mark.gpu
def test_c_program_pipeline_matches_oracle():
    """Three cases (ragged tiles, per-tensor with a general alpha, several
    256-row GEMM tiles), every output compared with the oracle."""
    assert os.path.exists(BIN), "build the C test program first: python -c 'import __graft_entry__ as g; g.build()'"
    print("c pipeline: 300x512x392, 64x1024x256, 2100x4096x3000", flush=True)
    r = subprocess.run([BIN, "gpu"], capture_output=True, text=True, timeout=240)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c pipeline ok" in r.stdout
