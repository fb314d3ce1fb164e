"""Job lists of the attention grids (host only, no GPU).

The attention kernels map each workgroup index to a (role, block, head,
sequence) job through attn_sched.hpp. A wrong mapping would leave output
blocks unwritten or address a head past the tensors, so the header is built
into a small host program (tests/attn_sched_check.cpp) that enumerates whole
grids over a sweep of shapes: every index maps to a distinct job inside the
grid, each XCD's list runs in rank order (longest causal jobs first), and
the lists have equal lengths where the grid is grouped by XCD.
"""
import os
import subprocess

import pytest

from tensor_model_transformer_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))


def test_job_lists_cover_each_job_once(tmp_path):
    exe = str(tmp_path / "attn_sched_check")
    cmd = [build._hipcc(), "-x", "hip", f"--offload-arch={build.ARCH}", "-O1", "-std=c++17",
           "-I", build.CSRC, os.path.join(HERE, "attn_sched_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("hipcc failed:\n" + r.stderr[-2000:])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
