"""Host-side checks of bench.py (no GPU): the step graph's branches cover
every phase once and keep the commit after the verify it reads, the
algorithmic byte counts follow from the workload shapes, and a request for
more than one GPU is refused before any work."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_step_branches_cover_every_phase_once():
    flat = [ph for br in bench.STEP_BRANCHES for ph in br]
    assert sorted(flat) == sorted(bench.STEP)
    assert len(flat) == len(set(flat))
    # the commit copies the verify's snapshots: same branch, after it
    for br in bench.STEP_BRANCHES:
        if "commit" in br:
            assert "verify" in br and br.index("verify") < br.index("commit")


def test_prefill_bytes_follow_the_shapes():
    from linear_attention_03_amd import workloads as wl
    c = wl.config2_prefill(4096)
    T, H, K, V = 4096, 16, 128, 128
    want = (T * H * K * 2 * 2      # q, k (bf16)
            + T * H * K * 2        # g (bf16)
            + T * H * V * 2 * 2    # v and o (bf16)
            + T * H * 2            # beta (bf16)
            + H * 4 + H * K * 4    # A_log, dt_bias (fp32)
            + 2 * H * V * K * 4)   # one state read and written (fp32)
    assert bench.prefill_bytes(c) == want


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one-GPU" in r.stderr
    assert r.stdout == ""
