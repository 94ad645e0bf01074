"""Host-side checks of bench.py: byte accounting, the one-GPU guard and the profiling
recipe.  No GPU is needed.

The throughput metric is effective bandwidth, bytes the method must move divided by
time ("Fused RMSNorm", aryanashta.me, "What it is": how close a kernel gets to the
card's memory ceiling).  The expected byte counts below were worked out by hand from
that definition for the four named workloads: read x, write y, read gamma (and beta),
write the saved fp32 statistics; backward read x, dy, gamma and the statistics, write
dx and the fp32 dgamma (and dbeta).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("kind,M,N,s,fwd,bwd", [
    # RMSNorm [4096, 1024] bf16: 2*8 MiB + 2 KiB gamma + 16 KiB rstd
    ("rms", 4096, 1024, 2, 16_795_648, 25_188_352),
    # LayerNorm [65536, 4096] bf16
    ("ln", 65536, 4096, 2, 1_074_282_496, 1_611_177_984),
    # RMSNorm [262144, 384] bf16
    ("rms", 262144, 384, 2, 403_702_528, 605_030_656),
    # RMSNorm [2048, 131072] bf16
    ("rms", 2048, 131072, 2, 1_074_012_160, 1_611_407_360),
])
def test_ideal_bytes_of_the_named_workloads(kind, M, N, s, fwd, bwd):
    assert bench.ideal_bytes(kind, M, N, s) == (fwd, bwd)
    # the backward's main kernel moves everything but the fp32 gradient vectors
    assert bench.main_bwd_kernel_bytes(kind, M, N, s) == bwd - (4 if kind == "rms" else 8) * N


def test_mixed_parameter_bytes():
    # fp32 gamma/beta beside bf16 activations: only the parameter reads change
    f16, b16 = bench.ideal_bytes("ln", 8, 64, 2)
    f32p, b32p = bench.ideal_bytes("ln", 8, 64, 2, 4)
    assert f32p - f16 == 2 * 64 * 2 and b32p - b16 == 64 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_profiling_recipe_keeps_counters_apart_from_traces():
    """Counter collection runs on its own: no --pmc run also asks for a trace domain."""
    trace_flags = ("--sys-trace", "-s ", "--runtime-trace", "-r ", "--hip-trace",
                   "--hsa-trace", "--memory-copy-trace", "--scratch-memory-trace",
                   "--marker-trace", "--kernel-trace", "--stats")
    cmds = [c.format(w="ln2", c=1 << 30) for c in bench.PROFILE_STEPS]
    pmc = [c for c in cmds if "--pmc" in c]
    assert len(pmc) == 5
    for c in pmc:
        assert not any(f in c for f in trace_flags), c
        # the program is what follows "--": never a launcher that re-executes
        prog = c.split(" -- ", 1)[1].split()[0]
        assert prog == "python3", c
    assert any("--kernel-trace --stats" in c for c in cmds)
