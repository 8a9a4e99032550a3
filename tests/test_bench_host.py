"""Host-side contract of bench.py (CPU only): the multi-GPU refusal, and the stored HBM traffic of
the dense pass being keyed to the kernel sources it was measured on."""

import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""                                         # no JSON line


def test_refuses_a_distributed_launch():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=120, cwd=ROOT, env=env)
    assert r.returncode == 2 and "WORLD_SIZE 4" in r.stderr


def test_stored_traffic_matches_the_current_kernel_sources():
    """roofline.traffic is reported only for the sources the counters were taken on: the digest of
    the dense pass's sources must be a key of KNOWN_TRAFFIC (re-measure FETCH_SIZE / WRITE_SIZE and
    re-key it after any change to them), and the stored value must be at least the pass's
    algorithmic bytes (32 x 131072 rows x 512 B of K and V)."""
    for f in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, f)), f
    d = bench.kernel_digest()
    assert re.fullmatch(r"[0-9a-f]{16}", d)
    assert d in bench.KNOWN_TRAFFIC, "kernel sources changed since the HBM counters were taken"
    assert bench.KNOWN_TRAFFIC[d] >= 32 * 131072 * 512
