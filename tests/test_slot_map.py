"""The grouped GEMM's XCD slot map, checked on the host: the kernels and
this check compile the same function (`xcd_slot_pair` in launch.hpp).  For
random tile tables (routed tiles followed by shared-expert tiles), every
active (M tile, N tile) pair must be taken by exactly one block of the grid
the launcher sizes (`job_blocks`), and every other block must get no work."""
import os
import subprocess
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fine_grained_sparse_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_every_tile_pair_has_exactly_one_block():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "slot_map_check")
        cmd = [HIPCC, "-O2", "-std=c++17", "-I" + CSRC, os.path.join(ROOT, "tests", "slot_map_check.cpp"), "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
        assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
