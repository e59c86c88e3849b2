"""Host-side checks of bench.py's contract (no GPU).

- More than one GPU is refused with a message and a non-zero status: the hot
  path is measured on one GPU.
- profiles/hbm_traffic.txt, which bench.py reads for roofline.traffic, is well
  formed: every line names a kernel key bench.py knows, a workload, a 16-digit
  source hash and two byte counts.
"""

import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_traffic_table_is_well_formed():
    keys = set(bench.KERNEL_SOURCES)
    n = 0
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.txt")) as fh:
        for line in fh:
            if not line.strip() or line.startswith("#"):
                continue
            f = line.split()
            assert len(f) == 5, line
            assert f[0] in keys, line
            assert re.fullmatch(r"[0-9a-f]{16}", f[2]), line
            assert int(f[3]) > 0 and int(f[4]) >= 0, line
            n += 1
    assert n >= 9
