"""Host-side checks of bench.py that need no GPU."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU only" in res.stdout + res.stderr


def test_exact_kernel_names_follow_the_library_rule():
    sys.path.insert(0, ROOT)
    import bench
    from synthetic import WORKLOADS
    names = {i: bench.exact_batched_kernel(WORKLOADS[i]) for i in WORKLOADS}
    assert names[1] == "sk_exact_tiled (VALU)"          # d = dv = 4
    assert names[2] == "sk_exact_mfma16"                # dv = 16
    assert names[3] == names[4] == "sk_exact_mfma"      # dv = 32, 64
    assert names[5] == "sk_exact_tiled (VALU)"          # d = dv = 8
