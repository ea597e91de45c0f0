"""Host-side checks of bench.py's contract (no GPU needed).

The benchmark runs on one GPU only; asking for more must stop with a message
and a nonzero status before anything touches a device.  The roofline fields
are plain ratios against MI355X's published peaks (8 TB/s HBM3E, 2.5 PFLOP/s
dense bf16 MFMA), and the 128-head workloads are judged on MFMA, the others
on HBM.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_roofline_fractions():
    import bench
    from workloads import configs
    w16, w128 = configs.BY_NAME["tplocal"], configs.BY_NAME["replq"]
    # 8e12 bytes and 2.5e15 FLOP in one second (1000 ms) are exactly the peaks
    r = bench.roofline_of(w16, 2.5e15, 8e12, 1000.0)
    assert r["bound"] == "hbm" and r["frac"] == pytest.approx(1.0) and r["mfma_frac"] == pytest.approx(1.0)
    r = bench.roofline_of(w128, 1.25e15, 2e12, 1000.0)
    assert r["bound"] == "mfma" and r["frac"] == pytest.approx(0.5) and r["hbm_frac"] == pytest.approx(0.25)
    assert r["gbps"] == pytest.approx(2000.0) and r["tflops"] == pytest.approx(1250.0)
