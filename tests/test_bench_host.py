"""Host-side checks of bench.py: the one-GPU guard and the record arithmetic."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def test_records():
    # 2 GB of algorithmic bytes in 1 ms: 2000 GB/s, a quarter of 8 TB/s, half of a 4 TB/s copy
    q = bench.op_record("q", "q", 2e9, [1.0, 1.0, 1.0])
    assert q["GBps"] == 2000.0 and q["frac_hbm"] == 0.25
    g = bench.op_record("g", "g_nv", 1.25e12, [1.0])
    assert g["TFLOPs"] == 1250.0 and g["frac_f16_peak"] == 0.5
    bench.add_copy_frac([q, g], 4000.0)
    assert q["frac_copy"] == 0.5 and "frac_copy" not in g
    # NVFP4 bf16 dual pass: read once (+ once for the amax), two orientations of
    # codes (0.5 B) and E4M3 scales (1/16 B) per element
    assert bench.algorithmic_bytes(1000, 2, 16, True, 2) == 1000 * (2 + 2 * 0.5625 + 2)
