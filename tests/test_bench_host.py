"""Host-side behaviour of bench.py that needs no GPU: it measures one GPU only and says so
when asked for more, and its kernel-source hash (which gates the stored traffic figures)
is a stable 64-bit hex digest."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""


def test_kernel_source_hash_is_stable_and_hex():
    h1, h2 = bench.kernel_source_hash(), bench.kernel_source_hash()
    assert h1 == h2 and len(h1) == 16
    int(h1, 16)
