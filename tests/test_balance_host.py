"""Host checks of the forward's balanced dispatch order (balance_one_round), compiled as
host code with hipcc; no GPU needed."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not found")
def test_balance_table_is_a_permutation_and_no_worse(tmp_path):
    exe = str(tmp_path / "balance_check")
    subprocess.run(["hipcc", "-O1", "-x", "hip", "--offload-arch=gfx950", os.path.join(HERE, "host", "balance_check.cpp"),
                    "-o", exe], check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
