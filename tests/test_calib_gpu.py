"""The matrix-core calibration kernel: its products are exact (every operand 1/64, so
each thread's sum is iters / 64), its flop count is the launch's, and its clock readout
is a plausible shader clock."""
import pytest

import causal_gqa_flash_amd as cg

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("blocks,iters", [(1, 1), (8, 1000), (300, 64)])
def test_calibration_products_and_clock(blocks, iters):
    import torch
    sink, clocks, flops = cg.calib_mfma(blocks, iters)
    torch.cuda.synchronize()
    assert bool((sink == iters / 64.0).all())
    assert flops == blocks * 4 * 4 * iters * 2 * 32 * 32 * 16
    sh, rt = clocks.cpu().tolist()
    assert sh > 0 and rt > 0
    if iters >= 1000:
        ghz = sh / (rt * 1e-8) / 1e9
        assert 0.5 < ghz < 3.5, ghz
