"""The matrix-core ceiling probe that bench.py reports beside the datasheet
FP8 peak: its accumulators hold the exact sums its instruction count
implies, so the timed launch really performs the matrix work it is credited
with."""

import numpy as np
import pytest
import torch

import routed_experts_fp8_amd as R
from helpers import np_

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("code,value", [(0x38, 1.0), (0x40, 2.0), (0xB0, -0.5)])
def test_probe_accumulators_are_exact(code, value):
    """E4M3 codes 0x38 = 1, 0x40 = 2, 0xB0 = -0.5: every instruction adds
    128 v^2 to each of a lane's 8 x 4 accumulator elements."""
    iters, blocks, waves = 1000, 3, 8
    out, flops = R.moe_probe_mfma_fp8(iters, blocks, waves, code=code)
    torch.cuda.synchronize()
    want = 8 * 4 * 128 * value * value * iters
    assert want < 2 ** 24
    assert np.all(np_(out) == np.float32(want))
    assert flops == blocks * waves * iters * 8 * 65536


def test_probe_zero_iterations():
    out, flops = R.moe_probe_mfma_fp8(0, 2, 4)
    torch.cuda.synchronize()
    assert np.all(np_(out) == 0) and flops == 0
