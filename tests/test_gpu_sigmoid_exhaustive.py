"""The GPU's binary32 sigmoid against the oracle's specification on every
binary32 input: all 2^32 bit patterns except NaNs (both signs, zeros,
subnormals, the clamped regions beyond |x| = 80 and the infinities), bit
for bit.  Routing turns the sigmoid into an integer decision (DeepSeek-V3
page section 2.1: sigmoid affinity, then top-K), so its bit-exactness rests
on this equality.  The oracle side is the plain C form of
oracle.spec_sigmoid (held to the numpy form by tests/test_oracle_native.py)."""

import numpy as np
import pytest
import torch

import routed_experts_fp8_amd as R
from helpers import dev
from oracle import native as N

pytestmark = pytest.mark.gpu

CHUNK = 1 << 26


@pytest.mark.timeout(900)
def test_sigmoid_every_binary32_input():
    base = torch.arange(CHUNK, dtype=torch.int64, device=dev())
    y = torch.empty(CHUNK, dtype=torch.float32, device=dev())
    compared = 0
    for c in range((1 << 32) // CHUNK):
        start = c * CHUNK
        bits = ((base + start) & 0xFFFFFFFF).to(torch.int64)
        bits = torch.where(bits >= (1 << 31), bits - (1 << 32), bits).to(torch.int32)
        x = bits.view(torch.float32)
        R.moe_sigmoid_f32(x, y=y)
        got = y.view(torch.int32).cpu().numpy().view(np.uint32)
        want = N.spec_sigmoid_bits(start, CHUNK).view(np.uint32)
        xb = (np.arange(CHUNK, dtype=np.uint64) + start).astype(np.uint32)
        finite_or_inf = (xb & 0x7F800000) != 0x7F800000
        finite_or_inf |= (xb & 0x007FFFFF) == 0                 # +-inf
        bad = (got != want) & finite_or_inf
        assert not bad.any(), (f"chunk {c}: {int(bad.sum())} mismatches, first x bits "
                               f"{int(xb[np.argmax(bad)]):#010x}")
        compared += int(finite_or_inf.sum())
    print(f"sigmoid: {compared} binary32 inputs compared bit for bit, 0 mismatches")
    assert compared == (1 << 32) - 2 * ((1 << 23) - 1)
