"""SwiGLU + 1x128 quantisation of the expert hidden state (oracle; test
infrastructure only).

The pages build on the DeepSeek-V3 FFN ([KANANA-FP8] adopts its
architecture) but do not write the activation down.  Reading: the gate/up
GEMM output row is [g | u] with g the first I columns and u the last I;
h = silu(g) * u with silu(x) = x * sigmoid(x) evaluated by the specified
binary32 sigmoid; h feeds the down-projection GEMM, which runs in FP8 like
the other expert GEMMs ([DSV3-FP8]), so h is quantised in 1x128 tiles along
I.  Each step is a binary32 operation so that the codes are reproducible.
"""

import numpy as np

from .quant import quant_act_1x128
from .specmath import spec_silu


def swiglu_quant(gate_up):
    """gate_up f32 [M, 2I] -> (hq u8 [M, I], hs f32 [M, I/128], h f32 [M, I])."""
    gu = np.asarray(gate_up, dtype=np.float32)
    M, twoI = gu.shape
    I = twoI // 2
    g = gu[:, :I]
    u = gu[:, I:]
    h = (spec_silu(g) * u).astype(np.float32)
    hq, hs = quant_act_1x128(h)
    return hq, hs, h
