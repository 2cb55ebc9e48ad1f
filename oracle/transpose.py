"""Transpose of block-quantised weights (oracle; test infrastructure only).

[KANANA-FP8]: only the FP8 weights the forward pass needs are kept, and the
backward pass gets the transposed operand by transposing the already
block-quantised weights instead of quantising again.  That is exact because a
128x128 block's amax, and therefore its scale and every x/s, does not depend
on the block's orientation: the codes move, the scale grid transposes.
"""

import numpy as np


def block_transpose(q, s):
    """q u8 [G, rows, cols], s f32 [G, rows/128, cols/128] ->
    (qt u8 [G, cols, rows], st f32 [G, cols/128, rows/128]), bit copies."""
    q = np.asarray(q)
    s = np.asarray(s)
    return np.ascontiguousarray(q.transpose(0, 2, 1)), np.ascontiguousarray(s.transpose(0, 2, 1))
