"""Gate-weighted combine of expert outputs (oracle; test infrastructure only).

[DSV3-MOE]: a token's output is the sum of its shared expert's output and its
routed experts' outputs weighted by their gates (the routed experts are the
ones selected for it; every selected pair is kept since no token is dropped).
Readings: the shared expert is added with weight 1; the result is stored as
bfloat16.

Two forms are given:
  combine_ref          the defining value: the sum in float64, rounded once to
                       bf16 (round half to even);
  combine_fp32_replay  the same sum in the binary32 order the GPU library
                       documents (acc = 0; acc = fl32(acc + fl32(g*c)) for
                       k = 0..K-1; acc = fl32(acc + S); bf16), used to check
                       that order bit for bit on an elementwise kernel.
"""

import numpy as np

from .codec import bf16_round

F32 = np.float32


def combine_ref(y_perm, dst_row, gate, shared=None):
    """y_perm [T*K, H] (float64 expert outputs in permuted order), dst_row
    [T, K], gate [T, K], shared [T, H] or None -> (y float64 rounded to bf16
    values, y_bits uint16)."""
    y_perm = np.asarray(y_perm, np.float64)
    dst = np.asarray(dst_row, np.int64)
    g = np.asarray(gate, np.float64)
    T, K = dst.shape
    acc = np.zeros((T, y_perm.shape[1]))
    for k in range(K):
        acc += g[:, k:k + 1] * y_perm[dst[:, k]]
    if shared is not None:
        acc += np.asarray(shared, np.float64)
    return bf16_round(acc)


def combine_fp32_replay(y_perm, dst_row, gate, shared=None):
    """Binary32 replay of the documented GPU order; returns (values, bits)."""
    y_perm = np.asarray(y_perm, np.float32)
    dst = np.asarray(dst_row, np.int64)
    g = np.asarray(gate, np.float32)
    T, K = dst.shape
    acc = np.zeros((T, y_perm.shape[1]), np.float32)
    for k in range(K):
        prod = (g[:, k:k + 1] * y_perm[dst[:, k]]).astype(np.float32)
        acc = (acc + prod).astype(np.float32)
    if shared is not None:
        acc = (acc + np.asarray(shared, np.float32)).astype(np.float32)
    return bf16_round(acc.astype(np.float64))
