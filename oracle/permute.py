"""Per-expert token permutation (oracle; test infrastructure only).

[DSV3-MOE]: no token is dropped, so every (token, slot) pair gets a row.
Each expert's rows are the operand of one group of the grouped GEMM (the role
[PANGU-MOGE]'s page gives its grouped-matmul kernel).  Readings: rows are
grouped by expert in expert order, with no padding and no capacity limit;
inside one expert the rows follow ascending token id.  That is the textbook
stable counting sort of the (expert, token) pairs.
"""

import numpy as np


def permute(topk_idx, E, xq=None, xs=None):
    """-> dict(offsets int32 [E+1], dst_row int32 [T, K], src_token int32
    [T*K], aq u8 [T*K, H] and as f32 [T*K, H/128] when xq/xs are given)."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, K = idx.shape
    counts = np.bincount(idx.ravel(), minlength=E)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    next_free = offsets[:-1].copy()
    dst_row = np.empty((T, K), np.int64)
    for t in range(T):                      # ascending token id
        for k in range(K):
            e = idx[t, k]
            dst_row[t, k] = next_free[e]
            next_free[e] += 1
    src_token = np.empty(T * K, np.int64)
    src_token[dst_row.ravel()] = np.repeat(np.arange(T), K)
    out = dict(offsets=offsets.astype(np.int32), dst_row=dst_row.astype(np.int32),
               src_token=src_token.astype(np.int32))
    if xq is not None:
        out["aq"] = np.asarray(xq)[src_token]
    if xs is not None:
        out["as"] = np.asarray(xs)[src_token]
    return out
