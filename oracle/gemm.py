"""Block-scaled FP8 grouped GEMM (oracle; test infrastructure only).

[DSV3-FP8]: the expert GEMMs take FP8 operands quantised per 1x128 tile
(activations) and 128x128 block (weights), and accumulate in higher
precision than the FP8 products.  Reading: with the reduction dimension cut
into 128-wide chunks kb,

    C[m, n] = sum_kb  P_kb[m, n] * sa[m, kb] * sb[n // 128, kb],
    P_kb[m, n] = sum_{k in kb} decode(qa[m, k]) * decode(qb[n, k]),

per group g over the rows offsets[g] <= m < offsets[g+1] of A and the g-th
weight matrix B_g stored [N, K] (output features by input features, so the
product is A @ B_g^T).  P_kb is exact in float64: decoded codes are multiples
of 2^-9 below 2^9, so each product is a multiple of 2^-18 below 2^18 and a
sum of 128 of them needs at most 43 bits.  The scale product sa*sb of two
binary32 numbers is exact in float64 too; only the sum over chunks rounds
(float64).  The oracle also returns the magnitude sum
sum_kb |P|_kb * |sa * sb| (with |P| the same sum over |decoded| products),
the natural scale for a componentwise tolerance.
"""

import numpy as np

from .codec import e4m3_decode

TILE = 128


def _group_rows(offsets, G):
    offsets = np.asarray(offsets, dtype=np.int64)
    if len(offsets) != G + 1 or offsets[0] != 0 or np.any(np.diff(offsets) < 0):
        raise ValueError("offsets must be [G+1], start at 0 and be non-decreasing")
    return offsets


def _chunks(Ad, Bd, sa, sb_row, with_mag):
    """sum over 128-wide chunks of P_kb * (sa * sb); Ad [m, K], Bd [N, K]."""
    m, K = Ad.shape
    N = Bd.shape[0]
    C = np.zeros((m, N))
    Mag = np.zeros((m, N)) if with_mag else None
    for kb in range(K // TILE):
        ks = slice(kb * TILE, (kb + 1) * TILE)
        P = Ad[:, ks] @ Bd[:, ks].T                       # exact
        scale = sa[:, kb][:, None] * np.repeat(sb_row[:, kb], TILE)[None, :]
        C += P * scale
        if with_mag:
            Mag += (np.abs(Ad[:, ks]) @ np.abs(Bd[:, ks]).T) * np.abs(scale)
    return C, Mag


def grouped_gemm(aq, as_, bq, bs, offsets, with_mag=True):
    """aq u8 [M, K], as f32 [M, K/128], bq u8 [G, N, K], bs f32
    [G, N/128, K/128], offsets [G+1] -> (C float64 [M, N], Mag or None)."""
    aq = np.asarray(aq)
    M, K = aq.shape
    G, N, K2 = bq.shape
    if K2 != K or K % TILE or N % TILE:
        raise ValueError("shape mismatch or dims not multiples of 128")
    off = _group_rows(offsets, G)
    if off[-1] != M:
        raise ValueError("offsets[G] must equal M")
    C = np.zeros((M, N))
    Mag = np.zeros((M, N)) if with_mag else None
    sa = np.asarray(as_, np.float64)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r1 == r0:
            continue
        Bd = e4m3_decode(bq[g])
        Ad = e4m3_decode(aq[r0:r1])
        c, mg = _chunks(Ad, Bd, sa[r0:r1], np.asarray(bs[g], np.float64), with_mag)
        C[r0:r1] = c
        if with_mag:
            Mag[r0:r1] = mg
    return C, Mag


def grouped_gemm_rows(aq, as_, bq, bs, offsets, rows, with_mag=True):
    """Same as grouped_gemm for the listed rows only (for outputs sampled
    from large problems).  Returns (C [len(rows), N], Mag)."""
    off = _group_rows(offsets, bq.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    grp = np.searchsorted(off, rows, side="right") - 1
    N = bq.shape[1]
    C = np.zeros((len(rows), N))
    Mag = np.zeros((len(rows), N)) if with_mag else None
    sa = np.asarray(as_, np.float64)
    for g in np.unique(grp):
        sel = np.nonzero(grp == g)[0]
        Bd = e4m3_decode(bq[g])
        Ad = e4m3_decode(np.asarray(aq)[rows[sel]])
        c, mg = _chunks(Ad, Bd, sa[rows[sel]], np.asarray(bs[g], np.float64), with_mag)
        C[sel] = c
        if with_mag:
            Mag[sel] = mg
    return C, Mag
