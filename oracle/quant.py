"""Fine-grained FP8 quantisation (oracle; test infrastructure only).

[KANANA-FP8] and [DSV3-FP8]: input activations are quantised per 1x128 tile,
weights per 128x128 block, each tile/block with its own scale.

Readings (the pages give the granularity only):
  * amax = max |x| over the tile or block (exact);
  * scale s = fl32(amax / 448) -- one IEEE binary32 division; s = 1 when
    amax == 0 so that an all-zero tile gets zero codes;
  * code q = E4M3-RNE(clamp(fl32(x / s), -448, 448)) -- a binary32 division,
    then a clamp (rounding of s can push |x/s| a hair above 448), then
    round-to-nearest-even into E4M3FN;
  * dequantised value = decode(q) * s;
  * activation tiles run along the row (the GEMM reduction dimension); weight
    blocks are anchored at (0, 0); dimensions are multiples of 128.
Inputs are float32 arrays (bf16 data is passed as its exact float32 value).
"""

import numpy as np

from .codec import E4M3_MAX, e4m3_decode, e4m3_encode

F32 = np.float32
TILE = 128


def _scale_from_amax(amax):
    """Shared step of both granularities: s = fl32(amax / 448), 1 if amax == 0."""
    s = (amax / F32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, F32(1.0), s).astype(np.float32)
    return s


def quant_act_1x128(x):
    """1x128-tile quantisation of x[rows, cols] -> (codes u8 [rows, cols],
    scales f32 [rows, cols/128]).  [KANANA-FP8], [DSV3-FP8]."""
    x = np.asarray(x, dtype=np.float32)
    rows, cols = x.shape
    if cols % TILE:
        raise ValueError("cols must be a multiple of 128")
    t = x.reshape(rows, cols // TILE, TILE)
    amax = np.max(np.abs(t), axis=2) if rows else np.zeros((0, cols // TILE), np.float32)
    s = _scale_from_amax(amax)
    y = (t / s[:, :, None]).astype(np.float32)
    y = np.clip(y, F32(-E4M3_MAX), F32(E4M3_MAX))
    q = e4m3_encode(y).reshape(rows, cols)
    return q, s


def quant_weight_128x128(w):
    """128x128-block quantisation of w[G, rows, cols] (all experts at once,
    as [KANANA-FP8]'s MoE quantisation kernel does) -> (codes u8
    [G, rows, cols], scales f32 [G, rows/128, cols/128])."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim == 2:
        w = w[None]
    G, rows, cols = w.shape
    if rows % TILE or cols % TILE:
        raise ValueError("rows and cols must be multiples of 128")
    b = w.reshape(G, rows // TILE, TILE, cols // TILE, TILE)
    amax = np.max(np.abs(b), axis=(2, 4))                     # [G, R/128, C/128]
    s = _scale_from_amax(amax)
    y = (b / s[:, :, None, :, None]).astype(np.float32)
    y = np.clip(y, F32(-E4M3_MAX), F32(E4M3_MAX))
    q = e4m3_encode(y).reshape(G, rows, cols)
    return q, s


def dequant_act(q, s):
    """decode(q) * s per 1x128 tile, float64."""
    rows, cols = q.shape
    d = e4m3_decode(q).reshape(rows, cols // TILE, TILE)
    return (d * np.asarray(s, np.float64)[:, :, None]).reshape(rows, cols)


def dequant_weight(q, s):
    """decode(q) * s per 128x128 block, float64."""
    G, rows, cols = q.shape
    d = e4m3_decode(q).reshape(G, rows // TILE, TILE, cols // TILE, TILE)
    d = d * np.asarray(s, np.float64)[:, :, None, :, None]
    return d.reshape(G, rows, cols)
