"""Weight gradients of the expert GEMMs in FP8 (oracle; test infrastructure
only).

[DSV3-FP8]: most GEMMs of training, forward and backward, take FP8 operands
with fine-grained (1x128 / 128x128) scaling and promoted accumulation.  For
the weight gradient of an expert GEMM the reduction runs over that expert's
tokens, so the activation-style tiles have to lie along the token
dimension.  The pages give no more than that; the readings taken here:

* Weight gradient of expert g for a layer out = in . W_g^T (W_g stored
  [out, in]):  dW_g[o, i] = sum over the expert's rows r of dOut[r, o] *
  In[r, i].  For the gate|up weights In = x (row src_token[r]) and
  dOut = dC1 = [dg | du]; for the down weights In = h and dOut = dC2.
* Both operands are quantised in 128x1 tiles: 128 consecutive rows of one
  expert in one column.  Each expert's rows are cut into tiles from its first
  row and the last tile is padded with zero rows (which add nothing), so no
  tile spans two experts.  Scale and code rules are the 1x128 quantiser's
  (s = fl32(amax / 448), 1 for an all-zero tile; code = RNE(clamp(x / s))).
* The operands are stored transposed, [column, padded row], so that both are
  contiguous along the reduction dimension as in the forward GEMM; expert g
  owns the padded rows [P_g, P_{g+1}) with P_g = sum over g' < g of
  128 * ceil(M_g' / 128).
* The values quantised are the high-precision ones: x as given (bf16), h =
  fl32(silu(g) * u) of the forward's float32 gate|up output, dC1 in float32
  from the SwiGLU backward, dC2 = fl32(gate * dy).
* The GEMM: dW_g[o, i] = sum over 128-row chunks kb of
  P_kb[o, i] * sa[o, kb] * sb[i, kb] with P_kb the exact dot product of the
  decoded codes over the chunk (float64 here; the scales of both operands
  now vary along both output axes).
"""

import numpy as np

from .codec import e4m3_decode
from .quant import quant_act_1x128

TILE = 128
F32 = np.float32


def padded_offsets(offsets):
    """[G+1] group offsets -> [G+1] offsets of the groups' 128-row padded
    ranges (each group rounded up to whole 128-row tiles)."""
    off = np.asarray(offsets, np.int64)
    sizes = np.diff(off)
    p = np.zeros(len(off), np.int64)
    p[1:] = np.cumsum((sizes + TILE - 1) // TILE * TILE)
    return p.astype(np.int32)


def grouped_rows(x, offsets, row_index=None, row_scale=None):
    """The grouped operand before quantisation, in padded layout:
    V [Mp, C] float32 with V[P_g + j] = fl32(row_scale[r] * x[row_index[r]])
    for r = offsets[g] + j (or x[r], unscaled), zero rows in the padding."""
    x = np.asarray(x, np.float32)
    off = np.asarray(offsets, np.int64)
    p = padded_offsets(off)
    M = int(off[-1])
    rows = np.arange(M) if row_index is None else np.asarray(row_index, np.int64)
    vals = x[rows]
    if row_scale is not None:
        vals = (np.asarray(row_scale, np.float32)[:, None] * vals).astype(np.float32)
    V = np.zeros((int(p[-1]), x.shape[1]), np.float32)
    for g in range(len(off) - 1):
        n = int(off[g + 1] - off[g])
        V[p[g]:p[g] + n] = vals[off[g]:off[g] + n]
    return V


def quant_act_128x1_grouped(x, offsets, row_index=None, row_scale=None):
    """128x1-tile quantisation of the grouped operand (see ``grouped_rows``)
    -> (qt u8 [C, Mp], st f32 [C, Mp/128], padded offsets int32 [G+1]).

    The padded operand transposed, [C, Mp], has its 128x1 tiles along rows,
    and every group starts at a multiple of 128: the tiles are exactly the
    1x128 tiles of that transposed matrix."""
    V = grouped_rows(x, offsets, row_index, row_scale)
    qt, st = quant_act_1x128(np.ascontiguousarray(V.T))
    return qt, st, padded_offsets(offsets)


def wgrad_gemm(aq, as_, bq, bs, poff, with_mag=True):
    """aq u8 [Na, Mp], as f32 [Na, Mp/128] (the output-gradient operand),
    bq u8 [Nb, Mp], bs f32 [Nb, Mp/128] (the input operand), poff [G+1]
    padded offsets -> (dW float64 [G, Na, Nb], magnitude sum or None).
    An empty group's gradient is zero."""
    aq, bq = np.asarray(aq), np.asarray(bq)
    sa, sb = np.asarray(as_, np.float64), np.asarray(bs, np.float64)
    p = np.asarray(poff, np.int64)
    G = len(p) - 1
    Na, Nb = aq.shape[0], bq.shape[0]
    if aq.shape[1] != bq.shape[1] or p[-1] > aq.shape[1] or np.any(p % TILE):
        raise ValueError("operands must share the padded row axis; offsets multiples of 128")
    C = np.zeros((G, Na, Nb))
    Mag = np.zeros((G, Na, Nb)) if with_mag else None
    for g in range(G):
        for kb in range(p[g] // TILE, p[g + 1] // TILE):
            ks = slice(kb * TILE, (kb + 1) * TILE)
            A = e4m3_decode(aq[:, ks])
            B = e4m3_decode(bq[:, ks])
            scale = sa[:, kb][:, None] * sb[:, kb][None, :]
            C[g] += (A @ B.T) * scale                    # chunk product exact
            if with_mag:
                Mag[g] += (np.abs(A) @ np.abs(B).T) * np.abs(scale)
    return C, Mag


def layer_wgrad(fwd, bwd, x, dy, shared=None):
    """Weight gradients of the routed experts (and the shared expert) from
    the oracle's forward and input-side backward (dicts of ``layer_forward``
    and ``layer_backward``), x f32 [T, H], dy f32 [T, H] (bf16 values).

    Returns dict(dw13 [E, 2I, H], dw2 [E, H, I] float64, with magnitude sums,
    the quantised operands, and shared_dw13 / shared_dw2 when shared)."""
    from .swiglu import swiglu_quant
    off = fwd["offsets"]
    src = fwd["src_token"]
    dst = fwd["dst_row"]
    T, K = dst.shape
    # down projection: dOut = dC2 rows (gate * dy of the row's token, the
    # combine backward's float32 product), In = h
    gate_row = np.zeros(T * K, np.float32)
    gate_row[dst.ravel()] = np.asarray(fwd["topk_gate"], np.float32).ravel()
    dc2q, dc2s, _ = quant_act_128x1_grouped(dy, off, src, gate_row)
    _, _, h = swiglu_quant(fwd["c1"].astype(np.float32))
    hq, hs, poff = quant_act_128x1_grouped(h, off)
    dw2, mag2 = wgrad_gemm(dc2q, dc2s, hq, hs, poff)
    # gate|up projection: dOut = dC1 = [dg | du], In = x (row src_token)
    d1q, d1s, _ = quant_act_128x1_grouped(bwd["d1"], off)
    xq, xs, _ = quant_act_128x1_grouped(x, off, src)
    dw13, mag13 = wgrad_gemm(d1q, d1s, xq, xs, poff)
    out = dict(poff=poff, dc2q=dc2q, dc2s=dc2s, hq=hq, hs=hs, d1q=d1q, d1s=d1s, xq=xq, xs=xs,
               dw2=dw2, mag_dw2=mag2, dw13=dw13, mag_dw13=mag13)
    if shared is not None:
        one = np.array([0, T], np.int32)
        sdq, sds, _ = quant_act_128x1_grouped(dy, one)
        _, _, sh = swiglu_quant(fwd["shared_c1"].astype(np.float32))
        shq, shs, sp = quant_act_128x1_grouped(sh, one)
        sdw2, smag2 = wgrad_gemm(sdq, sds, shq, shs, sp)
        s1q, s1s, _ = quant_act_128x1_grouped(bwd["shared_d1"], one)
        sxq, sxs, _ = quant_act_128x1_grouped(x, one)
        sdw13, smag13 = wgrad_gemm(s1q, s1s, sxq, sxs, sp)
        out.update(shared_dw2=sdw2, shared_mag_dw2=smag2, shared_dw13=sdw13, shared_mag_dw13=smag13,
                   shared_dyq=sdq, shared_dys=sds, shared_hq=shq, shared_hs=shs, shared_d1q=s1q,
                   shared_d1s=s1s, shared_xq=sxq, shared_xs=sxs)
    return out
