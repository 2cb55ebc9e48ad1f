"""Shared helpers of the parity tests: device/host transfers, the tolerance
rules, and the seeded random inputs used by the per-kernel tests."""

import numpy as np
import torch

from oracle import e4m3_decode


def dev():
    return torch.device("cuda:0")


def np_(t):
    """Host numpy copy of a tensor (bf16 becomes its exact float32 value)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def bf16_bits(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev())
    return t if dtype is None else t.to(dtype)


# Tolerance of a block-scaled FP8 GEMM result: "max relative error 1e-4 of the
# float64 accumulation of the same dequantised operands", read componentwise
# against the magnitude sum |A||B| of those operands (the relative error of a
# sum is unbounded under cancellation, so the error is measured against the
# sum of the terms' magnitudes).
GEMM_RTOL = 1e-4

# gfx950's FP8 matrix instruction (V_MFMA_SCALE_F32_16X16X128_F8F6F4) does not
# sum a 128-wide chunk exactly.  Measured with crafted codes
# (test_gpu_wgrad.py::test_fp8_chunk_accumulation_model): it splits the chunk
# into aligned groups of 8 consecutive products (16 groups per chunk) and
# truncates every product of a group toward zero to a multiple of 2^(E - 13),
# E the exponent of the group's largest product (448 + 2^-6 gives 448;
# 448 - 448 + 2^-9 gives 0).  This is the limited accumulation precision the
# per-chunk promotion to float32 answers.  On long reductions of ordinary data
# the truncations average out far below 1e-4 of the magnitude sum; a short
# reduction (a weight gradient over an expert's few rows, mostly zero padding)
# or codes spread over the whole E4M3 range can exceed it, legitimately.  For
# those cases trunc_model_bound gives the per-element bound this model
# implies, and the rule becomes |c - C| <= max(1e-4 |A||B|, model bound).


def trunc_model_bound(A, B, rows_per_block=32):
    """Per-element error bound of a promoted FP8 GEMM C = A . B^T under the
    measured truncation model, from dequantised operand magnitudes A [Na, K]
    and B [Nb, K] (reduction along axis 1, 128-wide chunks from column 0;
    the scales are constant over a chunk for every output, so they ride in
    the dequantised values).

    Per chunk and group of 8 products p_i: each product loses less than
    min(|p_i|, 2^(E - 13) s) with s the chunk's scale product, and
    2^(E - 13) s <= 2^-13 max_i |p_i| (E = floor(log2 of the largest code
    product)), so the group loses at most sum_i min(|p_i|, 2^-13 max_i |p_i|).
    The float32 side adds one rounding of the chunk result, of the scale
    product and of each promotion FMA: (K/128 + 2) 2^-24 |A||B|.  Monotone in
    every |p_i|, so magnitudes that over-estimate the operands (e.g. |A| plus
    the effect of differing codes) still give a valid bound."""
    A, B = np.abs(np.asarray(A, np.float64)), np.abs(np.asarray(B, np.float64))
    Na, K = A.shape
    Nb = B.shape[0]
    KB = K // 128
    out = np.zeros((Na, Nb))
    mag = np.zeros((Na, Nb))
    for r0 in range(0, Na, rows_per_block):
        a = A[r0:r0 + rows_per_block]
        for kb in range(KB):
            pa = a[:, kb * 128:(kb + 1) * 128].reshape(len(a), 1, 16, 8)
            pb = B[:, kb * 128:(kb + 1) * 128].reshape(1, Nb, 16, 8)
            p = pa * pb
            q = p.max(axis=3, keepdims=True) * 2.0 ** -13
            out[r0:r0 + len(a)] += np.minimum(p, q).sum(axis=(2, 3))
            mag[r0:r0 + len(a)] += p.sum(axis=(2, 3))
    return out + (KB + 2) * 2.0 ** -24 * mag


def assert_gemm_close(c_gpu, C, Mag, rtol=GEMM_RTOL, what="gemm", model=None):
    """Componentwise rule for float32 GEMM outputs: |c - C| <= rtol * (|A||B|)
    where (|A||B|) is the oracle's magnitude sum of the same dequantised
    operands.  With `model` (a trunc_model_bound array) the rule is
    |c - C| <= max(rtol |A||B|, model): for short reductions and full-range
    codes, where the matrix instruction's truncation may exceed rtol.  Prints
    and returns the worst observed |c - C| / (|A||B|)."""
    c = np.asarray(c_gpu, np.float64)
    err = np.abs(c - C)
    base = rtol * Mag
    bound = base if model is None else np.maximum(base, model)
    bad = err > bound + 1e-30
    worst = float(np.max(err / (Mag + 1e-300))) if err.size else 0.0
    over = int(np.sum(err > base + 1e-30))
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside the bound; "
                           f"worst |c-C|/(|A||B|) {worst:.3g}")
    print(f"[{what}] worst |c-C|/(|A||B|) = {worst:.3g} over {err.size} elements"
          + (f"; {over} above {rtol:g} (within the truncation model)" if model is not None else ""))
    return worst


def bf16_ulp_distance(a_bits, b_bits):
    """Distance in bf16 units in the last place between two bit patterns
    (ordered integer mapping of the sign-magnitude encoding)."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def e4m3_code_distance(a, b):
    """Distance between E4M3 codes along the number line (adjacent codes -> 1;
    +0 and -0 are the same point)."""
    def ordered(c):
        c = c.astype(np.int32)
        return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)
    return np.abs(ordered(a) - ordered(b))


def dequant_rows(q, s):
    rows, cols = q.shape
    return (e4m3_decode(q).reshape(rows, -1, 128) * s[:, :, None].astype(np.float64)).reshape(rows, cols)


def gemm_model_bound(aq, as_, bq, bs, offsets):
    """trunc_model_bound of a grouped GEMM's rows ([M, N]) from the oracle's
    operands: codes and 1x128 scales of A, block-quantised B per group."""
    from oracle import dequant_weight
    A = dequant_rows(aq, as_)
    out = np.zeros((A.shape[0], bq.shape[1]))
    for g in range(len(offsets) - 1):
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        if r1 > r0:
            out[r0:r1] = trunc_model_bound(A[r0:r1], dequant_weight(bq[g:g + 1], bs[g:g + 1])[0])
    return out


def rand_offsets(rng, sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def check_hidden(hq, hs, C1, Mag1, hq_o, tol=GEMM_RTOL):
    """Validity of GPU FP8 codes/scales of h = silu(g) * u computed from a
    float32 GEMM result, against the oracle's float64 gate|up output C1 and
    its magnitude sums Mag1.

    The GEMM bar allows |g_gpu - g| <= tol * Mag_g (same for u), hence
    |h_gpu - h| <= dh = tol * (|silu(g)| Mag_u + 1.1 |u| Mag_g) (|silu'| <= 1.1)
    plus a few float32 roundings.  The GPU's dequantised h must then lie within
    the quantisation bound of h_gpu (half a code step: 2^-4 |h| for normal
    codes, 2^-10 s for subnormal ones), and each tile scale within dh_max/448
    of the oracle's.  Returns (fraction of codes that differ from the oracle's,
    mask of rows with any differing code)."""
    I = C1.shape[1] // 2
    g, u = C1[:, :I], C1[:, I:]
    silu = g / (1.0 + np.exp(-g))
    h = silu * u
    dh = tol * (np.abs(silu) * Mag1[:, I:] + 1.1 * np.abs(u) * Mag1[:, :I]) + 2.0 ** -20 * np.abs(h)
    srep = np.repeat(np.asarray(hs, np.float64), 128, axis=1)
    deq = dequant_rows(hq, hs)
    bound = 2.0 ** -4 * (np.abs(h) + dh) + 2.0 ** -10 * srep + dh + 1e-300
    assert np.all(np.abs(deq - h) <= bound), f"h outside bound: worst ratio {np.max(np.abs(deq - h) / bound):.3g}"
    rows = h.shape[0]
    amax = np.abs(h).reshape(rows, -1, 128).max(axis=2)
    dmax = dh.reshape(rows, -1, 128).max(axis=2)
    s_o = np.where(amax == 0, 1.0, amax / 448.0)
    assert np.all(np.abs(hs - s_o) <= (dmax / 448.0) * 1.001 + 2.0 ** -22 * s_o), "h scales outside bound"
    diff = hq != hq_o
    return float(diff.mean()), diff.any(axis=1)


class Guarded:
    """A device output buffer of `shape` / `dtype` pre-filled with the byte
    `fill`, between two guard bands of `guard` bytes holding the same byte
    (the tensor starts `guard` bytes into the allocation, so its alignment
    is the allocation's).  Used to catch writes past either end and
    elements a kernel forgets: run the kernel into two buffers filled with
    0x00 and 0xFF; every element it writes agrees, an unwritten one differs."""

    def __init__(self, shape, dtype, fill, guard=4096):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.fill, self.guard, self.n = fill, guard, n
        self.raw = torch.full((2 * guard + n,), fill, dtype=torch.uint8, device=dev())
        self.t = self.raw[guard:guard + n].view(dtype).view(shape)

    def bands_intact(self):
        g = self.guard
        return bool((self.raw[:g] == self.fill).all()) and bool((self.raw[g + self.n:] == self.fill).all())

    def bytes(self):
        return self.raw[self.guard:self.guard + self.n].cpu().numpy()
