"""Pins of the oracle's plain C forms (oracle/oracle_c.c through
oracle/native.py): bit-identical to the numpy oracle they restate, and
checked directly against the E4M3 format's closed forms, the quantiser's
invariants and exact integer GEMMs."""

import numpy as np
import pytest

import oracle as O
from oracle import native as N

RNG = np.random.default_rng(1234)
F32 = np.float32


def test_encoder_closed_forms():
    # fields: sign, exponent + 7 (bias 7), 3 mantissa bits; exponent field 0
    # holds m * 2^-9; ties go to the even mantissa
    v = np.array([448.0, -448.0, 2.0 ** -9, 2.0 ** -6, 0.0, -0.0, 1.0, 17.0, 19.0, 0.53125, 440.0,
                  3 * 2.0 ** -11, 2.0 ** -10, -1e-9, 240.0, 256.0])
    want = np.array([0x7E, 0xFE, 0x01, 0x08, 0x00, 0x80, 0x38, 0x58, 0x5A, 0x30, 0x7E,
                     0x01, 0x00, 0x80, 0x77, 0x78], np.uint8)
    assert np.array_equal(N.e4m3_encode(v), want)
    # every finite code decodes and re-encodes to itself
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(N.e4m3_encode(O.e4m3_decode(codes)), codes)


def test_encoder_matches_numpy_and_bruteforce_near_every_code_and_midpoint():
    vals = O.e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(F32)
    bits = pts.view(np.int32)
    near = np.concatenate([bits + d for d in range(-4, 5)]).view(F32).astype(np.float64)
    near = near[np.isfinite(near) & (np.abs(near) <= 448.0) & (near >= 0)]
    near = np.concatenate([near, -near])
    c = N.e4m3_encode(near)
    assert np.array_equal(c, O.e4m3_encode(near))
    assert np.array_equal(c, O.e4m3_encode_bruteforce(near))
    with pytest.raises(ValueError):
        N.e4m3_encode(np.array([449.0]))


def test_weight_quant_matches_numpy():
    w = (RNG.standard_normal((3, 256, 384)) * np.exp2(RNG.integers(-20, 20, (3, 256, 1)))).astype(F32)
    w[1, :128, 128:256] = 0.0                                   # an all-zero block -> s = 1, codes 0
    w[2, 5, 7] = -0.0
    w[0, 3, 3] = 1e-42                                          # a subnormal input
    q, s = N.quant_weight_128x128(w)
    qo, so = O.quant_weight_128x128(w)
    assert np.array_equal(q, qo) and np.array_equal(s, so)
    assert s[1, 0, 1] == 1.0 and not q[1, :128, 128:256].any()


def test_weight_quant_invariants():
    w = (RNG.standard_normal((2, 128, 256)) * 0.02).astype(F32)
    q, s = N.quant_weight_128x128(w)
    # every block holds the largest code (its amax maps to 448)
    blocks = (q & 0x7F).reshape(2, 1, 128, 2, 128)
    assert np.all(blocks.max(axis=(2, 4)) == 0x7E)
    # power-of-two invariance: same codes, scales times 2^k exactly
    q2, s2 = N.quant_weight_128x128(w * F32(2.0 ** 7))
    assert np.array_equal(q2, q) and np.array_equal(s2, s * F32(2.0 ** 7))
    # dequantised values within half a code step of the input
    deq = O.dequant_weight(q, s)
    step = np.repeat(np.repeat(s, 128, axis=1), 128, axis=2).astype(np.float64)
    assert np.all(np.abs(deq - w) <= 2.0 ** -4 * np.abs(w) + 2.0 ** -10 * step + 1e-30)


def test_gemm_rows_matches_numpy_bit_for_bit():
    M, Nn, K = 7, 256, 512
    a = (RNG.standard_normal((M, K)) * np.exp2(RNG.integers(-6, 6, (M, 1)))).astype(F32)
    aq, as_ = O.quant_act_1x128(a)
    bq, bs = O.quant_weight_128x128((RNG.standard_normal((1, Nn, K)) * 0.02).astype(F32))
    C, Mag = N.gemm_rows(aq, as_, bq[0], bs[0])
    Co, Mo = O.grouped_gemm(aq, as_, bq, bs, np.array([0, M], np.int32))
    assert np.array_equal(C, Co) and np.array_equal(Mag, Mo)
    C2, none = N.gemm_rows(aq, as_, bq[0], bs[0], with_mag=False)
    assert none is None and np.array_equal(C2, C)


def test_gemm_rows_exact_integers_and_scaling():
    M, Nn, K = 5, 128, 384
    a = RNG.integers(-8, 9, (M, K)).astype(np.float64)
    b = RNG.integers(-8, 9, (Nn, K)).astype(np.float64)
    aq, bq = O.e4m3_encode(a), O.e4m3_encode(b)
    ones_a, ones_b = np.ones((M, K // 128), F32), np.ones((1, K // 128), F32)
    C, Mag = N.gemm_rows(aq, ones_a, bq, ones_b)
    assert np.array_equal(C, a @ b.T) and np.array_equal(Mag, np.abs(a) @ np.abs(b).T)
    # a power-of-two activation scale scales the result exactly
    C4, _ = N.gemm_rows(aq, ones_a * F32(4.0), bq, ones_b)
    assert np.array_equal(C4, 4.0 * C)
    # a transposed operand is not the same product
    Ct, _ = N.gemm_rows(aq, ones_a, bq[::-1].copy(), ones_b)
    assert not np.array_equal(Ct, C)


def test_sigmoid_matches_numpy_spec():
    """The C sigmoid equals specmath.spec_sigmoid bit for bit: 4M random bit
    patterns (every binade, both signs, infinities), every binary32 in
    [0.5, 0.5 + 2^-3) and around the clamp at |x| = 80; the bit-pattern form
    equals the value form."""
    from oracle.specmath import spec_sigmoid
    b = RNG.integers(0, 2 ** 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    x = b.view(F32)
    x = x[~np.isnan(x)]
    dense = (np.arange(1 << 20, dtype=np.uint32) + np.float32(0.5).view(np.uint32)).view(F32)
    clamp = np.concatenate([(np.arange(-4096, 4096) + np.float32(80.0).view(np.int32)).astype(np.int32).view(F32),
                            np.array([np.inf, -np.inf, 0.0, -0.0, 1e-45, -1e-45, 87.0, -87.0, 1e30, -1e30], F32)])
    clamp = np.concatenate([clamp, -clamp])
    for v in (x, dense, clamp):
        assert np.array_equal(N.spec_sigmoid(v).view(np.uint32), spec_sigmoid(v).view(np.uint32))
    start = int(np.float32(-3.0).view(np.uint32))
    got = N.spec_sigmoid_bits(start, 1 << 16)
    xs = (np.arange(1 << 16, dtype=np.uint64) + start).astype(np.uint32).view(F32)
    assert np.array_equal(got.view(np.uint32), N.spec_sigmoid(xs).view(np.uint32))
    # the specification itself: sigmoid(0) = 1/2, within 4 ulp of the float64 sigmoid
    assert N.spec_sigmoid(np.array([0.0], F32))[0] == 0.5
    xm = x[np.abs(x) < 80]
    ref = 1.0 / (1.0 + np.exp(-xm.astype(np.float64)))
    ulp = np.spacing(ref.astype(F32)).astype(np.float64)
    assert np.all(np.abs(N.spec_sigmoid(xm) - ref) <= 4 * ulp)
