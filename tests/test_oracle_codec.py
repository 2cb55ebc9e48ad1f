"""Pins of the oracle's E4M3FN codec and bf16 rounding.

The pins come from outside the oracle: closed forms of the format definition
(field layout, bias 7, 3 mantissa bits, one NaN pattern, max 448), a second
brute-force encoder, hand-worked roundings, and torch's own float8_e4m3fn /
bfloat16 casts (library routines, used on in-range inputs only).
"""

import numpy as np
import pytest
import torch

from oracle import bf16_round, e4m3_decode, e4m3_encode, e4m3_encode_bruteforce, e4m3_values


def _f32(v):
    return np.asarray(v, dtype=np.float32)


def test_decode_closed_forms():
    d = e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x39, 0x77, 0x7E, 0x80, 0xB8, 0xFE], np.uint8))
    expect = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 240.0, 448.0, -0.0, -1.0, -448.0]
    assert np.array_equal(d, np.array(expect))
    assert np.signbit(d[8])
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    allv = e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isfinite(allv).sum() == 254
    pos = e4m3_values()
    assert len(pos) == 127 and np.all(np.diff(pos) > 0) and pos[-1] == 448.0
    # binade structure: 8 values per binade above the subnormals, spacing 2^(e-3)
    for e in range(-6, 9):
        lo = 2.0 ** e
        inb = pos[(pos >= lo) & (pos < 2 * lo)]
        assert len(inb) == (8 if e < 8 else 7)
        assert np.allclose(np.diff(inb), 2.0 ** (e - 3))


def test_encode_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    back = e4m3_encode(e4m3_decode(codes))
    assert np.array_equal(back, codes)


@pytest.mark.parametrize("v,code", [
    (17.0, 0x58),            # 17 between 16 and 18 -> 16 (spacing 2 above 16)
    (19.0, 0x5A),            # tie 18/20 -> 20 (even mantissa)
    (0.53125, 0x30),         # tie 0.5/0.5625 -> 0.5
    (232.0, 0x76),           # tie 224/240 -> 224
    (3 * 2.0 ** -11, 0x01),  # 0.75 * 2^-9 -> 2^-9
    (2.0 ** -10, 0x00),      # tie 0 / 2^-9 -> 0 (even)
    (-1e-9, 0x80),           # negative underflow keeps the sign
    (448.0, 0x7E), (-448.0, 0xFE), (440.0, 0x7E), (431.9, 0x7D),
])
def test_encode_hand_values(v, code):
    assert int(e4m3_encode(_f32(v))) == code


def _boundary_sweep():
    """Every float32 within +-4 ulp of each rounding midpoint and of each
    representable value, both signs, |v| <= 448."""
    pos = e4m3_values()
    mids = (pos[:-1] + pos[1:]) / 2
    centers = np.concatenate([pos, mids]).astype(np.float32)
    bits = centers.view(np.int32)
    offs = np.arange(-4, 5, dtype=np.int32)
    v = (bits[:, None] + offs[None, :]).ravel()
    v = v[v >= 0].view(np.float32)
    v = v[v <= 448.0]
    return np.concatenate([v, -v])


def _bf16_grid():
    b = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    v = b.view(np.float32)
    return v[np.isfinite(v) & (np.abs(v) <= 448.0)]


def test_encode_matches_bruteforce_and_torch():
    rng = np.random.default_rng(0)
    sets = [_boundary_sweep(), _bf16_grid(),
            rng.uniform(-448, 448, 1_000_000).astype(np.float32),
            (rng.standard_normal(200_000) * 2.0 ** rng.integers(-14, 8, 200_000)).clip(-448, 448).astype(np.float32)]
    for v in sets:
        a = e4m3_encode(v)
        assert np.array_equal(a, e4m3_encode_bruteforce(v))
        t = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(a, t)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3_encode(_f32(449.0))
    with pytest.raises(ValueError):
        e4m3_encode(_f32(np.nan))


def test_bf16_round_hand_values():
    one = 1.0
    cases = [
        (one + 2.0 ** -8, one),                         # tie -> even (1.0)
        (one + 3 * 2.0 ** -8, one + 2.0 ** -6),         # tie -> even (mantissa 2)
        (one + 2.0 ** -8 + 2.0 ** -40, one + 2.0 ** -7),  # just above the tie: single rounding goes up
        (-(one + 2.0 ** -8 + 2.0 ** -40), -(one + 2.0 ** -7)),
        (3.0, 3.0), (0.0, 0.0),
    ]
    for v, r in cases:
        got, _ = bf16_round(np.array([v]))
        assert got[0] == r, (v, got[0], r)


def test_bf16_round_matches_torch_on_float32():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(500_000) * 2.0 ** rng.integers(-60, 60, 500_000)).astype(np.float32)
    vals, bits = bf16_round(v.astype(np.float64))
    t = torch.from_numpy(v).to(torch.bfloat16)
    assert np.array_equal(bits, t.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(vals, t.to(torch.float64).numpy())
