"""Pins of the oracle's router projection and balancing bias update (CPU):
brute-force dot products (math.fsum, correctly rounded), an exact integer
case, the stored [E, H] orientation, hand-worked bias updates, and the
balancing property itself: repeated route -> permute -> update steps on a
skewed router drive the per-expert load towards the mean."""

import math

import numpy as np
import torch

import oracle as O
import synth

RNG = np.random.default_rng(61)
F32 = np.float32


def test_router_logits_bruteforce():
    T, H, E = 5, 37, 7
    x = RNG.standard_normal((T, H)).astype(F32)
    w = RNG.standard_normal((E, H)).astype(F32)
    got, mag = O.router_logits(x, w)
    for t in range(T):
        for e in range(E):
            ref = math.fsum(float(x[t, h]) * float(w[e, h]) for h in range(H))
            assert abs(got[t, e] - ref) <= 1e-13 * mag[t, e]
            assert mag[t, e] == math.fsum(abs(float(x[t, h]) * float(w[e, h])) for h in range(H)) or \
                abs(mag[t, e] - math.fsum(abs(float(x[t, h]) * float(w[e, h])) for h in range(H))) <= 1e-13 * mag[t, e]


def test_router_logits_exact_integers_and_orientation():
    T, H, E = 6, 64, 64
    x = RNG.integers(-9, 10, (T, H)).astype(F32)
    w = RNG.integers(-9, 10, (E, H)).astype(F32)
    got, _ = O.router_logits(x, w)
    ref = [[sum(int(x[t, h]) * int(w[e, h]) for h in range(H)) for e in range(E)] for t in range(T)]
    assert np.array_equal(got, np.array(ref, np.float64))
    # W_r is stored [E, H] (expert rows); read as [H, E] the result differs
    assert not np.array_equal(got, x.astype(np.float64) @ w.astype(np.float64))


def test_bias_update_hand_worked():
    off = np.array([0, 5, 5, 7, 12], np.int32)          # loads 5, 0, 2, 5; mean 3
    b = np.array([0.25, -0.5, 0.0, 1.0], F32)
    g = F32(2.0 ** -8)
    nb = O.bias_update(b, off, g)
    assert nb.dtype == F32
    assert list(nb) == [F32(0.25 - 2 ** -8), F32(-0.5 + 2 ** -8), F32(2 ** -8), F32(1.0 - 2 ** -8)]
    off = np.array([0, 3, 6, 9, 12], np.int32)          # every load at the mean
    assert np.array_equal(O.bias_update(b, off, g), b)
    off = np.array([0, 4, 8, 12], np.int32) + 100       # offsets need not start at 0
    assert np.array_equal(O.bias_update(b[:3], off, g), b[:3])
    off = np.array([0, 1, 3], np.int32)                 # total 3 over 2 experts: mean 1.5
    assert list(O.bias_update(np.zeros(2, F32), off, F32(0.125))) == [0.125, -0.125]


def test_bias_update_balances_a_skewed_router():
    """Skewed router logits (a fixed per-expert offset plus fresh noise each
    step): without the bias the busiest expert carries several times the
    mean load; after a few hundred update steps the load is close to even."""
    T, E, K = 512, 32, 4
    skew = synth.zipf_offsets(E, 1.2, 1.5, seed=7).numpy()
    g = torch.Generator().manual_seed(5)
    b = np.zeros(E, F32)

    def step(bias):
        logits = (torch.randn((T, E), generator=g).numpy() + skew[None, :]).astype(F32)
        idx, _ = O.route_sigmoid_bias(logits, bias, K, True)
        return O.permute(idx, E)["offsets"]

    def imbalance(off):
        load = np.diff(off)
        return load.max() / (T * K / E)

    first = imbalance(step(b))
    hist = []
    for _ in range(300):
        off = step(b)
        hist.append(imbalance(off))
        b = O.bias_update(b, off, F32(2e-3))
    late = float(np.mean(hist[-30:]))
    assert first > 2.5, first
    assert late < 0.5 * first and late < 1.5, (first, late)
    # popular experts (large skew) end with the lowest bias
    assert np.corrcoef(skew, b)[0, 1] < -0.9
