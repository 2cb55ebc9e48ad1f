"""Pins of the oracle's routing: brute force with Python's sorted on small
inputs (including exact ties), the MoGE invariants (exactly K' picks per group,
equal group loads, Imbalance Score 0), shift invariance of the softmax mode,
scipy's softmax as a library cross-check, and the bias-only-in-selection
reading."""

import numpy as np
import pytest
from scipy.special import softmax

from oracle import imbalance_score, route_sigmoid_bias, route_softmax_grouped, spec_sigmoid

RNG = np.random.default_rng(7)


def _brute_sigmoid(logits, bias, K, normalize):
    T, E = logits.shape
    s = spec_sigmoid(logits)
    idx = np.zeros((T, K), np.int32)
    gate = np.zeros((T, K), np.float32)
    for t in range(T):
        keys = [(np.float32(s[t, e] + bias[e]), e) for e in range(E)]
        top = sorted(keys, key=lambda p: (-float(p[0]), p[1]))[:K]
        idx[t] = [e for _, e in top]
        g = [s[t, e] for _, e in top]
        if normalize:
            tot = np.float32(0)
            for v in g:
                tot = np.float32(tot + v)
            g = [np.float32(v / tot) for v in g]
        gate[t] = g
    return idx, gate


@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("ties", [False, True])
def test_sigmoid_bias_brute_force(normalize, ties):
    T, E, K = 60, 24, 6
    if ties:
        logits = RNG.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(T, E))
        bias = RNG.choice(np.array([0.0, 0.25], np.float32), size=E)
    else:
        logits = RNG.standard_normal((T, E)).astype(np.float32)
        bias = (RNG.standard_normal(E) * 0.3).astype(np.float32)
    idx, gate = route_sigmoid_bias(logits, bias, K, normalize)
    bi, bg = _brute_sigmoid(logits, bias, K, normalize)
    assert np.array_equal(idx, bi)
    assert np.array_equal(gate, bg)


def test_all_equal_logits_pick_lowest_indices():
    logits = np.zeros((5, 16), np.float32)
    idx, gate = route_sigmoid_bias(logits, None, 4, True)
    assert np.array_equal(idx, np.tile(np.arange(4), (5, 1)))
    assert np.all(gate == np.float32(0.25))
    idx2, _ = route_softmax_grouped(logits, 4, 2)
    assert np.array_equal(idx2, np.tile(np.array([0, 1, 4, 5, 8, 9, 12, 13]), (5, 1)))


def test_bias_selects_but_does_not_gate():
    logits = RNG.standard_normal((40, 32)).astype(np.float32)
    bias = np.zeros(32, np.float32)
    bias[17] = 10.0                                     # always selected, first slot
    idx, gate = route_sigmoid_bias(logits, bias, 4, normalize=False)
    assert np.all(idx[:, 0] == 17)
    assert np.array_equal(gate[:, 0], spec_sigmoid(logits[:, 17]))
    _, gn = route_sigmoid_bias(logits, bias, 4, normalize=True)
    assert np.allclose(gn.sum(axis=1), 1.0, atol=1e-6)


def test_sigmoid_invariants():
    T, E, K = 500, 64, 8
    logits = RNG.standard_normal((T, E)).astype(np.float32)
    idx, gate = route_sigmoid_bias(logits, None, K)
    assert all(len(set(r)) == K for r in idx.tolist())
    assert np.bincount(idx.ravel(), minlength=E).sum() == T * K
    # no expert outside the selection has a larger key than a selected one
    s = spec_sigmoid(logits)
    kth = np.take_along_axis(s, idx[:, -1:], axis=1)
    mask = np.ones_like(s, bool)
    np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
    assert np.all(np.where(mask, s, -np.inf) <= kth)


def _brute_grouped(logits, G, Kp):
    T, E = logits.shape
    per = E // G
    p = softmax(logits.astype(np.float64), axis=1)
    idx = []
    for t in range(T):
        row = []
        for g in range(G):
            cand = sorted(range(g * per, (g + 1) * per), key=lambda e: (-float(logits[t, e]), e))
            row += cand[:Kp]
        idx.append(row)
    idx = np.array(idx, np.int32)
    return idx, np.take_along_axis(p, idx.astype(np.int64), axis=1).astype(np.float32)


@pytest.mark.parametrize("G,Kp", [(1, 2), (8, 1), (4, 3)])
def test_softmax_grouped_brute_force(G, Kp):
    T, E = 50, 24
    logits = RNG.standard_normal((T, E)).astype(np.float32)
    logits[::7, 3] = logits[::7, 4]                     # a few exact ties
    idx, gate = route_softmax_grouped(logits, G, Kp)
    bi, bg = _brute_grouped(logits, G, Kp)
    assert np.array_equal(idx, bi)
    assert np.array_equal(gate, bg)


def test_moge_invariants_imbalance_zero():
    T, E, G, Kp = 2048, 64, 8, 1
    logits = (RNG.standard_normal((T, E)) + np.linspace(-3, 3, E)).astype(np.float32)  # skewed scores
    idx, gate = route_softmax_grouped(logits, G, Kp)
    per = E // G
    grp = idx // per
    for g in range(G):
        assert np.all((grp == g).sum(axis=1) == Kp)
    assert imbalance_score(idx, E, G) == 0.0
    # the dense-softmax router is not balanced on the same scores
    idx_dense, _ = route_softmax_grouped(logits, 1, G * Kp)
    assert imbalance_score(idx_dense, E, G) > 0.5
    # unselected experts carry zero score: gates are a subset of the softmax row
    p = softmax(logits.astype(np.float64), axis=1)
    assert np.all(gate.sum(axis=1) <= p.sum(axis=1) + 1e-6)


def test_softmax_shift_invariance():
    logits = RNG.standard_normal((100, 32)).astype(np.float32)
    i0, g0 = route_softmax_grouped(logits, 4, 2)
    shift = np.float32(0.5) * (np.arange(100) % 5).astype(np.float32)[:, None]
    i1, g1 = route_softmax_grouped((logits + shift).astype(np.float32), 4, 2)
    assert np.array_equal(i0, i1)
    assert np.allclose(g0, g1, rtol=2e-6, atol=0)


def test_route_errors():
    with pytest.raises(ValueError):
        route_sigmoid_bias(np.zeros((2, 4), np.float32), None, 5)
    with pytest.raises(ValueError):
        route_softmax_grouped(np.zeros((2, 6), np.float32), 4, 1)
