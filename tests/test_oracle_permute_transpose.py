"""Pins of the oracle's permutation (equality with a sort of (expert, token)
pairs, bijection, commuting with row-local quantisation, empty experts) and of
the block transpose (element map, involution)."""

import numpy as np
import pytest

from oracle import block_transpose, permute, quant_act_1x128, route_sigmoid_bias

RNG = np.random.default_rng(99)


def _rand_idx(T, E, K, rng=RNG):
    return np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,K", [(1, 4, 2), (37, 16, 4), (300, 64, 8), (20, 6, 6)])
def test_permute_is_sorted_pairs(T, E, K):
    idx = _rand_idx(T, E, K)
    p = permute(idx, E)
    pairs = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K))
    expect_dst = np.empty((T, K), np.int64)
    for pos, (_, t, k) in enumerate(pairs):
        expect_dst[t, k] = pos
    assert np.array_equal(p["dst_row"], expect_dst)
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(np.bincount(idx.ravel(), minlength=E))]))
    assert p["offsets"][-1] == T * K
    assert np.array_equal(np.sort(p["dst_row"].ravel()), np.arange(T * K))      # bijection
    assert np.array_equal(p["src_token"][p["dst_row"]], np.repeat(np.arange(T)[:, None], K, axis=1))
    for e in range(E):
        seg = p["src_token"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)                                      # ascending tokens


def test_permute_empty_experts_and_all_on_few():
    T, E, K = 50, 32, 2
    idx = np.stack([np.array([3, 30])] * T).astype(np.int32)
    p = permute(idx, E)
    counts = np.diff(p["offsets"])
    assert counts[3] == T and counts[30] == T and counts.sum() == T * K
    assert np.all(counts[[e for e in range(E) if e not in (3, 30)]] == 0)


def test_permute_commutes_with_row_quantisation():
    T, E, K, H = 64, 8, 2, 256
    x = RNG.standard_normal((T, H)).astype(np.float32)
    logits = RNG.standard_normal((T, E)).astype(np.float32)
    idx, _ = route_sigmoid_bias(logits, None, K)
    xq, xs = quant_act_1x128(x)
    p = permute(idx, E, xq, xs)
    q2, s2 = quant_act_1x128(x[p["src_token"]])
    assert np.array_equal(p["aq"], q2) and np.array_equal(p["as"], s2)


def test_block_transpose_element_map_and_involution():
    G, R, C = 2, 256, 384
    q = RNG.integers(0, 256, size=(G, R, C)).astype(np.uint8)
    s = RNG.standard_normal((G, R // 128, C // 128)).astype(np.float32)
    qt, st = block_transpose(q, s)
    assert qt.shape == (G, C, R) and st.shape == (G, C // 128, R // 128)
    for _ in range(200):
        g, r, c = RNG.integers(0, G), RNG.integers(0, R), RNG.integers(0, C)
        assert qt[g, c, r] == q[g, r, c]
    assert st[1, 2, 0] == s[1, 0, 2]
    q2, s2 = block_transpose(qt, st)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
