"""Pins of the oracle's FP8 weight gradient (CPU): a brute-force 128x1
quantiser written with loops and the second (table-scan) E4M3 encoder, group
isolation of the tiles, the gradient against the unquantised float64 product
within the operands' quantisation bound, an exact small-integer case, and the
whole layer's weight gradients against torch float64 autograd."""

import numpy as np
import pytest
import torch

import oracle as O
import synth
from oracle import e4m3_decode, e4m3_encode_bruteforce

RNG = np.random.default_rng(31)
F32 = np.float32


def _groups(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def test_padded_offsets():
    assert list(O.padded_offsets(_groups([0, 1, 128, 129, 0, 300]))) == [0, 0, 128, 256, 512, 512, 896]


def test_quant_128x1_bruteforce():
    """Tiles of 128 rows of one group in one column, written out with loops:
    amax, s = fl32(amax/448), the table-scan encoder of fl32(v/s) clamped."""
    sizes = [5, 0, 130, 1, 128]
    off = _groups(sizes)
    C = 6
    R = 400
    x = (RNG.standard_normal((R, C)) * np.exp2(RNG.integers(-6, 6, (R, 1)))).astype(F32)
    x[0, 0] = 0.0
    x[3, 1] = -0.0
    M = off[-1]
    idx = RNG.integers(0, R, M).astype(np.int32)
    scale = RNG.uniform(0.1, 1.0, M).astype(F32)
    qt, st, poff = O.quant_act_128x1_grouped(x, off, idx, scale)
    assert qt.shape == (C, poff[-1]) and st.shape == (C, poff[-1] // 128)
    seen = np.zeros(qt.shape, bool)
    for g in range(len(sizes)):
        n = sizes[g]
        for j0 in range(0, n, 128):
            rows = range(j0, min(j0 + 128, n))
            for c in range(C):
                vals = [F32(scale[off[g] + j]) * x[idx[off[g] + j], c] for j in rows]
                amax = max(abs(float(v)) for v in vals)
                s = F32(1.0) if amax == 0 else F32(F32(amax) / F32(448))
                kb = (poff[g] + j0) // 128
                assert st[c, kb] == s
                for j, v in zip(rows, vals):
                    y = np.clip(F32(F32(v) / s), F32(-448), F32(448))
                    assert qt[c, poff[g] + j] == e4m3_encode_bruteforce(np.array([y]))[0]
                    seen[c, poff[g] + j] = True
    assert np.all(qt[~seen] == 0)                 # padding rows: +0 codes


def test_quant_128x1_groups_are_isolated():
    """Scaling one group's rows by 2^5 scales only that group's tile scales
    (codes unchanged): no tile reaches across an expert boundary."""
    sizes = [70, 200, 3]
    off = _groups(sizes)
    x = RNG.standard_normal((off[-1], 256)).astype(F32)
    q1, s1, p = O.quant_act_128x1_grouped(x, off)
    x2 = x.copy()
    x2[off[1]:off[2]] *= F32(32)
    q2, s2, _ = O.quant_act_128x1_grouped(x2, off)
    assert np.array_equal(q1, q2)
    kb = np.arange(s1.shape[1])
    in_g1 = (kb * 128 >= p[1]) & (kb * 128 < p[2])
    assert np.array_equal(s2[:, in_g1], s1[:, in_g1] * F32(32))
    assert np.array_equal(s2[:, ~in_g1], s1[:, ~in_g1])
    # a 1x128 quantisation of the ungrouped rows along the same axis differs
    # (tiles would straddle the expert boundary at row 70)
    qn, sn = O.quant_act_1x128(np.ascontiguousarray(np.pad(x, ((0, 384 - len(x)), (0, 0))).T))
    assert not np.array_equal(sn[:, :1], s1[:, :1])


def _operands(sizes, Na, Nb, rng=RNG):
    off = _groups(sizes)
    M = off[-1]
    dout = (rng.standard_normal((M, Na)) * np.exp2(rng.integers(-4, 4, (M, 1)))).astype(F32)
    inp = rng.standard_normal((M, Nb)).astype(F32)
    aq, as_, p = O.quant_act_128x1_grouped(dout, off)
    bq, bs, _ = O.quant_act_128x1_grouped(inp, off)
    return off, dout, inp, aq, as_, bq, bs, p


def _deq(q, s):
    return e4m3_decode(q) * np.repeat(np.asarray(s, np.float64), 128, axis=1)


@pytest.mark.parametrize("sizes,Na,Nb", [([5, 0, 300, 1], 256, 384), ([128], 128, 128), ([0, 0], 128, 256)])
def test_wgrad_against_unquantised_product(sizes, Na, Nb):
    """dW_g = sum_r dOut[r]^T In[r]: the FP8 result equals the float64 product
    of the dequantised operands (a different formula: dequantise, then one
    matmul per group) and lies within the quantisation bound of the exact
    product of the unquantised operands."""
    off, dout, inp, aq, as_, bq, bs, p = _operands(sizes, Na, Nb)
    dW, Mag = O.wgrad_gemm(aq, as_, bq, bs, p)
    A, B = _deq(aq, as_), _deq(bq, bs)
    for g in range(len(sizes)):
        ref = A[:, p[g]:p[g + 1]] @ B[:, p[g]:p[g + 1]].T
        assert np.all(np.abs(dW[g] - ref) <= 1e-13 * Mag[g] + 1e-300)
        exact = dout[off[g]:off[g + 1]].astype(np.float64).T @ inp[off[g]:off[g + 1]].astype(np.float64)
        # per element |v^ - v| <= 2^-4 |v| (normal codes) + 2^-10 s (subnormal step / 2)
        ea = 2.0 ** -4 * np.abs(A[:, p[g]:p[g + 1]]) + 2.0 ** -10 * np.repeat(as_, 128, 1)[:, p[g]:p[g + 1]]
        eb = 2.0 ** -4 * np.abs(B[:, p[g]:p[g + 1]]) + 2.0 ** -10 * np.repeat(bs, 128, 1)[:, p[g]:p[g + 1]]
        bound = ea @ (np.abs(B[:, p[g]:p[g + 1]]) + eb).T + np.abs(A[:, p[g]:p[g + 1]]) @ eb.T
        assert np.all(np.abs(dW[g] - exact) <= 1.01 * bound + 1e-300)
        if sizes[g] == 0:
            assert np.all(dW[g] == 0)
    # swapping the operands gives the transposed gradient
    if Na != Nb and sum(sizes):
        dT, _ = O.wgrad_gemm(bq, bs, aq, as_, p, with_mag=False)
        assert np.array_equal(dT, np.transpose(dW, (0, 2, 1)))


def test_wgrad_exact_small_integers():
    """Integers in [-7, 7] with a 7 in every tile: s = 7/448 = 2^-6 exactly and
    64 v is an E4M3 value for each of them, so the quantisation is exact and
    the gradient is the exact integer product."""
    sizes = [3, 130]
    off = _groups(sizes)
    M = off[-1]
    ia = RNG.integers(-7, 8, (M, 128)).astype(F32)
    ib = RNG.integers(-7, 8, (M, 256)).astype(F32)
    for g in range(2):
        for j0 in range(0, sizes[g], 128):
            ia[off[g] + j0] = 7
            ib[off[g] + j0] = -7
    aq, as_, p = O.quant_act_128x1_grouped(ia, off)
    bq, bs, _ = O.quant_act_128x1_grouped(ib, off)
    # codes times scales reproduce the integers exactly
    assert np.all(as_ == F32(2.0 ** -6)) and np.all(bs == F32(2.0 ** -6))
    assert np.array_equal(_deq(aq, as_)[:, p[1]:p[1] + 130], ia[3:].T)
    dW, _ = O.wgrad_gemm(aq, as_, bq, bs, p, with_mag=False)
    for g in range(2):
        r = slice(off[g], off[g + 1])
        exact = [[sum(int(ia[m, o]) * int(ib[m, i]) for m in range(off[g], off[g + 1])) for i in range(0, 256, 37)]
                 for o in range(0, 128, 29)]
        assert np.array_equal(dW[g][::29, ::37], np.array(exact, np.float64)), g
        assert np.array_equal(dW[g], ia[r].astype(np.float64).T @ ib[r].astype(np.float64))


def _tiny_case(name):
    cfg = synth.get_config("tiny")
    if name == "sigmoid_shared":
        cfg.update(T=64, E=8, K=2, I=256, route=dict(mode="sigmoid_bias", K=2, normalize=True),
                   bias_std=0.01, shared_I=256)
    else:
        cfg.update(T=64)
    return cfg


@pytest.mark.parametrize("name", ["tiny_softmax", "sigmoid_shared"])
def test_layer_wgrad_vs_autograd(name):
    """The oracle's FP8 weight gradients against torch float64 autograd of the
    same layer with the dequantised weights as leaves (routing and gates held
    at the oracle's): the FP8 operands move each gradient by a few percent at
    most, and the gradients stay aligned."""
    cfg = _tiny_case(name)
    d = synth.layer_inputs(cfg, torch.device("cpu"), seed=3)
    x, logits = d["x"].float().numpy(), d["logits"].numpy()
    bias = None if d["bias"] is None else d["bias"].numpy()
    w13q, w13s = O.quant_weight_128x128(d["w13"].float().numpy())
    w2q, w2s = O.quant_weight_128x128(d["w2"].float().numpy())
    shared = None
    if cfg.get("shared_I"):
        a, b = O.quant_weight_128x128(d["sw13"].float().numpy())
        c, e = O.quant_weight_128x128(d["sw2"].float().numpy())
        shared = (a, b, c, e)
    fwd = O.layer_forward(x, logits, bias, cfg["route"], w13q, w13s, w2q, w2s, shared=shared)
    dy = O.bf16_round(RNG.standard_normal(x.shape))[0].astype(F32)
    bwd = O.layer_backward(fwd, dy, logits, cfg["route"], w13q, w13s, w2q, w2s, shared=shared)
    wg = O.layer_wgrad(fwd, bwd, x, dy, shared=shared)

    E, I = cfg["E"], cfg["I"]
    W13 = torch.from_numpy(O.dequant_weight(w13q, w13s)).requires_grad_(True)
    W2 = torch.from_numpy(O.dequant_weight(w2q, w2s)).requires_grad_(True)
    xt = torch.from_numpy(x.astype(np.float64))
    idx = torch.from_numpy(fwd["topk_idx"].astype(np.int64))
    gate = torch.from_numpy(fwd["topk_gate"].astype(np.float64))
    T, K = idx.shape
    y = torch.zeros_like(xt)
    for k in range(K):
        for e in range(E):
            rows = (idx[:, k] == e).nonzero().flatten()
            if len(rows) == 0:
                continue
            c1 = xt[rows] @ W13[e].T
            h = torch.nn.functional.silu(c1[:, :I]) * c1[:, I:]
            y = y.index_add(0, rows, gate[rows, k:k + 1] * (h @ W2[e].T))
    leaves = [W13, W2]
    if shared is not None:
        S13 = torch.from_numpy(O.dequant_weight(shared[0], shared[1])).requires_grad_(True)
        S2 = torch.from_numpy(O.dequant_weight(shared[2], shared[3])).requires_grad_(True)
        c1 = xt @ S13[0].T
        Is = S13.shape[1] // 2
        y = y + (torch.nn.functional.silu(c1[:, :Is]) * c1[:, Is:]) @ S2[0].T
        leaves += [S13, S2]
    grads = torch.autograd.grad((y * torch.from_numpy(dy.astype(np.float64))).sum(), leaves)
    pairs = [(wg["dw13"], grads[0]), (wg["dw2"], grads[1])]
    if shared is not None:
        pairs += [(wg["shared_dw13"], grads[2]), (wg["shared_dw2"], grads[3])]
    for got, ref in pairs:
        ref = ref.numpy()
        err = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        cos = np.sum(got * ref) / (np.linalg.norm(got) * np.linalg.norm(ref))
        assert err < 0.1 and cos > 0.995, (err, cos)
    # experts that received no rows get exactly zero gradient
    empty = np.diff(fwd["offsets"]) == 0
    assert np.all(wg["dw13"][empty] == 0) and np.all(wg["dw2"][empty] == 0)
