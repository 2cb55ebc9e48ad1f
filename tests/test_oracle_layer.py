"""Pins of the oracle's SwiGLU, combine and whole-layer composition: float64
formulas, closed forms (silu(0) = 0, u = 0, K = 1 identity), torch's bf16 cast,
and the permuted layer against a token-by-token evaluation with no
permutation at all."""

import numpy as np
import pytest
import torch

import synth
from oracle import (combine_fp32_replay, combine_ref, layer_forward, layer_forward_dense,
                    quant_weight_128x128, swiglu_quant)

RNG = np.random.default_rng(11)


def test_swiglu_matches_float64_formula():
    M, I = 64, 256
    gu = (RNG.standard_normal((M, 2 * I)) * 2).astype(np.float32)
    hq, hs, h = swiglu_quant(gu)
    g = gu[:, :I].astype(np.float64)
    u = gu[:, I:].astype(np.float64)
    ref = g / (1 + np.exp(-g)) * u
    assert np.all(np.abs(h - ref) <= 6 * np.spacing(np.abs(ref).astype(np.float32)) + 1e-40)
    # the halves are not interchangeable
    ref_swapped = u / (1 + np.exp(-u)) * g
    assert not np.allclose(h, ref_swapped, rtol=1e-3)


def test_swiglu_zero_cases():
    M, I = 3, 128
    gu = RNG.standard_normal((M, 2 * I)).astype(np.float32)
    gu[0, :I] = 0.0            # silu(0) = 0 -> h = 0
    gu[1, I:] = 0.0            # u = 0 -> h = 0
    hq, hs, h = swiglu_quant(gu)
    assert np.all(h[:2] == 0) and np.all((hq[:2] & 0x7F) == 0) and np.all(hs[:2] == 1.0)
    gu2 = gu.copy()
    gu2[2, I:] = 1.0           # u = 1 -> h = silu(g)
    _, _, h2 = swiglu_quant(gu2)
    g = gu2[2, :I].astype(np.float64)
    assert np.allclose(h2[2], g / (1 + np.exp(-g)), rtol=1e-6, atol=1e-30)


def test_combine_identity_k1():
    T, H = 20, 256
    c = RNG.standard_normal((T, H)).astype(np.float32)
    y, bits = combine_ref(c.astype(np.float64), np.arange(T)[:, None], np.ones((T, 1), np.float32))
    tb = torch.from_numpy(c).to(torch.bfloat16)
    assert np.array_equal(bits, tb.view(torch.int16).numpy().view(np.uint16))
    y2, bits2 = combine_fp32_replay(c, np.arange(T)[:, None], np.ones((T, 1), np.float32))
    assert np.array_equal(bits2, bits)


def test_combine_weights_rows_and_shared():
    T, K, H = 6, 3, 128
    vals = RNG.standard_normal((T * K, H))
    dst = RNG.permutation(T * K).reshape(T, K)
    gate = RNG.uniform(0, 1, (T, K)).astype(np.float32)
    S = RNG.standard_normal((T, H))
    y, _ = combine_ref(vals, dst, gate, S)
    for t in range(T):
        ref = sum(float(gate[t, k]) * vals[dst[t, k]] for k in range(K)) + S[t]
        half_ulp = np.exp2(np.floor(np.log2(np.abs(ref))) - 8)      # bf16 keeps 8 bits
        assert np.all(np.abs(y[t] - ref) <= half_ulp)                # correctly rounded
        assert np.array_equal(y[t], y[t].astype(np.float32).astype(np.float64))
    yr, _ = combine_fp32_replay(vals.astype(np.float32), dst, gate, S.astype(np.float32))
    assert np.all(np.abs(yr - y) <= 2.0 ** -7 * np.abs(y) + 1e-30)


def _quant_weights(d, shared):
    w13q, w13s = quant_weight_128x128(d["w13"].float().numpy())
    w2q, w2s = quant_weight_128x128(d["w2"].float().numpy())
    sh = None
    if shared:
        a, b = quant_weight_128x128(d["sw13"].float().numpy())
        c, e = quant_weight_128x128(d["sw2"].float().numpy())
        sh = (a, b, c, e)
    return w13q, w13s, w2q, w2s, sh


@pytest.mark.parametrize("variant", ["tiny", "tiny_sigmoid_shared"])
def test_layer_permuted_equals_dense(variant):
    cfg = synth.get_config("tiny")
    shared = False
    if variant == "tiny_sigmoid_shared":
        cfg.update(T=48, E=16, K=4, route=dict(mode="sigmoid_bias", K=4, normalize=True),
                   bias_std=0.05, shared_I=128)
        shared = True
    else:
        cfg.update(T=64)
    d = synth.layer_inputs(cfg, "cpu", seed=3)
    w13q, w13s, w2q, w2s, sh = _quant_weights(d, shared)
    x = d["x"].float().numpy()
    logits = d["logits"].numpy()
    bias = None if d["bias"] is None else d["bias"].numpy()
    out = layer_forward(x, logits, bias, cfg["route"], w13q, w13s, w2q, w2s, shared=sh)
    yd, bd = layer_forward_dense(x, logits, bias, cfg["route"], w13q, w13s, w2q, w2s, shared=sh)
    assert np.array_equal(out["y_bits"], bd)
    assert np.abs(out["y"]).max() > 0
