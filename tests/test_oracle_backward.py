"""Pins of the oracle's backward (CPU): finite differences of the float64
definitions, the float64 derivative of SwiGLU, and torch autograd (float64)
of the same layer as an independent reference for the whole chain."""

import numpy as np
import pytest
import torch

import oracle as O
import synth

RNG = np.random.default_rng(11)


def _gates_sigmoid(l, idx, normalize):
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(l, idx, axis=1)))
    return s / s.sum(axis=1, keepdims=True) if normalize else s


def _gates_softmax(l, idx):
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, idx, axis=1)


def _fd(f, l, h=1e-6):
    g = np.zeros_like(l)
    for t in range(l.shape[0]):
        for e in range(l.shape[1]):
            lp, lm = l.copy(), l.copy()
            lp[t, e] += h
            lm[t, e] -= h
            g[t, e] = (f(lp)[t] - f(lm)[t]) / (2 * h)
    return g


@pytest.mark.parametrize("normalize", [True, False])
def test_route_backward_sigmoid_finite_differences(normalize):
    T, E, K = 6, 16, 4
    logits = RNG.standard_normal((T, E)).astype(np.float32)
    bias = (RNG.standard_normal(E) * 0.3).astype(np.float32)
    idx, gate = O.route_sigmoid_bias(logits, bias, K, normalize)
    dg = RNG.standard_normal((T, K))
    l64 = logits.astype(np.float64)
    fd = _fd(lambda l: np.sum(dg * _gates_sigmoid(l, idx.astype(np.int64), normalize), axis=1), l64)
    d = O.route_backward_sigmoid(logits, idx, gate, dg, normalize)
    assert np.allclose(d, fd, atol=1e-8, rtol=1e-6)
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, idx.astype(np.int64), True, axis=1)
    assert np.all(d[~sel] == 0.0)            # unselected experts (and the bias) get nothing


def test_route_backward_softmax_finite_differences():
    T, E, G, Kp = 5, 16, 4, 1
    logits = RNG.standard_normal((T, E)).astype(np.float32)
    idx, gate = O.route_softmax_grouped(logits, G, Kp)
    dg = RNG.standard_normal(idx.shape)
    fd = _fd(lambda l: np.sum(dg * _gates_softmax(l, idx.astype(np.int64)), axis=1), logits.astype(np.float64))
    d = O.route_backward_softmax(logits, idx, dg)
    assert np.allclose(d, fd, atol=1e-8, rtol=1e-6)
    assert np.allclose(d.sum(axis=1), 0.0, atol=1e-12)   # softmax gradients sum to zero over experts


def test_swiglu_backward_derivative():
    M, I = 8, 256
    gu = (RNG.standard_normal((M, 2 * I)) * 3).astype(np.float32)
    dh = RNG.standard_normal((M, I)).astype(np.float32)
    dq, ds, d = O.swiglu_backward(gu, dh)
    g, u = gu[:, :I].astype(np.float64), gu[:, I:].astype(np.float64)
    s = 1.0 / (1.0 + np.exp(-g))
    dg_exact = dh * u * (s + g * s * (1 - s))
    du_exact = dh * g * s
    # binary32 evaluation with the specified sigmoid: a few ulp of the terms'
    # magnitudes (silu' crosses zero near g = -1.28, so not relative to dg)
    mag_g = np.abs(dh * u) * s * (1 + np.abs(g) * (1 - s))
    assert np.all(np.abs(d[:, :I] - dg_exact) <= 16 * 2.0 ** -24 * mag_g)
    assert np.all(np.abs(d[:, I:] - du_exact) <= 8 * 2.0 ** -24 * np.abs(du_exact))
    # finite differences of h = silu(g) u in float64
    h = 1e-6
    f = lambda gg, uu: gg / (1.0 + np.exp(-gg)) * uu
    assert np.all(np.abs(d[:, :I] - dh * (f(g + h, u) - f(g - h, u)) / (2 * h)) <= 1e-5 * mag_g + 1e-9)
    assert np.allclose(d[:, I:], dh * (f(g, u + h) - f(g, u - h)) / (2 * h), rtol=1e-5, atol=1e-9)
    # the FP8 operand is d quantised in 1x128 tiles along 2I (gate half, then up half)
    q2, s2 = O.quant_act_1x128(d)
    assert np.array_equal(dq, q2) and np.array_equal(ds, s2)
    # zero upstream gradient -> zero codes
    zq, zs, zd = O.swiglu_backward(gu, np.zeros_like(dh))
    assert np.all(zd == 0) and np.all((zq & 0x7F) == 0)


def test_combine_backward_definition():
    T, K, H = 7, 3, 256
    y = RNG.standard_normal((T * K, H)).astype(np.float32)
    dst = RNG.permutation(T * K).reshape(T, K).astype(np.int32)
    gate = RNG.uniform(0, 1, (T, K)).astype(np.float32)
    dy = O.bf16_round(RNG.standard_normal((T, H)))[0].astype(np.float32)
    dq, ds, d, dgate = O.combine_backward(dy, y, dst, gate)
    for t in range(T):
        for k in range(K):
            assert np.array_equal(d[dst[t, k]], (np.float32(gate[t, k]) * dy[t]).astype(np.float32))
    # d_gate is the derivative of <dy, y_out> along the gate (the combine is linear in it)
    ref = np.einsum("th,tkh->tk", dy.astype(np.float64), y[dst].astype(np.float64))
    assert np.allclose(dgate, ref, rtol=1e-12, atol=1e-12)
    q2, s2 = O.quant_act_1x128(d)
    assert np.array_equal(dq, q2) and np.array_equal(ds, s2)


def _autograd_reference(cfg, x, logits, bias, w, fwd, dy):
    """torch float64 autograd of the layer with the oracle's routing held
    fixed: experts use the dequantised FP8 weights and unquantised
    activations; returns (dx, d_logits with expert outputs from the oracle's
    forward held constant)."""
    E, I = cfg["E"], cfg["I"]
    W13 = torch.from_numpy(O.dequant_weight(w["w13q"], w["w13s"]))
    W2 = torch.from_numpy(O.dequant_weight(w["w2q"], w["w2s"]))
    idx = torch.from_numpy(fwd["topk_idx"].astype(np.int64))
    xt = torch.from_numpy(x.astype(np.float64)).requires_grad_(True)
    lt = torch.from_numpy(logits.astype(np.float64)).requires_grad_(True)
    rc = cfg["route"]
    if rc["mode"] == "sigmoid_bias":
        s = torch.sigmoid(torch.gather(lt, 1, idx))
        gate = s / s.sum(dim=1, keepdim=True) if rc.get("normalize", True) else s
    else:
        gate = torch.gather(torch.softmax(lt, dim=1), 1, idx)
    T, K = idx.shape
    y = torch.zeros((T, x.shape[1]), dtype=torch.float64)
    for k in range(K):
        for e in range(E):
            rows = (idx[:, k] == e).nonzero().flatten()
            if len(rows) == 0:
                continue
            c1 = xt[rows] @ W13[e].T
            h = torch.nn.functional.silu(c1[:, :I]) * c1[:, I:]
            y = y.index_add(0, rows, gate[rows, k:k + 1].detach() * (h @ W2[e].T))
    if cfg.get("shared_I"):
        S13 = torch.from_numpy(O.dequant_weight(w["sw13q"], w["sw13s"]))[0]
        S2 = torch.from_numpy(O.dequant_weight(w["sw2q"], w["sw2s"]))[0]
        c1 = xt @ S13.T
        Is = S13.shape[0] // 2
        y = y + (torch.nn.functional.silu(c1[:, :Is]) * c1[:, Is:]) @ S2.T
    dyt = torch.from_numpy(dy.astype(np.float64))
    (dx,) = torch.autograd.grad((y * dyt).sum(), xt)
    # router path: expert outputs as the oracle computed them (float32), gates live
    c2 = torch.from_numpy(fwd["c2"].astype(np.float32).astype(np.float64))
    dst = torch.from_numpy(fwd["dst_row"].astype(np.int64))
    yr = sum(gate[:, k:k + 1] * c2[dst[:, k]] for k in range(K))
    (dl,) = torch.autograd.grad((yr * dyt).sum(), lt)
    return dx.numpy(), dl.numpy()


def _tiny_case(name):
    cfg = synth.get_config("tiny")
    if name == "sigmoid_shared":
        cfg.update(T=64, E=8, K=2, I=256, route=dict(mode="sigmoid_bias", K=2, normalize=True),
                   bias_std=0.01, shared_I=256)
    else:
        cfg.update(T=64)
    return cfg


@pytest.mark.parametrize("name", ["tiny_softmax", "sigmoid_shared"])
def test_layer_backward_vs_autograd(name):
    cfg = _tiny_case(name)
    d = synth.layer_inputs(cfg, torch.device("cpu"), seed=3)
    x, logits = d["x"].float().numpy(), d["logits"].numpy()
    bias = None if d["bias"] is None else d["bias"].numpy()
    w = {}
    w["w13q"], w["w13s"] = O.quant_weight_128x128(d["w13"].float().numpy())
    w["w2q"], w["w2s"] = O.quant_weight_128x128(d["w2"].float().numpy())
    shared = None
    if cfg.get("shared_I"):
        w["sw13q"], w["sw13s"] = O.quant_weight_128x128(d["sw13"].float().numpy())
        w["sw2q"], w["sw2s"] = O.quant_weight_128x128(d["sw2"].float().numpy())
        shared = (w["sw13q"], w["sw13s"], w["sw2q"], w["sw2s"])
    fwd = O.layer_forward(x, logits, bias, cfg["route"], w["w13q"], w["w13s"], w["w2q"], w["w2s"], shared=shared)
    dy = O.bf16_round(RNG.standard_normal(x.shape))[0].astype(np.float32)
    bwd = O.layer_backward(fwd, dy, logits, cfg["route"], w["w13q"], w["w13s"], w["w2q"], w["w2s"], shared=shared)
    dx_ref, dl_ref = _autograd_reference(cfg, x, logits, bias, w, fwd, dy)
    # router gradient: no FP8 on its path -> float64 agreement
    assert np.allclose(bwd["d_logits"], dl_ref, rtol=1e-9, atol=1e-9)
    # dx: FP8 operands (x, dC2, dC1 quantised) against the unquantised float64
    # chain -> a few percent, and aligned
    err = np.linalg.norm(bwd["dx"] - dx_ref) / np.linalg.norm(dx_ref)
    cos = np.sum(bwd["dx"] * dx_ref) / (np.linalg.norm(bwd["dx"]) * np.linalg.norm(dx_ref))
    assert err < 0.08 and cos > 0.995, (err, cos)
