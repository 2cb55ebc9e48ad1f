"""GPU parity of the input-side backward: each new kernel against the oracle
on generator inputs, then the whole layer backward against the oracle's own
forward + backward."""

import numpy as np
import pytest
import torch

import oracle as O
import routed_experts_fp8_amd as R
import synth
from helpers import GEMM_RTOL, bf16_bits, bf16_ulp_distance, dequant_rows, dev, np_, to_dev
from test_gpu_layer import _variant

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(23)


@pytest.mark.parametrize("T,K,H", [(1, 1, 128), (37, 4, 512), (200, 8, 1024), (60, 16, 256)])   # K = 16: the limit
def test_combine_backward(T, K, H):
    y = RNG.standard_normal((T * K, H)).astype(np.float32)
    y[::5] *= np.float32(1e-3)
    dst = RNG.permutation(T * K).reshape(T, K).astype(np.int32)
    gate = RNG.uniform(0, 1, (T, K)).astype(np.float32)
    gate[0, 0] = 0.0                                        # a zero gate -> all-zero tile, scale 1
    dy = torch.from_numpy(RNG.standard_normal((T, H)).astype(np.float32)).to(torch.bfloat16)
    dq, ds, dg = R.moe_combine_backward(dy.to(dev()), to_dev(y), to_dev(dst), to_dev(gate))
    dyf = dy.float().numpy()
    qo, so, _, dgo = O.combine_backward(dyf, y, dst, gate)
    assert np.array_equal(np_(dq), qo) and np.array_equal(np_(ds), so)
    # float32 dot products of H terms in a fixed order vs float64
    mag = np.einsum("th,tkh->tk", np.abs(dyf).astype(np.float64), np.abs(y[dst]).astype(np.float64))
    assert np.all(np.abs(np_(dg) - dgo) <= (H + 8) * 2.0 ** -24 * mag + 1e-30)


@pytest.mark.parametrize("M,I", [(1, 128), (300, 256), (77, 2048)])
def test_swiglu_backward_bitexact(M, I):
    gu = (RNG.standard_normal((M, 2 * I)) * 3).astype(np.float32)
    gu[0, :8] = [0.0, -0.0, 80.0, -80.0, 100.0, -100.0, 1e-30, -1.2785]
    dh = RNG.standard_normal((M, I)).astype(np.float32)
    dh[-1] = 0.0                                             # zero row -> zero codes, scale 1
    dq, ds = R.swiglu_backward(to_dev(gu), to_dev(dh))
    qo, so, _ = O.swiglu_backward(gu, dh)
    assert np.array_equal(np_(dq), qo)
    assert np.array_equal(np_(ds), so)


def _route_inputs(T, E, mode, **kw):
    logits = (RNG.standard_normal((T, E)) * 2).astype(np.float32)
    lt = to_dev(logits)
    if mode == "sigmoid_bias":
        bias = (RNG.standard_normal(E) * 0.1).astype(np.float32)
        idx_g, _ = R.moe_route(lt, to_dev(bias), kw["K"], "sigmoid_bias", normalize=kw["normalize"])
        idx_o, gate_o = O.route_sigmoid_bias(logits, bias, kw["K"], kw["normalize"])
    else:
        idx_g, _ = R.moe_route(lt, None, kw["G"] * kw["Kp"], "softmax_grouped", n_groups=kw["G"],
                               k_per_group=kw["Kp"])
        idx_o, gate_o = O.route_softmax_grouped(logits, kw["G"], kw["Kp"])
    assert np.array_equal(np_(idx_g), idx_o)
    return logits, lt, idx_g, idx_o, gate_o


@pytest.mark.parametrize("normalize,T,E,K", [(True, 300, 256, 8), (False, 300, 256, 8),
                                              (True, 40, 256, 64)])          # K = 64: the limit
def test_route_backward_sigmoid(normalize, T, E, K):
    logits, lt, idx_g, idx_o, gate_o = _route_inputs(T, E, "sigmoid_bias", K=K, normalize=normalize)
    dg = RNG.standard_normal((T, K)).astype(np.float32)
    d = np_(R.moe_route_backward(lt, idx_g, to_dev(dg), "sigmoid_bias", normalize=normalize))
    ref = O.route_backward_sigmoid(logits, idx_o, gate_o, dg, normalize)
    # float64 inside, one rounding to float32 (plus float64 exp differences)
    assert np.all(np.abs(d - ref) <= np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-37)


@pytest.mark.parametrize("T,E,G,Kp", [(300, 64, 8, 1), (50, 16, 1, 2), (40, 128, 8, 8)])   # K = 64: the limit
def test_route_backward_softmax(T, E, G, Kp):
    logits, lt, idx_g, idx_o, gate_o = _route_inputs(T, E, "softmax_grouped", G=G, Kp=Kp)
    dg = RNG.standard_normal((T, G * Kp)).astype(np.float32)
    d = np_(R.moe_route_backward(lt, idx_g, to_dev(dg), "softmax_grouped"))
    ref = O.route_backward_softmax(logits, idx_o, dg)
    assert np.all(np.abs(d - ref) <= np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) + 1e-37)


def _oracle_weights(d, cfg):
    w13q, w13s = O.quant_weight_128x128(np_(d["w13"]).astype(np.float32))
    w2q, w2s = O.quant_weight_128x128(np_(d["w2"]).astype(np.float32))
    shared = None
    if cfg.get("shared_I"):
        a, b = O.quant_weight_128x128(np_(d["sw13"]).astype(np.float32))
        c, e = O.quant_weight_128x128(np_(d["sw2"]).astype(np.float32))
        shared = (a, b, c, e)
    return w13q, w13s, w2q, w2s, shared


def _flip_effect(dq_g, ds_g, dq_o, ds_o, W, groups, tol=GEMM_RTOL):
    """Per-row bound on how far a GEMM output row of the GPU may sit from the
    oracle's when its FP8 input row differs (codes next to a rounding
    boundary, scales by float32 rounding): |W_e| . |dequant difference|,
    plus the GEMM tolerance on that extra magnitude.  W [G, N, K] float64
    dequantised weights (output features N); groups [rows] expert ids.
    Returns (bound [rows, N], fraction of differing codes)."""
    rows = np.nonzero(np.any((dq_g != dq_o) | (np.repeat(ds_g, 128, 1) != np.repeat(ds_o, 128, 1)), axis=1))[0]
    out = np.zeros((dq_g.shape[0], W.shape[1]))
    if len(rows):
        diff = np.abs(dequant_rows(dq_g[rows], ds_g[rows]) - dequant_rows(dq_o[rows], ds_o[rows]))
        for i, r in enumerate(rows):
            out[r] = (1 + tol) * (np.abs(W[groups[r]]) @ diff[i])
    return out, float(np.mean(dq_g != dq_o))


def _row_groups(offsets):
    return np.repeat(np.arange(len(offsets) - 1), np.diff(offsets))


def _dlogits_bound(rc, fo, logits, B):
    """Bound on the router gradient's change when d_gate moves by at most B
    [T, K] (the map is linear in d_gate; see the oracle's router backward)."""
    idx = fo["topk_idx"].astype(np.int64)
    l = logits.astype(np.float64)
    T, E = l.shape
    out = np.zeros((T, E))
    if rc["mode"] == "sigmoid_bias":
        s = 1.0 / (1.0 + np.exp(-np.take_along_axis(l, idx, axis=1)))
        if rc.get("normalize", True):
            S = s.sum(axis=1, keepdims=True)
            dS = (B + np.sum(B * s / S, axis=1, keepdims=True)) / S
        else:
            dS = B
        np.put_along_axis(out, idx, dS * s * (1 - s), axis=1)
    else:
        p = np.exp(l - l.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        D = np.zeros((T, E))
        np.put_along_axis(D, idx, B, axis=1)
        out = p * (D + np.sum(B * np.take_along_axis(p, idx, axis=1), axis=1, keepdims=True))
    return out


@pytest.mark.parametrize("name", ["tiny", "tiny_sigmoid_shared", "small_moge"])
def test_layer_backward_matches_oracle(name):
    """Whole input-side backward against the oracle's forward + backward on
    the same seeded inputs, element by element:

    * dC2 codes are bit-exact where the gates are (sigmoid gates); softmax
      gates may differ by one float32 ulp, so a code at a boundary may move;
    * d_gate within the float32 dot-product bound, plus the effect of the
      forward's hidden-state boundary flips on the expert outputs;
    * d_logits within the image of that d_gate bound under the (linear)
      router backward, plus one float32 ulp;
    * dx within one bf16 ulp plus the GEMM tolerances and the effect of the
      dC1 codes that differ (boundary flips) through |W13|."""
    cfg = _variant(name)
    T, H, E, I = cfg["T"], cfg["H"], cfg["E"], cfg["I"]
    d = synth.layer_inputs(cfg, dev(), seed=0)
    w = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"))
    wt = R.transpose_weights(w)
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev(), fused=False, shared_I=cfg.get("shared_I"))
    fwd(d["x"], d["logits"], d["bias"])
    dy = synth.output_grad(T, H, dev(), seed=4)
    bwd = R.MoEBackward(fwd, wt)
    dx, dl = bwd(dy, d["logits"])
    torch.cuda.synchronize()

    x = np_(d["x"]).astype(np.float32)
    logits = np_(d["logits"])
    bias = None if d["bias"] is None else np_(d["bias"])
    w13q, w13s, w2q, w2s, shared = _oracle_weights(d, cfg)
    fo = O.layer_forward(x, logits, bias, cfg["route"], w13q, w13s, w2q, w2s, shared=shared)
    dyf = np_(dy)
    bo = O.layer_backward(fo, dyf, logits, cfg["route"], w13q, w13s, w2q, w2s, shared=shared)
    fb = {k: np_(v) for k, v in fwd.buf.items()}
    b = {k: np_(v) for k, v in bwd.buf.items()}
    groups = _row_groups(fo["offsets"])
    dst = fo["dst_row"]
    K = dst.shape[1]
    adx = np.abs(dyf).astype(np.float64)

    same = np.mean(b["dc2q"] == bo["dc2q"])
    assert same == 1.0 if cfg["route"]["mode"] == "sigmoid_bias" else same > 0.999, same

    # d_gate
    W2 = O.dequant_weight(w2q, w2s)                      # [E, H, I]
    dc2_flip, hfrac = _flip_effect(fb["hq"], fb["hs"], fo["hq"], fo["hs"], W2, groups)
    assert hfrac < 0.01, hfrac
    dc2_bound = dc2_flip + GEMM_RTOL * fo["mag2"]
    B = np.zeros((T, K))
    for k in range(K):
        r = dst[:, k]
        B[:, k] = np.sum(adx * dc2_bound[r], axis=1) + (H + 8) * 2.0 ** -24 * np.sum(
            adx * (fo["mag2"][r] + dc2_bound[r]), axis=1)
    assert np.all(np.abs(b["d_gate"] - bo["d_gate"]) <= B + 1e-30)

    # router gradient
    dlg = np_(dl).astype(np.float64)
    bl = _dlogits_bound(cfg["route"], fo, logits, B)
    ulp32 = np.spacing(np.abs(bo["d_logits"]).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(dlg - bo["d_logits"]) <= bl + ulp32 + 1e-37)
    if cfg["route"]["mode"] == "sigmoid_bias":
        sel = np.zeros((T, E), bool)
        np.put_along_axis(sel, fo["topk_idx"].astype(np.int64), True, axis=1)
        assert np.all(dlg[~sel] == 0.0)

    # dx
    W13 = O.dequant_weight(w13q, w13s)                   # [E, 2I, H]
    W13t = np.transpose(W13, (0, 2, 1))                  # output features H
    dxp_flip, dfrac = _flip_effect(b["dq1"], b["ds1"], bo["dq1"], bo["ds1"], W13t, groups)
    assert dfrac < 0.01, dfrac
    bound = np.zeros((T, H))
    mag = np.zeros((T, H))
    for k in range(K):
        r = dst[:, k]
        bound += dxp_flip[r] + GEMM_RTOL * bo["mag_dxp"][r]
        mag += bo["mag_dxp"][r]
    if shared is not None:
        SW13t = np.transpose(O.dequant_weight(shared[0], shared[1]), (0, 2, 1))
        sflip, sfrac = _flip_effect(b["dq1s"], b["ds1s"], bo["shared_dq1"], bo["shared_ds1"], SW13t,
                                    np.zeros(T, np.int64))
        assert sfrac < 0.01, sfrac
        assert np.array_equal(b["dyq"], bo["shared_dyq"]) and np.array_equal(b["dys"], bo["shared_dys"])
        bound += sflip + GEMM_RTOL * bo["shared_mag_dx"]
        mag += bo["shared_mag_dx"]
    bound += (K + 2) * 2.0 ** -24 * (mag + bound)          # float32 sum of K (+1) rows
    dxg = np_(dx).astype(np.float64)
    ulp16 = np.spacing(np.abs(bo["dx"]).astype(np.float32)).astype(np.float64) * 2 ** 16
    err = np.abs(dxg - bo["dx_f64"])
    assert np.all(err <= bound + ulp16), f"{np.sum(err > bound + ulp16)} dx elements out of bound"
    within = float(np.mean(bf16_ulp_distance(bf16_bits(dx), bo["dx_bits"]) <= 1))
    print(name, dict(h_code_diff=hfrac, dc1_code_diff=dfrac, dx_within_1ulp=within))
