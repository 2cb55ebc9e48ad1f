"""GPU parity of the router projection and the balancing bias update."""

import numpy as np
import pytest
import torch

import oracle as O
import routed_experts_fp8_amd as R
import synth
from helpers import dev, np_, to_dev

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(71)
F32 = np.float32


def _check_logits(x, w):
    lg = np_(R.moe_router_logits(x, w)).astype(np.float64)
    ref, mag = O.router_logits(np_(x), np_(w))
    H = x.shape[1]
    bound = (H + 2) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(lg - ref)
    assert np.all(err <= bound), f"worst ratio {np.max(err / bound):.3g}"
    return float(np.max(err / (mag + 1e-300)))


@pytest.mark.parametrize("T,H,E", [(1, 64, 1), (65, 64, 40), (300, 512, 256), (129, 7168, 64),
                                   (8192, 128, 256), (8200, 64, 200)])      # the last two use 64-token tiles
def test_router_logits_shapes(T, H, E):
    x = to_dev(RNG.standard_normal((T, H)).astype(F32)).to(torch.bfloat16)
    w = to_dev((RNG.standard_normal((E, H)) / np.sqrt(H)).astype(F32))
    _check_logits(x, w)


def test_router_logits_deepseek_shape():
    """The DeepSeek-V3 layer's router: 4096 tokens, hidden 7168, 256 experts,
    generator inputs (x of the layer workload, N(0, 1/H) router weight)."""
    cfg = synth.get_config("dsv3")
    d = synth.layer_inputs(cfg, dev(), seed=0, weights=False)
    w = synth.router_weight(cfg, dev(), seed=0)
    worst = _check_logits(d["x"], w)
    print("worst |error| / magnitude sum:", worst)


def test_bias_update_bitexact():
    for E, T, K in [(8, 64, 2), (256, 4096, 8), (3, 5, 1)]:
        loads = RNG.multinomial(T * K, RNG.dirichlet(np.ones(E)))
        if E == 8:
            loads = np.full(E, T * K // E)                    # all at the mean: no change
        off = np.concatenate([[0], np.cumsum(loads)]).astype(np.int32)
        b = (RNG.standard_normal(E) * 0.01).astype(F32)
        b[0] = -0.0
        bg = to_dev(b)
        R.moe_bias_update(to_dev(off), 1e-3, bg)
        ref = O.bias_update(b, off, F32(1e-3))
        assert np.array_equal(np_(bg).view(np.uint32), ref.view(np.uint32))


def test_balancing_loop_matches_oracle():
    """40 training steps of route -> permute -> bias update on a skewed router
    (generator logits with fixed per-expert offsets), on the GPU and in the
    oracle from the same logits: the bias stays bit-identical every step and
    the load imbalance falls."""
    T, E, K = 512, 32, 4
    skew = synth.zipf_offsets(E, 1.2, 1.5, seed=7, device=dev())
    b_gpu = torch.zeros(E, dtype=torch.float32, device=dev())
    b_ref = np.zeros(E, F32)
    imb = []
    for step in range(40):
        logits = (synth.randn((T, E), 1.0, torch.float32, dev(), seed=100 + step, tid=1) + skew[None, :]).contiguous()
        idx, _ = R.moe_route(logits, b_gpu, K, "sigmoid_bias", normalize=True)
        off = R.moe_permute(idx, E)["offsets"]
        R.moe_bias_update(off, 5e-3, b_gpu)
        l_np = np_(logits)
        idx_o, _ = O.route_sigmoid_bias(l_np, b_ref, K, True)
        off_o = O.permute(idx_o, E)["offsets"]
        assert np.array_equal(np_(off), off_o), step
        b_ref = O.bias_update(b_ref, off_o, F32(5e-3))
        assert np.array_equal(np_(b_gpu).view(np.uint32), b_ref.view(np.uint32)), step
        imb.append(np.diff(off_o).max() / (T * K / E))
    assert np.mean(imb[-5:]) < 0.7 * imb[0], imb


def test_layer_with_router_weight():
    """MoEForward with a router weight computes its logits from x (the same
    bits as the standalone projection), routes on them, and update_bias
    applies one balancing step from that routing."""
    from test_gpu_layer import _variant
    cfg = _variant("tiny_sigmoid_shared")
    T, H, E, I = cfg["T"], cfg["H"], cfg["E"], cfg["I"]
    d = synth.layer_inputs(cfg, dev(), seed=0)
    w = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"))
    wr = synth.router_weight(cfg, dev(), seed=0)
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev(), shared_I=cfg.get("shared_I"), router_weight=wr)
    bias = d["bias"].clone()
    y = fwd(d["x"], None, bias).clone()
    lg = R.moe_router_logits(d["x"], wr)
    ref = R.MoEForward(T, H, E, I, cfg["route"], w, dev(), shared_I=cfg.get("shared_I"))
    y2 = ref(d["x"], lg, bias)
    torch.cuda.synchronize()
    assert torch.equal(fwd.buf["logits"], lg)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    off = np_(fwd.buf["offsets"])
    b0 = np_(bias)
    fwd.update_bias(bias, 1e-3)
    assert np.array_equal(np_(bias).view(np.uint32), O.bias_update(b0, off, F32(1e-3)).view(np.uint32))
