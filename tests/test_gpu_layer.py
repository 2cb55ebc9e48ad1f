"""End-to-end parity of the layer forward (the launch sequence the bench
times) against the oracle's independent evaluation of the same layer.

Rule for the bf16 output y:
  * every intermediate that is integer or FP8 (routing, activation codes,
    permutation) must match the oracle bit for bit;
  * the hidden state h is quantised from a float32 GEMM result, so its FP8
    codes may differ from the oracle's only by one step next to a rounding
    boundary (rare) and its scales only by float32 rounding;
  * tokens whose every h code matches the oracle: y within 1 bf16 ulp of the
    oracle's y (rounded once from float64);
  * tokens with a boundary flip in h: |y - y_oracle| within 1 bf16 ulp plus
    the effect of the flipped codes through the down projection
    (sum_k gate * |W2| . |dequant difference|) plus the GEMM tolerance;
  * every token, with the down GEMM and the combine fed the oracle's own h
    (the same launches, so the rounding boundary of h is out of the way):
    within 1 bf16 ulp, or under cancellation the GEMM tolerance of the
    magnitude sum; the fraction within 1 ulp is reported.
"""

import numpy as np
import pytest
import torch

import oracle as O
import routed_experts_fp8_amd as R
import synth
from helpers import GEMM_RTOL, bf16_bits, bf16_ulp_distance, check_hidden, dev, dequant_rows, np_

pytestmark = pytest.mark.gpu


def _variant(name):
    cfg = synth.get_config("tiny")
    if name == "tiny_sigmoid_shared":
        cfg.update(T=200, E=16, K=4, I=256, route=dict(mode="sigmoid_bias", K=4, normalize=True),
                   bias_std=0.01, shared_I=256, x_dtype="bf16", w_dtype="bf16")
    if name == "small_moge":
        cfg.update(T=512, H=1024, E=32, I=384, K=8, route=dict(mode="softmax_grouped", n_groups=8,
                                                                 k_per_group=1),
                   x_dtype="bf16", w_dtype="bf16")
    return cfg


def run_layer(cfg, fused, seed=0, overlap_shared=True, **fusions):
    d = synth.layer_inputs(cfg, dev(), seed=seed)
    w = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"))
    fwd = R.MoEForward(cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["route"], w, dev(), fused=fused,
                       shared_I=cfg.get("shared_I"), overlap_shared=overlap_shared, **fusions)
    y = fwd(d["x"], d["logits"], d["bias"])
    torch.cuda.synchronize()
    return d, w, fwd, y


def check_layer_against_oracle(cfg, d, w, fwd, y):
    x = np_(d["x"])
    logits = np_(d["logits"])
    bias = None if d["bias"] is None else np_(d["bias"])
    wq = {k: np_(v) for k, v in w.items()}
    # weights: the GPU's quantised weights must equal the oracle's (checked),
    # then the oracle layer runs on its own quantised weights
    w13q, w13s = O.quant_weight_128x128(np_(d["w13"]))
    w2q, w2s = O.quant_weight_128x128(np_(d["w2"]))
    assert np.array_equal(wq["w13q"], w13q) and np.array_equal(wq["w13s"], w13s)
    assert np.array_equal(wq["w2q"], w2q) and np.array_equal(wq["w2s"], w2s)
    shared = None
    if cfg.get("shared_I"):
        a, b = O.quant_weight_128x128(np_(d["sw13"]))
        c, e = O.quant_weight_128x128(np_(d["sw2"]))
        shared = (a, b, c, e)
    ref = O.layer_forward(x, logits, bias, cfg["route"], w13q, w13s, w2q, w2s, shared=shared)
    b = {k: np_(v) for k, v in fwd.buf.items()}
    assert np.array_equal(b["idx"], ref["topk_idx"])
    if cfg["route"]["mode"] == "sigmoid_bias":
        assert np.array_equal(b["gate"], ref["topk_gate"])
    else:
        assert np.all(np.abs(b["gate"] - ref["topk_gate"]) <= np.spacing(np.abs(ref["topk_gate"])))
    for k_gpu, k_ref in (("xq", "xq"), ("xs", "xs"), ("offsets", "offsets"), ("dst_row", "dst_row"),
                         ("src_token", "src_token")):
        assert np.array_equal(b[k_gpu], ref[k_ref]), k_gpu
    # GEMM1 reads its grouped rows from x's codes through src_token: that
    # operand is the oracle's permuted one
    assert np.array_equal(b["xq"][b["src_token"]], ref["aq"])
    assert np.array_equal(b["xs"][b["src_token"]], ref["as"])

    T, K = ref["dst_row"].shape
    H = x.shape[1]
    # hidden state: codes valid under the GEMM tolerance (boundary flips only)
    frac, row_dirty = check_hidden(b["hq"], b["hs"], ref["c1"], ref["mag1"], ref["hq"])
    assert frac < 0.01, frac
    dh = np.abs(dequant_rows(b["hq"], b["hs"]) - dequant_rows(ref["hq"], ref["hs"]))
    dh[~row_dirty] = 0.0
    shared_dirty = np.zeros(T, bool)
    dsh = None
    if shared is not None:
        sfrac, shared_dirty = check_hidden(b["shq"], b["shs"], ref["shared_c1"], ref["shared_mag1"],
                                           ref["shared_hq"])
        assert sfrac < 0.01, sfrac
        dsh = np.abs(dequant_rows(b["shq"], b["shs"]) - dequant_rows(ref["shared_hq"], ref["shared_hs"]))
        dsh[~shared_dirty] = 0.0
    tok_dirty = row_dirty[ref["dst_row"]].any(axis=1) | shared_dirty

    yb = bf16_bits(y)
    ulp = bf16_ulp_distance(yb, ref["y_bits"])
    clean = ~tok_dirty
    # clean tokens: 1 bf16 ulp, or (under cancellation) the GEMM tolerance of
    # the magnitude sum of the terms that make up y
    mag_y = np.zeros((T, H))
    for k in range(K):
        mag_y += ref["topk_gate"][:, k:k + 1].astype(np.float64) * ref["mag2"][ref["dst_row"][:, k]]
    if shared is not None:
        mag_y += ref["shared_mag2"]
    yg = np_(y).astype(np.float64)
    ok = (ulp <= 1) | (np.abs(yg - ref["y"]) <= GEMM_RTOL * mag_y)
    assert ok[clean].all(), f"clean tokens: {(~ok[clean]).sum()} elements beyond 1 ulp"
    n_cancel = int(((ulp > 1) & clean[:, None]).sum())
    n_dirty = int(tok_dirty.sum())
    if n_dirty:
        W2 = O.dequant_weight(w2q, w2s)
        for t in np.nonzero(tok_dirty)[0]:
            bound = np.zeros(H)
            for k in range(K):
                r = ref["dst_row"][t, k]
                e = ref["topk_idx"][t, k]
                bound += float(ref["topk_gate"][t, k]) * (np.abs(W2[e]) @ dh[r] + GEMM_RTOL * ref["mag2"][r])
            if dsh is not None:
                SW2 = O.dequant_weight(shared[2], shared[3])[0]
                bound += np.abs(SW2) @ dsh[t]
            ulp_ref = np.spacing(np.abs(ref["y"][t]).astype(np.float32)).astype(np.float64) * 2 ** 16
            assert np.all(np.abs(yg[t] - ref["y"][t]) <= ulp_ref + bound), t
    # the down projection and the combine fed the oracle's own h: every token
    c2_f = R.grouped_gemm_fp8_blockscaled(torch.from_numpy(ref["hq"]).to(dev()),
                                          torch.from_numpy(ref["hs"]).to(dev()), w["w2q"], w["w2s"],
                                          fwd.buf["offsets"])
    sc2_f = None
    if shared is not None:
        sc2_f = R.grouped_gemm_fp8_blockscaled(torch.from_numpy(ref["shared_hq"]).to(dev()),
                                               torch.from_numpy(ref["shared_hs"]).to(dev()), w["sw2q"],
                                               w["sw2s"], fwd.buf["one_group"])
    y_f = R.moe_combine(c2_f, fwd.buf["dst_row"], fwd.buf["gate"], sc2_f)
    ulp_f = bf16_ulp_distance(bf16_bits(y_f), ref["y_bits"])
    ok_f = (ulp_f <= 1) | (np.abs(np_(y_f).astype(np.float64) - ref["y"]) <= GEMM_RTOL * mag_y)
    assert ok_f.all(), f"oracle h: {(~ok_f).sum()} elements beyond 1 ulp + GEMM tolerance"
    return dict(dirty_tokens=n_dirty, tokens=T, h_code_diff_frac=frac, cancel_elems=n_cancel,
                y_within_1ulp=float(np.mean(ulp <= 1)), y_within_1ulp_oracle_h=float(np.mean(ulp_f <= 1)))


@pytest.mark.parametrize("name", ["tiny", "tiny_sigmoid_shared", "small_moge"])
@pytest.mark.parametrize("fused", [True, False])
def test_layer_matches_oracle(name, fused):
    cfg = _variant(name)
    d, w, fwd, y = run_layer(cfg, fused)
    stats = check_layer_against_oracle(cfg, d, w, fwd, y)
    print(name, fused, stats)


@pytest.mark.parametrize("name", ["tiny_sigmoid_shared", "small_moge"])
def test_layer_fused_combine_matches_oracle(name):
    """The forward with the combine inside the down projection's epilogue
    meets the same oracle rule."""
    cfg = _variant(name)
    d, w, fwd, y = run_layer(cfg, True, fuse_combine=True)
    print(name, check_layer_against_oracle(cfg, d, w, fwd, y))


@pytest.mark.parametrize("name", ["tiny_sigmoid_shared", "small_moge"])
def test_layer_stage_fusions_are_bit_identical(name):
    """Routing + permutation in one launch and the combine in the down
    projection's epilogue change no bit of any buffer the forward writes,
    with the shared expert on its side stream or in line, over repeated
    calls."""
    cfg = _variant(name)
    keys = ("idx", "gate", "offsets", "dst_row", "src_token", "hq", "hs", "c2", "y")
    ref = None
    for frp in (False, True):
        for fc in (False, True):
            for overlap in (True, False):
                d, _, fwd, _ = run_layer(cfg, True, overlap_shared=overlap, fuse_route_permute=frp,
                                         fuse_combine=fc)
                for _ in range(2):
                    fwd(d["x"], d["logits"], d["bias"])
                torch.cuda.synchronize()
                got = {k: np_(fwd.buf[k].view(torch.uint8)) for k in keys}
                if ref is None:
                    ref = got
                for k in keys:
                    assert np.array_equal(got[k], ref[k]), (k, frp, fc, overlap)
                assert not fwd.buf["combine_ctr"].any() and not fwd.buf["rp_ws"][:256].any()


def test_layer_fused_equals_unfused_and_is_deterministic():
    cfg = _variant("tiny_sigmoid_shared")
    _, _, _, y1 = run_layer(cfg, True)
    _, _, _, y2 = run_layer(cfg, False)
    _, _, _, y3 = run_layer(cfg, True)
    assert np.array_equal(bf16_bits(y1), bf16_bits(y2))
    assert np.array_equal(bf16_bits(y1), bf16_bits(y3))


def test_layer_shared_expert_side_stream_equals_in_line():
    """The shared expert on its own stream (the default) and in line on the
    caller's stream give the same bits, over repeated calls of one layer
    object (buffers reused across steps)."""
    cfg = _variant("tiny_sigmoid_shared")
    d, _, fwd, y1 = run_layer(cfg, True, overlap_shared=True)
    _, _, _, y2 = run_layer(cfg, True, overlap_shared=False)
    assert np.array_equal(bf16_bits(y1), bf16_bits(y2))
    for _ in range(3):
        y = fwd(d["x"], d["logits"], d["bias"])
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y), bf16_bits(y2))


@pytest.mark.parametrize("fuse_combine", [False, True])
def test_layer_forward_in_a_hip_graph(fuse_combine):
    """The forward allocates nothing and joins its side stream, so it can be
    captured once in a HIP graph and replayed: every replay (with the
    program's own eager work and synchronisations in between) gives the
    eager result bit for bit, also after the inputs change in place.  The
    fused stages' counters live in the layer's workspaces and are reset by
    the kernels themselves, so replays need no clearing either."""
    cfg = _variant("tiny_sigmoid_shared")
    d, w, fwd, y_eager = run_layer(cfg, True, fuse_combine=fuse_combine, fuse_route_permute=fuse_combine)
    ref = bf16_bits(y_eager)
    x, logits, bias = d["x"].clone(), d["logits"].clone(), d["bias"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on the capture stream
        fwd(x, logits, bias)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_graph = fwd(x, logits, bias)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y_graph), ref)
        fwd(d["x"], d["logits"], d["bias"])       # eager work between replays
        torch.cuda.synchronize()
    # new inputs written into the captured tensors: replay follows them
    d2 = synth.layer_inputs(cfg, dev(), seed=1, weights=False)
    ref2 = bf16_bits(fwd(d2["x"], d2["logits"], d2["bias"]))   # eager, same weights
    assert not np.array_equal(ref2, ref)
    x.copy_(d2["x"]), logits.copy_(d2["logits"]), bias.copy_(d2["bias"])
    g.replay()
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y_graph), ref2)


def test_training_step_in_a_hip_graph():
    """A whole training step of the layer (forward keeping its gate|up
    output, input-side backward, FP8 weight gradients, balancing bias
    update) captured once and replayed: nothing in it allocates or clears
    memory, its side-stream work joins the capturing stream, so every
    replay (with eager steps in between, the bias reset before each) gives
    the eager step's results bit for bit."""
    cfg = _variant("tiny_sigmoid_shared")
    T, H, E, I = cfg["T"], cfg["H"], cfg["E"], cfg["I"]
    d = synth.layer_inputs(cfg, dev(), seed=0)
    w, wt = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"), transposed=True)
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev(), fused=False, shared_I=cfg.get("shared_I"))
    bwd = R.MoEBackward(fwd, wt, weight_grad=True)
    wg = R.MoEWeightGrad(bwd)
    x, logits, bias0 = d["x"].clone(), d["logits"].clone(), d["bias"].clone()
    dy = synth.output_grad(T, H, dev(), seed=4)
    bias = bias0.clone()

    def step():
        y = fwd(x, logits, bias)
        dx, dl = bwd(dy, logits)
        grads = wg(x, dy)
        fwd.update_bias(bias, 1e-3)
        return [y, dx, dl, bias] + [grads[k] for k in sorted(grads)]

    def snapshot(outs):
        return [o.clone() for o in outs]

    ref = snapshot(step())
    torch.cuda.synchronize()
    assert not torch.equal(ref[3], bias0)               # the update moved the bias
    bias.copy_(bias0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                          # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    bias.copy_(bias0)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    for _ in range(3):
        bias.copy_(bias0)
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8))
        bias.copy_(bias0)
        step()                                          # eager work between replays
        torch.cuda.synchronize()
