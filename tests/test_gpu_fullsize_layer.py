"""End-to-end parity of the layer forward at the full workload sizes, in the
launch sequence the bench times: MoEForward with the fused gate|up GEMM
(rows gathered from x's codes), the shared expert on its side stream, the
down GEMM and the combine.  The oracle evaluates, independently and from the
generator's inputs only, the routing and permutation of every token and the
whole layer for a sample of tokens (every expert row those tokens use, their
shared expert rows and their combine), with its own quantised weights of
every expert involved (checked bit for bit against the GPU's).

Rules (DeepSeek-V3 page section 2.1: shared plus routed experts, no token
dropped; Pangu page, MoGE section: exactly K' picks per group):
  * routing, gates (sigmoid mode), permutation, activation codes and the
    involved experts' weight codes: bit-exact;
  * h codes from the fused GEMM1: valid under the 1e-4 GEMM tolerance
    (boundary flips only, under 1 %);
  * GEMM2 in the bench's launch (same M, groups, offsets): on the sampled
    rows, fed the oracle's own h codes, within 1e-4 of the magnitude sum;
  * y (bf16) of the timed forward: within 1 bf16 ulp of the oracle's y
    (rounded once from float64), or within 1 ulp plus the propagated bound
    (the GPU's h codes that differ from the oracle's, and its scales, through
    |W2|; the GEMM tolerance of the terms).  h is quantised from a float32
    GEMM result, so a code next to a rounding boundary may legitimately land
    on the other side (about 0.17 % of codes, some 18 per token at the MoGE
    shape, each worth a fraction of an ulp of y): the fraction of y within
    1 ulp is printed, not required;
  * y of the down GEMM + combine launches (bench configuration) fed the
    oracle's own h on the sampled rows: every element within 1 bf16 ulp of
    the oracle's y or, where the terms cancel (y small against the sum of the
    terms' magnitudes), within the GEMM tolerance of that magnitude sum; the
    fraction needing the second clause is printed (0.2 % measured at the
    DeepSeek-V3 shape) and must stay under 1 %.
"""

import numpy as np
import pytest
import torch

import oracle as O
import routed_experts_fp8_amd as R
import synth
from helpers import (GEMM_RTOL, assert_gemm_close, bf16_bits, bf16_ulp_distance, check_hidden, dev,
                     np_)
from oracle import native as N

pytestmark = pytest.mark.gpu

F32 = np.float32
LUT = O.e4m3_decode(np.arange(256, dtype=np.uint8))


def _deq_rows(q, s):
    """Dequantised 1x128-tile rows (float64) by table lookup."""
    rows, cols = q.shape
    return (LUT[q].reshape(rows, -1, 128) * np.asarray(s, np.float64)[:, :, None]).reshape(rows, cols)


def _deq_weight(q, s):
    """Dequantised [rows, cols] 128x128-block matrix (float64) by table lookup."""
    rows, cols = q.shape
    sc = np.repeat(np.repeat(np.asarray(s, np.float64), 128, axis=0), 128, axis=1)
    return LUT[q] * sc


def _sample_tokens(idx, counts, T, rng, n=64):
    """First and last token, up to 8 tokens of the least and of the most
    loaded non-empty expert, random ones up to n."""
    nz = np.nonzero(counts)[0]
    lo, hi = nz[np.argmin(counts[nz])], nz[np.argmax(counts[nz])]
    pick = {0, T - 1}
    for e in (lo, hi):
        toks = np.nonzero((idx == e).any(axis=1))[0]
        pick |= set(rng.choice(toks, min(8, len(toks)), replace=False).tolist())
    while len(pick) < n:
        pick.add(int(rng.integers(0, T)))
    return np.array(sorted(pick)), int(lo), int(hi)


def _inputs(key):
    cfg = synth.get_config("skewed" if key == "skewed_dead" else key)
    d = synth.layer_inputs(cfg, dev(), seed=0, weights=True)
    if key == "skewed_dead":
        # the four least popular experts receive no token at all
        low = torch.argsort(d["logits"].mean(0))[:4]
        d["logits"][:, low] = -30.0
    return cfg, d


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["dsv3", "moge", "skewed", "skewed_dead"])
def test_fullsize_layer_forward_end_to_end(key):
    rng = np.random.default_rng(2026)
    cfg, d = _inputs(key)
    T, H, E, I, K = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["K"]
    w = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"))
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev(), fused=True, shared_I=cfg.get("shared_I"))
    y = fwd(d["x"], d["logits"], d["bias"])
    torch.cuda.synchronize()
    b = fwd.buf

    # routing and permutation of every token: bit-exact
    logits = np_(d["logits"])
    rc = cfg["route"]
    if rc["mode"] == "sigmoid_bias":
        io, go = O.route_sigmoid_bias(logits, None if d["bias"] is None else np_(d["bias"]), K,
                                      rc["normalize"])
        assert np.array_equal(np_(b["gate"]), go)
    else:
        io, go = O.route_softmax_grouped(logits, rc["n_groups"], rc["k_per_group"])
        assert np.all(np.abs(np_(b["gate"]) - go) <= np.spacing(np.abs(go)))
        assert O.imbalance_score(io, E, rc["n_groups"]) == 0.0
    assert np.array_equal(np_(b["idx"]), io)
    po = O.permute(io, E)
    for k in ("offsets", "dst_row", "src_token"):
        assert np.array_equal(np_(b[k]), po[k]), k
    counts = np.diff(po["offsets"])
    if key == "skewed_dead":
        assert (counts == 0).sum() >= 4

    toks, e_lo, e_hi = _sample_tokens(io, counts, T, rng)
    nt = len(toks)
    x_s = np_(d["x"][torch.from_numpy(toks).to(dev())]).astype(F32)
    xq_o, xs_o = O.quant_act_1x128(x_s)
    assert np.array_equal(np_(b["xq"])[toks], xq_o) and np.array_equal(np_(b["xs"])[toks], xs_o)

    rows = po["dst_row"][toks]                      # [nt, K] grouped rows of the sampled pairs
    hq_g_all, hs_g_all = np_(b["hq"]), np_(b["hs"])
    c2_o = np.zeros((nt * K, H))                    # oracle expert outputs, local slot order
    mag2 = np.zeros((nt * K, H))
    flip = np.zeros((nt * K, H))                    # |W2| . |h_gpu - h_oracle| per slot
    hq_o_rows = np.zeros((nt * K, I), np.uint8)
    hs_o_rows = np.zeros((nt * K, I // 128), F32)
    code_diff, n_rows = 0, 0
    for e in np.unique(io[toks]):
        sel = np.nonzero(io[toks] == e)             # (token position, slot) pairs using expert e
        slots = sel[0] * K + sel[1]
        r_e = rows[sel]
        q13, s13 = N.quant_weight_128x128(np_(d["w13"][e]).astype(F32))
        q2, s2 = N.quant_weight_128x128(np_(d["w2"][e]).astype(F32))
        assert np.array_equal(np_(w["w13q"][e]), q13[0]) and np.array_equal(np_(w["w13s"][e]), s13[0])
        assert np.array_equal(np_(w["w2q"][e]), q2[0]) and np.array_equal(np_(w["w2s"][e]), s2[0])
        C1, Mag1 = N.gemm_rows(xq_o[sel[0]], xs_o[sel[0]], q13[0], s13[0])
        hq_o, hs_o, _ = O.swiglu_quant(C1.astype(F32))
        frac, _ = check_hidden(hq_g_all[r_e], hs_g_all[r_e], C1, Mag1, hq_o)
        code_diff += frac * len(r_e)
        n_rows += len(r_e)
        C2, M2 = N.gemm_rows(hq_o, hs_o, q2[0], s2[0])
        c2_o[slots], mag2[slots] = C2, M2
        hq_o_rows[slots], hs_o_rows[slots] = hq_o, hs_o
        dh = np.abs(_deq_rows(hq_g_all[r_e], hs_g_all[r_e]) - _deq_rows(hq_o, hs_o))
        if dh.any():
            flip[slots] = dh @ np.abs(_deq_weight(q2[0], s2[0])).T
    assert code_diff / n_rows < 0.01

    # GEMM2 in the bench's launch configuration, fed the oracle's own h on
    # the sampled rows (rows are independent, the others keep the GPU's h)
    rflat = torch.from_numpy(rows.ravel().astype(np.int64)).to(dev())
    hq_mix, hs_mix = b["hq"].clone(), b["hs"].clone()
    hq_mix[rflat] = torch.from_numpy(hq_o_rows).to(dev())
    hs_mix[rflat] = torch.from_numpy(hs_o_rows).to(dev())
    c2_mix = R.grouped_gemm_fp8_blockscaled(hq_mix, hs_mix, w["w2q"], w["w2s"], b["offsets"])
    worst2 = assert_gemm_close(np_(c2_mix[rflat]), c2_o, mag2, what=f"{key} gemm2 (bench launch)")
    del hq_mix, hs_mix

    S = S_mag = S_flip = None
    if cfg.get("shared_I"):
        q13, s13 = N.quant_weight_128x128(np_(d["sw13"][0]).astype(F32))
        q2, s2 = N.quant_weight_128x128(np_(d["sw2"][0]).astype(F32))
        assert np.array_equal(np_(w["sw13q"][0]), q13[0]) and np.array_equal(np_(w["sw2q"][0]), q2[0])
        C1, Mag1 = N.gemm_rows(xq_o, xs_o, q13[0], s13[0])
        hq_o, hs_o, _ = O.swiglu_quant(C1.astype(F32))
        shq, shs = np_(b["shq"])[toks], np_(b["shs"])[toks]
        sfrac, _ = check_hidden(shq, shs, C1, Mag1, hq_o)
        assert sfrac < 0.01
        S, S_mag = N.gemm_rows(hq_o, hs_o, q2[0], s2[0])
        dh = np.abs(_deq_rows(shq, shs) - _deq_rows(hq_o, hs_o))
        S_flip = dh @ np.abs(_deq_weight(q2[0], s2[0])).T
        tsel = torch.from_numpy(toks.astype(np.int64)).to(dev())
        shq_mix, shs_mix = b["shq"].clone(), b["shs"].clone()
        shq_mix[tsel] = torch.from_numpy(hq_o).to(dev())
        shs_mix[tsel] = torch.from_numpy(hs_o).to(dev())
        one = b["one_group"]
        sc2_mix = R.grouped_gemm_fp8_blockscaled(shq_mix, shs_mix, w["sw2q"], w["sw2s"], one)
        assert_gemm_close(np_(sc2_mix[tsel]), S, S_mag, what=f"{key} shared gemm2 (bench launch)")
        del shq_mix, shs_mix
    else:
        sc2_mix = None

    # the layer output of the timed forward
    local = np.arange(nt * K).reshape(nt, K)
    y_o, y_bits_o = O.combine_ref(c2_o, local, go[toks], S)
    gate = go[toks].astype(np.float64)
    bound = np.zeros((nt, H))
    mag_y = np.zeros((nt, H))
    for k in range(K):
        bound += gate[:, k:k + 1] * flip[local[:, k]]
        mag_y += gate[:, k:k + 1] * mag2[local[:, k]]
    if S is not None:
        bound += S_flip
        mag_y += S_mag
    ulp_ref = np.spacing(np.abs(y_o).astype(np.float32)).astype(np.float64) * 2 ** 16
    ulp = bf16_ulp_distance(bf16_bits(y)[toks], y_bits_o)
    yg = np_(y)[toks].astype(np.float64)
    ok = (ulp <= 1) | (np.abs(yg - y_o) <= ulp_ref + bound + GEMM_RTOL * mag_y)
    assert ok.all(), f"{key}: {(~ok).sum()} elements of y outside the bound"
    within = float(np.mean(ulp <= 1))

    # the down GEMM + combine launches fed the oracle's h: 1 ulp
    y_mix = R.moe_combine(c2_mix, b["dst_row"], b["gate"], sc2_mix)
    ulp_m = bf16_ulp_distance(bf16_bits(y_mix)[toks], y_bits_o)
    ym = np_(y_mix)[toks].astype(np.float64)
    ok_m = (ulp_m <= 1) | (np.abs(ym - y_o) <= ulp_ref + GEMM_RTOL * mag_y)
    assert ok_m.all(), f"{key}: {(~ok_m).sum()} elements of y (oracle h) beyond 1 ulp + GEMM tolerance"
    within_m = float(np.mean(ulp_m <= 1))
    print(f"{key}: {nt} tokens ({nt * K} expert rows, {len(np.unique(io[toks]))} experts; least / most "
          f"loaded expert {e_lo} ({counts[e_lo]} rows) / {e_hi} ({counts[e_hi]} rows)); h codes differing "
          f"{code_diff / n_rows:.2e}; gemm2 worst {worst2:.3g}; y within 1 bf16 ulp: timed forward "
          f"{within:.4f}, fed the oracle's h {within_m:.6f} (max {int(ulp_m.max())} ulp)")
    assert within_m >= 0.99, within_m


@pytest.mark.timeout(600)
@pytest.mark.parametrize("key", ["dsv3", "moge", "skewed", "skewed_dead"])
def test_fullsize_stage_fusions_bit_identical(key):
    """At the full workload sizes, routing + permutation in one launch and
    the combine in the down projection's epilogue write the same bits as
    the separate launches into every buffer of the forward (routing,
    permutation, h, the expert outputs and y), over repeated calls, and
    leave their counters zero."""
    cfg, d = _inputs(key)
    T, H, E, I = cfg["T"], cfg["H"], cfg["E"], cfg["I"]
    w = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"))
    del d["w13"], d["w2"]
    keys = ("idx", "gate", "offsets", "dst_row", "src_token", "hq", "hs", "c2", "y")
    ref = None
    for fused_stages in (False, True):
        fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev(), fused=True, shared_I=cfg.get("shared_I"),
                           fuse_route_permute=fused_stages, fuse_combine=fused_stages)
        for _ in range(2):
            fwd(d["x"], d["logits"], d["bias"])
        torch.cuda.synchronize()
        got = {k: fwd.buf[k].view(torch.uint8).clone() for k in keys}
        assert not fwd.buf["combine_ctr"].any() and not fwd.buf["rp_ws"][:256].any()
        if ref is None:
            ref = got
        else:
            for k in keys:
                assert torch.equal(got[k], ref[k]), k
        del fwd
