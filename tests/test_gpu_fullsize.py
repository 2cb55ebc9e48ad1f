"""Parity at the full workload sizes, in the launch configuration the bench
times (the same entry points, grids and fused/unfused choices), checked on
outputs the oracle can compute one by one: whole routing / permutation
results and quantised tensors where they are cheap, sampled GEMM rows (every
sampled group with its ragged tail rows), and invariants that hold at any
size (IS = 0 for MoGE, transpose involution, bijective permutation).

Workloads: DeepSeek-V3-shaped layer (T=4096, H=7168, 256 experts top-8 +
shared), MoGE (T=8192, H=5120, 64 experts in 8 groups), skewed load (T=16384,
H=2048, 128 experts, Zipf-like logit offsets) with a variant whose four
least popular experts receive no token, and the backward-side block
transpose + dgrad on the DeepSeek-V3 expert shapes.
"""

import numpy as np
import pytest
import torch

import oracle as O
import routed_experts_fp8_amd as R
import synth
from helpers import assert_gemm_close, bf16_bits, check_hidden, dev, gemm_model_bound, np_

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(77)


def _route_and_permute(cfg, d):
    rc = cfg["route"]
    K = cfg["K"]
    if rc["mode"] == "sigmoid_bias":
        idx, gate = R.moe_route(d["logits"], d["bias"], K, "sigmoid_bias", normalize=rc["normalize"])
        io, go = O.route_sigmoid_bias(np_(d["logits"]), None if d["bias"] is None else np_(d["bias"]), K,
                                      rc["normalize"])
        assert np.array_equal(np_(idx), io) and np.array_equal(np_(gate), go)
    else:
        idx, gate = R.moe_route(d["logits"], None, K, "softmax_grouped", n_groups=rc["n_groups"],
                                k_per_group=rc["k_per_group"])
        io, go = O.route_softmax_grouped(np_(d["logits"]), rc["n_groups"], rc["k_per_group"])
        assert np.array_equal(np_(idx), io)
        assert np.all(np.abs(np_(gate) - go) <= np.spacing(np.abs(go)))
    xq, xs = R.quant_act_1x128_e4m3(d["x"])
    perm = R.moe_permute(idx, cfg["E"], xq, xs)
    po = O.permute(io, cfg["E"])
    for k in ("offsets", "dst_row", "src_token"):
        assert np.array_equal(np_(perm[k]), po[k]), k
    return idx, gate, xq, xs, perm, io


def _sample_rows(offsets, groups, per_group=8):
    """Up to `per_group` rows from each listed group: its first rows, its
    last (ragged-tail) rows and random ones in between."""
    rows = []
    for g in groups:
        r0, r1 = int(offsets[g]), int(offsets[g + 1])
        n = r1 - r0
        if n == 0:
            continue
        pick = {r0, r1 - 1, r0 + (n - 1) // 2}
        pick |= set((r0 + RNG.integers(0, n, per_group)).tolist())
        # rows of the last, possibly partial 128-row tile
        tail0 = r0 + (n - 1) // 128 * 128
        pick |= set(range(tail0, min(r1, tail0 + 3)))
        rows += sorted(pick)
    return np.array(rows, np.int64)


def _oracle_rows(x_np, src_o, rows):
    """Oracle operand rows: its own quantisation of the tokens its own
    permutation puts at those rows."""
    return O.quant_act_1x128(x_np[src_o[rows]])


def _check_gemm1(cfg, d, perm, w, x_np, po, groups, xq, xs):
    """Fused gate|up GEMM + SwiGLU + quantisation at full size (GPU launch as
    in the bench: rows gathered from x's codes through src_token) on sampled
    rows of sampled experts, against the oracle's own operands and its own
    quantised weights; the launch on the permuted copy gives the same bits."""
    off = po["offsets"]
    rows = _sample_rows(off, groups)
    hq, hs = R.grouped_gemm_fp8_swiglu(xq, xs, w["w13q"], w["w13s"], perm["offsets"], a_row=perm["src_token"])
    hq2, hs2 = R.grouped_gemm_fp8_swiglu(perm["aq"], perm["as"], w["w13q"], w["w13s"], perm["offsets"])
    assert torch.equal(hq, hq2) and torch.equal(hs, hs2)
    del hq2, hs2
    hq, hs = np_(hq), np_(hs)
    grp = np.searchsorted(off, rows, side="right") - 1
    for g in np.unique(grp):
        rg = rows[grp == g]
        q13, s13 = O.quant_weight_128x128(np_(d["w13"][g:g + 1]))
        assert np.array_equal(np_(w["w13q"][g]), q13[0]) and np.array_equal(np_(w["w13s"][g]), s13[0])
        aq_o, as_o = _oracle_rows(x_np, po["src_token"], rg)
        zero = np.array([0, len(rg)], np.int32)
        C1, Mag1 = O.grouped_gemm(aq_o, as_o, q13, s13, zero)
        hq_o, _, _ = O.swiglu_quant(C1.astype(np.float32))
        frac, _ = check_hidden(hq[rg], hs[rg], C1, Mag1, hq_o)
        assert frac < 0.01, frac
    return len(rows)


def _check_gemm2_synthetic(cfg, w, off_t, off, groups, seed=5):
    """Down-projection GEMM at full size (same grid as in the bench: same M,
    groups, offsets, N, K) on generator-made hidden-state codes and scales."""
    M, I = int(off[-1]), cfg["I"]
    g = torch.Generator(device=dev())
    g.manual_seed(seed)
    codes = torch.randint(0, 0x7F, (M, I), dtype=torch.uint8, device=dev(), generator=g)
    codes |= (torch.randint(0, 2, (M, I), dtype=torch.uint8, device=dev(), generator=g) << 7)
    scales = torch.exp2(torch.randint(-12, -4, (M, I // 128), device=dev(), generator=g).float()) * \
        (1 + torch.rand((M, I // 128), device=dev(), generator=g))
    c2 = np_(R.grouped_gemm_fp8_blockscaled(codes, scales, w["w2q"], w["w2s"], off_t))
    rows = _sample_rows(off, groups)
    hq_h, hs_h = np_(codes), np_(scales)
    grp = np.searchsorted(off, rows, side="right") - 1
    for gg in np.unique(grp):
        rg = rows[grp == gg]
        q2, s2 = w["_w2_oracle"](gg)
        zero = np.array([0, len(rg)], np.int32)
        C2, Mag2 = O.grouped_gemm(hq_h[rg], hs_h[rg], q2, s2, zero)
        # codes drawn over the whole E4M3 range: the truncation model's clause
        assert_gemm_close(c2[rg], C2, Mag2, what=f"gemm2 group {gg}",
                          model=gemm_model_bound(hq_h[rg], hs_h[rg], q2, s2, zero))


@pytest.mark.parametrize("key", ["dsv3", "moge", "skewed", "skewed_dead"])
def test_fullsize_layer_pieces(key):
    cfg = synth.get_config("skewed" if key == "skewed_dead" else key)
    d = synth.layer_inputs(cfg, dev(), seed=0, weights=True)
    if key == "skewed_dead":
        # four least popular experts receive no token at all
        lo = torch.argsort(d["logits"].mean(0))[:4]
        d["logits"][:, lo] = -30.0
    w = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"))
    idx, gate, xq, xs, perm, io = _route_and_permute(cfg, d)
    E, K, T = cfg["E"], cfg["K"], cfg["T"]
    counts = np.diff(np_(perm["offsets"]))
    assert counts.sum() == T * K
    if cfg["route"]["mode"] == "softmax_grouped":
        assert O.imbalance_score(io, E, cfg["route"]["n_groups"]) == 0.0
        per = E // cfg["route"]["n_groups"]
        assert np.all(counts.reshape(cfg["route"]["n_groups"], per).sum(1) == T)
    if key == "skewed_dead":
        assert (counts == 0).sum() >= 4
    x_np = np_(d["x"])
    # activation quantisation: bit-exact on a row sample
    rs = np.sort(RNG.choice(T, 64, replace=False))
    qo, so = O.quant_act_1x128(x_np[rs])
    assert np.array_equal(np_(xq)[rs], qo) and np.array_equal(np_(xs)[rs], so)
    po = O.permute(io, E)
    # gathered rows are the tokens' rows
    rr = RNG.choice(T * K, 256, replace=False)
    qr, sr = _oracle_rows(x_np, po["src_token"], rr)
    assert np.array_equal(np_(perm["aq"])[rr], qr) and np.array_equal(np_(perm["as"])[rr], sr)
    # GEMMs on sampled experts: smallest, largest, median and random ones
    order = np.argsort(counts)
    nz = order[counts[order] > 0]
    groups = sorted(set([int(nz[0]), int(nz[-1]), int(nz[len(nz) // 2])] +
                        RNG.choice(nz, 3, replace=False).tolist()))
    n_rows = _check_gemm1(cfg, d, perm, w, x_np, po, groups, xq, xs)

    def w2_oracle(g):
        q2, s2 = O.quant_weight_128x128(np_(d["w2"][g:g + 1]))
        assert np.array_equal(np_(w["w2q"][g]), q2[0]) and np.array_equal(np_(w["w2s"][g]), s2[0])
        return q2, s2
    w["_w2_oracle"] = w2_oracle
    _check_gemm2_synthetic(cfg, w, perm["offsets"], po["offsets"], groups)
    n_groups = len(groups)
    print(key, "checked rows", n_rows, "in", n_groups, "experts; load range", counts.min(), counts.max())


def test_fullsize_dsv3_shared_expert_and_combine():
    """Shared expert (one group over all 4096 tokens) and the combine, at the
    DeepSeek-V3 shapes, in the bench's launch configuration."""
    cfg = synth.get_config("dsv3")
    T, H, K, E = cfg["T"], cfg["H"], cfg["K"], cfg["E"]
    d = synth.layer_inputs(cfg, dev(), seed=0, weights=False)
    sw13 = synth.expert_weights(cfg, "sw13", dev())
    sw2 = synth.expert_weights(cfg, "sw2", dev())
    s13q, s13s = R.quant_weight_128x128_e4m3(sw13)
    s2q, s2s = R.quant_weight_128x128_e4m3(sw2)
    s13q_o, s13s_o = O.quant_weight_128x128(np_(sw13))
    s2q_o, s2s_o = O.quant_weight_128x128(np_(sw2))
    assert np.array_equal(np_(s13q), s13q_o) and np.array_equal(np_(s2s), s2s_o)
    xq, xs = R.quant_act_1x128_e4m3(d["x"])
    one = torch.tensor([0, T], dtype=torch.int32, device=dev())
    hq, hs = R.grouped_gemm_fp8_swiglu(xq, xs, s13q, s13s, one)
    x_np = np_(d["x"])
    toks = np.sort(RNG.choice(T, 24, replace=False))
    toks[-1] = T - 1
    aq_o, as_o = O.quant_act_1x128(x_np[toks])
    zero = np.array([0, len(toks)], np.int32)
    C1, Mag1 = O.grouped_gemm(aq_o, as_o, s13q_o, s13s_o, zero)
    hq_o, _, _ = O.swiglu_quant(C1.astype(np.float32))
    frac, _ = check_hidden(np_(hq)[toks], np_(hs)[toks], C1, Mag1, hq_o)
    assert frac < 0.01
    w = dict(w2q=s2q, w2s=s2s, _w2_oracle=lambda g: (s2q_o, s2s_o))
    _check_gemm2_synthetic(dict(cfg, I=cfg["shared_I"]), w, one, np.array([0, T]), [0])
    # combine at full size: generator-made expert outputs, oracle routing
    io, go = O.route_sigmoid_bias(np_(d["logits"]), np_(d["bias"]), K)
    po = O.permute(io, E)
    g = torch.Generator(device=dev())
    g.manual_seed(9)
    y_perm = torch.randn((T * K, H), device=dev(), generator=g)
    shared = torch.randn((T, H), device=dev(), generator=g)
    dst = torch.from_numpy(po["dst_row"]).to(dev())
    gate = torch.from_numpy(go).to(dev())
    y = R.moe_combine(y_perm, dst, gate, shared)
    toks = np.sort(RNG.choice(T, 64, replace=False))
    yp = np_(y_perm)
    sel = po["dst_row"][toks]
    _, bits = O.combine_fp32_replay(yp[sel.ravel()], np.arange(len(toks) * K).reshape(len(toks), K),
                                    go[toks], np_(shared)[toks])
    assert np.array_equal(bf16_bits(y)[toks], bits)


def test_fullsize_backward_transpose_and_dgrad():
    """Block transpose of all 256 experts' quantised 2048x7168 gate projection
    and the dgrad grouped GEMM dX = dY . W with the DeepSeek-V3 routing."""
    cfg = synth.get_config("dsv3")
    E, H, I, T, K = cfg["E"], cfg["H"], cfg["I"], cfg["T"], cfg["K"]
    bcfg = dict(synth.get_config("bwd"), I=I // 2)          # gate projection [E, 2048, 7168]
    wg = synth.expert_weights(bcfg, "w13", dev(), seed=1)
    wq, ws = R.quant_weight_128x128_e4m3(wg)
    qt, st = R.fp8_block_transpose(wq, ws)
    # every expert: the transpose is an exact permutation of the codes and scales
    assert torch.equal(qt, wq.transpose(1, 2))
    assert torch.equal(st, ws.transpose(1, 2))
    # the oracle's own quantise + transpose on sampled experts, and the
    # requantise identity (quantising W^T gives the transposed blocks)
    for e in sorted(set(RNG.choice(E, 3, replace=False).tolist())):
        w_np = np_(wg[e:e + 1])
        qo, so = O.quant_weight_128x128(w_np)
        qto, sto = O.block_transpose(qo, so)
        assert np.array_equal(np_(qt[e]), qto[0]) and np.array_equal(np_(st[e]), sto[0])
    # dgrad with the oracle's routing offsets (an input to both sides)
    d = synth.layer_inputs(cfg, dev(), seed=0, weights=False)
    io, _ = O.route_sigmoid_bias(np_(d["logits"]), np_(d["bias"]), K)
    off = O.permute(io, E)["offsets"]
    M = T * K
    dy = synth.output_grad(M, I, dev(), seed=0)
    dyq, dys = R.quant_act_1x128_e4m3(dy)
    dx = np_(R.grouped_gemm_fp8_blockscaled(dyq, dys, qt, st, torch.from_numpy(off).to(dev())))
    groups = RNG.choice(E, 4, replace=False).tolist()
    rows = _sample_rows(off, groups, per_group=6)
    dy_rows = np_(dy[torch.from_numpy(rows).to(dev())])
    dyq_o, dys_o = O.quant_act_1x128(dy_rows)
    assert np.array_equal(np_(dyq)[rows], dyq_o) and np.array_equal(np_(dys)[rows], dys_o)
    grp = np.searchsorted(off, rows, side="right") - 1
    for g in np.unique(grp):
        sel = grp == g
        qo, so = O.quant_weight_128x128(np_(wg[g:g + 1]))
        qto, sto = O.block_transpose(qo, so)
        zero = np.array([0, int(sel.sum())], np.int32)
        Cx, Mag = O.grouped_gemm(dyq_o[sel], dys_o[sel], qto, sto, zero)
        assert_gemm_close(dx[rows[sel]], Cx, Mag, what=f"dgrad group {g}")
