"""Parity of the input-side backward and the FP8 weight gradients at the full
DeepSeek-V3 layer size, in the launch configuration the bench times
(weights quantised with their transposed copies in one pass, MoEForward with
its float32 gate|up output kept, MoEBackward, MoEWeightGrad),
checked on every grouped row of sampled experts (the least and most loaded
ones and a random one) against the oracle's own chain for those experts:
its own quantised weights, forward rows, combine gradient, dgrad GEMMs,
SwiGLU backward and 128x1-quantised weight-gradient operands.  The weight
gradients are compared on sampled output-feature rows of each sampled
expert (the oracle computes those rows in full)."""

import numpy as np
import pytest
import torch

import oracle as O
import routed_experts_fp8_amd as R
import synth
from helpers import GEMM_RTOL, assert_gemm_close, dequant_rows, dev, np_, trunc_model_bound

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(83)
F32 = np.float32


def _deq_t(q, s):
    """Dequantise a [C, n] 128x1 operand whose scales are [C, n/128]."""
    return O.e4m3_decode(q) * np.repeat(np.asarray(s, np.float64), 128, axis=1)


def _gpu_operand(qt, st, p0, n_pad):
    """Expert slice [C, n_pad] of the GPU's [C, ld] codes and tile-major
    [ld/128, C] scales, scales returned as [C, n_pad/128]."""
    q = np_(qt[:, p0:p0 + n_pad])
    s = np.ascontiguousarray(np_(st[p0 // 128:(p0 + n_pad) // 128, :]).T)
    return q, s


def _wgrad_check(name, dw_gpu_rows, aq, as_, bq, bs, aq_g, as_g, bq_g, bs_g, o_rows):
    """dW rows o_rows of one expert: GPU vs oracle within max(GEMM_RTOL of the
    magnitude sum, the matrix instruction's truncation model: the reduction
    runs over the expert's few hundred rows) plus the effect of the operand
    codes that differ."""
    p = np.array([0, aq.shape[1]], np.int32)
    C, Mag = O.wgrad_gemm(aq[o_rows], as_[o_rows], bq, bs, p)
    A, B = _deq_t(aq[o_rows], as_[o_rows]), _deq_t(bq, bs)
    dA = np.abs(_deq_t(aq_g[o_rows], as_g[o_rows]) - A)
    dB = np.abs(_deq_t(bq_g, bs_g) - B)
    extra = dA @ (np.abs(B) + dB).T + np.abs(A) @ dB.T
    model = trunc_model_bound(np.abs(A) + dA, np.abs(B) + dB)
    bound = np.maximum(GEMM_RTOL * (Mag[0] + extra), model) + extra + 1e-30
    err = np.abs(dw_gpu_rows.astype(np.float64) - C[0])
    assert np.all(err <= bound), f"{name}: worst ratio {np.max(err / bound):.3g}"
    return float(np.max(err / (Mag[0] + 1e-300)))


def test_fullsize_dsv3_backward_and_weight_gradients():
    cfg = synth.get_config("dsv3")
    T, H, E, I, K = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["K"]
    d = synth.layer_inputs(cfg, dev(), seed=0)
    # the training-step path: quantisation writing the transposed copies too
    w, wt = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"), transposed=True)
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev(), fused=False, shared_I=cfg.get("shared_I"))
    fwd(d["x"], d["logits"], d["bias"])
    dy = synth.output_grad(T, H, dev(), seed=4)
    bwd = R.MoEBackward(fwd, wt, weight_grad=True)
    bwd(dy, d["logits"])
    wg = R.MoEWeightGrad(bwd)
    out = wg(d["x"], dy)
    torch.cuda.synchronize()

    # the oracle's own routing and permutation (bit-exact with the GPU's)
    logits, bias = np_(d["logits"]), np_(d["bias"])
    io, go = O.route_sigmoid_bias(logits, bias, K, True)
    po = O.permute(io, E)
    off, src, dst = po["offsets"], po["src_token"], po["dst_row"]
    assert np.array_equal(np_(fwd.buf["offsets"]), off) and np.array_equal(np_(fwd.buf["src_token"]), src)
    gate_row = np.zeros(T * K, F32)
    gate_row[dst.ravel()] = go.ravel()
    poff = O.padded_offsets(off)
    assert np.array_equal(np_(wg.buf["poff"]), poff)
    x_np, dy_np = np_(d["x"]), np_(dy)

    counts = np.diff(off)
    order = np.argsort(counts, kind="stable")
    nz = order[counts[order] > 0]
    experts = sorted({int(nz[0]), int(nz[-1]), int(RNG.choice(nz))})
    b = {k: v for k, v in bwd.buf.items()}
    stats = []
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        n = r1 - r0
        rows = np.arange(r0, r1)
        one = np.array([0, n], np.int32)
        q13, s13 = O.quant_weight_128x128(np_(d["w13"][e:e + 1]))
        q2, s2 = O.quant_weight_128x128(np_(d["w2"][e:e + 1]))
        # forward rows of this expert
        aq, as_ = O.quant_act_1x128(x_np[src[rows]])
        C1, _ = O.grouped_gemm(aq, as_, q13, s13, one, with_mag=False)
        c1 = C1.astype(F32)
        # combine gradient: bit-exact codes
        dc2 = (gate_row[rows][:, None] * dy_np[src[rows]]).astype(F32)
        dc2q, dc2s = O.quant_act_1x128(dc2)
        assert np.array_equal(np_(b["dc2q"][r0:r1]), dc2q) and np.array_equal(np_(b["dc2s"][r0:r1]), dc2s)
        # down dgrad from identical codes: GEMM tolerance
        q2t, s2t = O.block_transpose(q2, s2)
        DH, MagH = O.grouped_gemm(dc2q, dc2s, q2t, s2t, one)
        assert_gemm_close(np_(b["dh"][r0:r1]), DH, MagH, what=f"down dgrad expert {e}")
        # SwiGLU backward on the oracle's own c1 and dh: codes may flip at
        # rounding boundaries (the GPU's c1 and dh are float32 GEMM results)
        dq1, ds1, d1 = O.swiglu_backward(c1, DH.astype(F32))
        g_dq1, g_ds1 = np_(b["dq1"][r0:r1]), np_(b["ds1"][r0:r1])
        flip = float(np.mean(g_dq1 != dq1))
        assert flip < 0.01, flip
        # gate|up dgrad: GEMM tolerance plus the differing codes through |W13|
        q13t, s13t = O.block_transpose(q13, s13)
        DX, MagX = O.grouped_gemm(dq1, ds1, q13t, s13t, one)
        W13 = O.dequant_weight(q13, s13)[0]                    # [2I, H]
        dd = np.abs(dequant_rows(g_dq1, g_ds1) - dequant_rows(dq1, ds1))
        extra = dd @ np.abs(W13)
        err = np.abs(np_(b["dxp"][r0:r1]).astype(np.float64) - DX)
        assert np.all(err <= GEMM_RTOL * (MagX + extra) + extra + 1e-30), f"gate|up dgrad expert {e}"
        # weight-gradient operands of this expert: the GPU's padded slice
        p0, n_pad = int(poff[e]), int(poff[e + 1] - poff[e])
        wb = wg.buf
        dq_o, ds_o, _ = O.quant_act_128x1_grouped(dc2, one)
        _, _, h = O.swiglu_quant(c1)
        hq_o, hs_o, _ = O.quant_act_128x1_grouped(h, one)
        d1q_o, d1s_o, _ = O.quant_act_128x1_grouped(d1, one)
        xq_o, xs_o, _ = O.quant_act_128x1_grouped(x_np[src[rows]], one)
        g_dc2t = _gpu_operand(wb["dc2t"], wb["dc2ts"], p0, n_pad)
        g_ht = _gpu_operand(wb["ht"], wb["hts"], p0, n_pad)
        g_d1t = _gpu_operand(wb["d1t"], wb["d1ts"], p0, n_pad)
        g_xt = _gpu_operand(wb["xt"], wb["xts"], p0, n_pad)
        assert np.array_equal(g_dc2t[0], dq_o) and np.array_equal(g_dc2t[1], ds_o)
        assert np.array_equal(g_xt[0], xq_o) and np.array_equal(g_xt[1], xs_o)
        assert np.mean(g_ht[0] != hq_o) < 0.01 and np.mean(g_d1t[0] != d1q_o) < 0.01
        # sampled output-feature rows: one random 128-row block and the last rows
        o2 = np.unique(np.concatenate([128 * RNG.integers(0, H // 128) + np.arange(128), np.arange(H - 8, H)]))
        r2 = _wgrad_check(f"dW2 expert {e}", np_(out["dw2"][e][o2]), dq_o, ds_o, hq_o, hs_o,
                          *g_dc2t, *g_ht, o2)
        o13 = np.unique(np.concatenate([128 * RNG.integers(0, 2 * I // 128) + np.arange(128),
                                        np.arange(2 * I - 8, 2 * I), np.arange(I - 4, I + 4)]))
        r13 = _wgrad_check(f"dW13 expert {e}", np_(out["dw13"][e][o13]), d1q_o, d1s_o, xq_o, xs_o,
                           *g_d1t, *g_xt, o13)
        stats.append((e, n, flip, r2, r13))
    print("expert, rows, dC1 code flips, dW2 / dW13 worst err/mag:", stats)
    # bf16 weight gradients of every expert at full size (the 16-byte store
    # path of the persistent tile walk): exactly the float32 results rounded
    # once to nearest-even
    wb = wg.buf
    for name, ops, ref in (("dW2", (wb["dc2t"], wb["dc2ts"], wb["ht"], wb["hts"]), out["dw2"]),
                           ("dW13", (wb["d1t"], wb["d1ts"], wb["xt"], wb["xts"]), out["dw13"])):
        cb = R.grouped_wgrad_fp8(*ops, wb["poff"], out_dtype=torch.bfloat16)
        assert cb.data_ptr() % 16 == 0
        for g in range(E):
            assert torch.equal(cb[g], ref[g].to(torch.bfloat16)), f"bf16 {name} expert {g}"
        del cb
