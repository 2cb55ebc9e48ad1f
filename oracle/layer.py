"""Routed-expert FP8 MoE FFN layer forward, composed from the oracle steps
(oracle; test infrastructure only).

Dataflow ([DSV3-MOE], [DSV3-FP8], [KANANA-FP8], [PANGU-MOGE]):
  route -> quantise x in 1x128 tiles -> permute rows by expert ->
  GEMM1 (gate|up) -> SwiGLU -> quantise h in 1x128 tiles -> GEMM2 (down) ->
  [shared expert: the same three steps on the unpermuted tokens] ->
  gate-weighted combine (+ shared) -> bf16.

``layer_forward`` follows that dataflow with the permutation;
``layer_forward_dense`` evaluates the same mathematics token by token with
no permutation at all, so the two can be compared to pin the permutation and
combine bookkeeping.
"""

import numpy as np

from .codec import bf16_round
from .combine import combine_ref
from .gemm import grouped_gemm
from .permute import permute
from .quant import quant_act_1x128
from .route import route_sigmoid_bias, route_softmax_grouped
from .swiglu import swiglu_quant


def route(logits, bias, rc):
    """rc: dict(mode='sigmoid_bias', K, normalize) or
    dict(mode='softmax_grouped', n_groups, k_per_group)."""
    if rc["mode"] == "sigmoid_bias":
        return route_sigmoid_bias(logits, bias, rc["K"], rc.get("normalize", True))
    return route_softmax_grouped(logits, rc["n_groups"], rc["k_per_group"])


def _expert_ffn(aq, as_, offsets, w13q, w13s, w2q, w2s):
    c1, mag1 = grouped_gemm(aq, as_, w13q, w13s, offsets, with_mag=True)
    hq, hs, _ = swiglu_quant(c1.astype(np.float32))
    c2, mag2 = grouped_gemm(hq, hs, w2q, w2s, offsets, with_mag=True)
    return dict(c1=c1, mag1=mag1, hq=hq, hs=hs, c2=c2, mag2=mag2)


def layer_forward(x, logits, bias, rc, w13q, w13s, w2q, w2s, shared=None):
    """x f32 [T, H]; weights already block-quantised ([G, rows, cols] codes
    and scales).  shared: None or (w13q, w13s, w2q, w2s) with G = 1.
    Every intermediate is the oracle's own (nothing is taken from outside).
    Returns a dict of every intermediate and y (float64 bf16 values, bits)."""
    E = w13q.shape[0]
    idx, gate = route(logits, bias, rc)
    xq, xs = quant_act_1x128(x)
    perm = permute(idx, E, xq, xs)
    routed = _expert_ffn(perm["aq"], perm["as"], perm["offsets"], w13q, w13s, w2q, w2s)
    out = dict(topk_idx=idx, topk_gate=gate, xq=xq, xs=xs, **perm, **routed)
    S = None
    if shared is not None:
        T = x.shape[0]
        sh = _expert_ffn(xq, xs, np.array([0, T], np.int32), *shared)
        S = sh["c2"]
        out.update({"shared_" + k: v for k, v in sh.items()})
    y, y_bits = combine_ref(routed["c2"], perm["dst_row"], gate, S)
    out.update(y=y, y_bits=y_bits)
    return out


def _dot_chunks(aq_row, as_row, bq, bs):
    """One token row against one weight matrix with the chunked formula,
    written as explicit loops over output features (no grouping)."""
    from .codec import e4m3_decode
    a = e4m3_decode(aq_row)
    B = e4m3_decode(bq)
    N, K = B.shape
    out = np.zeros(N)
    for kb in range(K // 128):
        ks = slice(kb * 128, (kb + 1) * 128)
        P = B[:, ks] @ a[ks]
        out += P * (float(as_row[kb]) * np.repeat(np.asarray(bs[:, kb], np.float64), 128))
    return out


def layer_forward_dense(x, logits, bias, rc, w13q, w13s, w2q, w2s, shared=None):
    """Token-by-token evaluation with no permutation (for tiny shapes)."""
    idx, gate = route(logits, bias, rc)
    xq, xs = quant_act_1x128(x)
    T, H = x.shape
    y = np.zeros((T, H))
    for t in range(T):
        acc = np.zeros(H)
        for k in range(idx.shape[1]):
            e = idx[t, k]
            c1 = _dot_chunks(xq[t], xs[t], w13q[e], w13s[e])
            hq, hs, _ = swiglu_quant(c1.astype(np.float32)[None, :])
            c2 = _dot_chunks(hq[0], hs[0], w2q[e], w2s[e])
            acc += float(gate[t, k]) * c2
        if shared is not None:
            s13q, s13s, s2q, s2s = shared
            c1 = _dot_chunks(xq[t], xs[t], s13q[0], s13s[0])
            hq, hs, _ = swiglu_quant(c1.astype(np.float32)[None, :])
            acc += _dot_chunks(hq[0], hs[0], s2q[0], s2s[0])
        y[t] = acc
    return bf16_round(y)
