"""Backward of the routed-expert FP8 layer, input side (oracle; test
infrastructure only).

[KANANA-FP8]: only the forward FP8 weights are stored, and the backward
pass uses the block-transposed copies of them; the expert GEMMs of the
backward run in FP8 like the forward ones ([DSV3-FP8]: most GEMMs, forward
and backward, in FP8 with 1x128 / 128x128 scaling).  The pages give no more
detail, so every step below is a reading, stated where it is taken:

* Gradients flow straight through the FP8 rounding (the quantiser is treated
  as the identity in the backward pass).
* Every GEMM input of the backward is quantised in 1x128 tiles along its own
  reduction dimension (H for the combine gradient, 2I for the gate|up
  gradient), exactly like the forward activations.
* The SwiGLU derivative and the gate-scaled combine gradient are binary32
  sequences written out below, because their results are quantised (an
  integer decided by floating point): both implementations must take the same
  binary32 steps.  Sums of many terms (the gate gradient's dot product, the
  router gradient) are float64 here.
* The router gradient flows only through the selected experts' scores: top-K
  selection is piecewise constant, and the balancing bias enters the
  selection only ([DSV3-MOE]), so it receives no gradient.
"""

import numpy as np

from .quant import quant_act_1x128
from .specmath import spec_sigmoid

F32 = np.float32


def combine_backward(dy, c2, dst_row, gate):
    """Gradient of y[t] = sum_k gate[t,k] * c2[dst_row[t,k]] (+ shared[t]).

    dy f32 [T, H] (values of the bf16 upstream gradient), c2 f32 [T*K, H],
    dst_row [T, K], gate f32 [T, K] ->
      (dc2q u8 [T*K, H], dc2s f32 [T*K, H/128], dc2 f32 [T*K, H],
       d_gate f64 [T, K]).
    dc2[dst_row[t,k]] = fl32(gate[t,k] * dy[t]) (one binary32 product),
    quantised in 1x128 tiles for the FP8 dgrad GEMM; d_gate[t,k] is the
    float64 dot product of dy[t] with that expert's output row.  The shared
    expert's gradient is dy itself."""
    dy = np.asarray(dy, np.float32)
    c2 = np.asarray(c2, np.float32)
    dst = np.asarray(dst_row, np.int64)
    g = np.asarray(gate, np.float32)
    T, K = dst.shape
    H = dy.shape[1]
    dc2 = np.zeros((T * K, H), np.float32)
    d_gate = np.zeros((T, K))
    for k in range(K):
        dc2[dst[:, k]] = (g[:, k:k + 1] * dy).astype(np.float32)
        d_gate[:, k] = np.sum(dy.astype(np.float64) * c2[dst[:, k]].astype(np.float64), axis=1)
    dc2q, dc2s = quant_act_1x128(dc2)
    return dc2q, dc2s, dc2, d_gate


def swiglu_backward(gate_up, dh):
    """Gradient of h = silu(g) * u, g = gate_up[:, :I], u = gate_up[:, I:].

    gate_up f32 [M, 2I] (the forward's float32 gate|up output), dh f32 [M, I]
    -> (dq u8 [M, 2I], ds f32 [M, 2I/128], d f32 [M, 2I]) with d = [dg | du]
    quantised in 1x128 tiles along 2I for the FP8 dgrad GEMM.

    Reading, as binary32 steps (silu'(g) = s + g s (1 - s) = s (1 + g (1 - s))
    with s the specified sigmoid):
      s = sigmoid(g); silu = g * s
      ds = s * (1 + g * (1 - s))
      du = dh * silu;  dg = (dh * u) * ds."""
    gu = np.asarray(gate_up, np.float32)
    dh = np.asarray(dh, np.float32)
    M, twoI = gu.shape
    I = twoI // 2
    g, u = gu[:, :I], gu[:, I:]
    one = F32(1.0)
    s = spec_sigmoid(g)
    silu = (g * s).astype(np.float32)
    t = (one - s).astype(np.float32)
    t = (g * t).astype(np.float32)
    t = (one + t).astype(np.float32)
    dsilu = (s * t).astype(np.float32)
    du = (dh * silu).astype(np.float32)
    dg = ((dh * u).astype(np.float32) * dsilu).astype(np.float32)
    d = np.concatenate([dg, du], axis=1)
    dq, ds = quant_act_1x128(d)
    return dq, ds, d


def route_backward_sigmoid(logits, topk_idx, topk_gate, d_gate, normalize=True):
    """Router gradient for the sigmoid mode (float64).

    gate_k = s_k / S (normalised; S = sum of the K selected scores) or s_k,
    with s_k = sigmoid(logit of the k-th selected expert).  Then
      dL/ds_k = (d_gate_k - sum_j d_gate_j gate_j) / S   (normalised)
              = d_gate_k                                  (not normalised)
      dL/dlogit_e = dL/ds_k * s_k (1 - s_k) for e = topk_idx[k], else 0.
    The scores are recomputed in float64 from the logits."""
    l = np.asarray(logits, np.float64)
    idx = np.asarray(topk_idx, np.int64)
    dg = np.asarray(d_gate, np.float64)
    T, E = l.shape
    s = 1.0 / (1.0 + np.exp(-np.take_along_axis(l, idx, axis=1)))
    if normalize:
        S = s.sum(axis=1, keepdims=True)
        gate = s / S
        ds = (dg - np.sum(dg * gate, axis=1, keepdims=True)) / S
    else:
        ds = dg
    d_logits = np.zeros((T, E))
    np.put_along_axis(d_logits, idx, ds * s * (1.0 - s), axis=1)
    return d_logits


def route_backward_softmax(logits, topk_idx, d_gate):
    """Router gradient for the grouped-softmax mode (float64).

    gate_k = p[topk_idx[k]] with p = softmax(logits) over all E experts (not
    renormalised), so dL/dlogit_j = p_j (D_j - sum_k d_gate_k gate_k) with
    D_j = d_gate_k where j = topk_idx[k], else 0."""
    l = np.asarray(logits, np.float64)
    idx = np.asarray(topk_idx, np.int64)
    dg = np.asarray(d_gate, np.float64)
    T, E = l.shape
    z = l - l.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    gate = np.take_along_axis(p, idx, axis=1)
    D = np.zeros((T, E))
    np.put_along_axis(D, idx, dg, axis=1)
    return p * (D - np.sum(dg * gate, axis=1, keepdims=True))


def layer_backward(fwd, dy, logits, rc, w13q, w13s, w2q, w2s, shared=None):
    """Input-side backward of ``layer_forward`` (dgrad of x and of the router
    logits), composed from the steps above and the forward's own GEMM and
    block transpose:

      combine backward -> dC2 (1x128 FP8) and d_gate
      GEMM2 dgrad   dH  = dC2 . W2      (B operand: block-transposed W2)
      SwiGLU backward on the forward's float32 gate|up output -> dC1 (FP8)
      GEMM1 dgrad   dXp = dC1 . W13     (B operand: block-transposed W13)
      shared expert: the same chain from dy with one group
      dx[t] = sum_k dXp[dst_row[t,k]] + dx_shared[t]   (float64, then bf16)
      router: route_backward_* from d_gate.

    fwd: the dict returned by layer_forward; dy f32 [T, H] (bf16 values).
    Expert outputs and gate|up outputs enter as float32 (the forward keeps
    them in float32).  Returns a dict with every intermediate, dx (float64
    bf16 values and bits) and d_logits (float64)."""
    from .codec import bf16_round
    from .gemm import grouped_gemm
    from .transpose import block_transpose
    dy = np.asarray(dy, np.float32)
    T = dy.shape[0]
    off = fwd["offsets"]
    dst = fwd["dst_row"]
    dc2q, dc2s, _, d_gate = combine_backward(dy, fwd["c2"].astype(np.float32), dst, fwd["topk_gate"])
    w2tq, w2ts = block_transpose(w2q, w2s)
    dh, mag_dh = grouped_gemm(dc2q, dc2s, w2tq, w2ts, off)
    dq1, ds1, d1 = swiglu_backward(fwd["c1"].astype(np.float32), dh.astype(np.float32))
    w13tq, w13ts = block_transpose(w13q, w13s)
    dxp, mag_dxp = grouped_gemm(dq1, ds1, w13tq, w13ts, off)
    out = dict(dc2q=dc2q, dc2s=dc2s, d_gate=d_gate, dh=dh, mag_dh=mag_dh, dq1=dq1, ds1=ds1, d1=d1,
               dxp=dxp, mag_dxp=mag_dxp)
    dx = np.zeros(dy.shape)
    for k in range(dst.shape[1]):
        dx += dxp[dst[:, k]]
    if shared is not None:
        s13q, s13s, s2q, s2s = shared
        one = np.array([0, T], np.int32)
        dyq, dys = quant_act_1x128(dy)
        s2tq, s2ts = block_transpose(s2q, s2s)
        dhs, mag_dhs = grouped_gemm(dyq, dys, s2tq, s2ts, one)
        dq1s, ds1s, d1s = swiglu_backward(fwd["shared_c1"].astype(np.float32), dhs.astype(np.float32))
        s13tq, s13ts = block_transpose(s13q, s13s)
        dxs, mag_dxs = grouped_gemm(dq1s, ds1s, s13tq, s13ts, one)
        dx += dxs
        out.update(shared_dyq=dyq, shared_dys=dys, shared_dh=dhs, shared_mag_dh=mag_dhs,
                   shared_dq1=dq1s, shared_ds1=ds1s, shared_d1=d1s, shared_dx=dxs, shared_mag_dx=mag_dxs)
    dx_val, dx_bits = bf16_round(dx)
    if rc["mode"] == "sigmoid_bias":
        d_logits = route_backward_sigmoid(logits, fwd["topk_idx"], fwd["topk_gate"], d_gate,
                                          rc.get("normalize", True))
    else:
        d_logits = route_backward_softmax(logits, fwd["topk_idx"], d_gate)
    out.update(dx_f64=dx, dx=dx_val, dx_bits=dx_bits, d_logits=d_logits)
    return out
