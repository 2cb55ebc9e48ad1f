"""Token -> expert routing (oracle; test infrastructure only).

Two modes:

SIGMOID_BIAS  [DSV3-MOE]: each token's affinity to expert e is a sigmoid of
  its router logit; the K experts with the largest affinity are selected; a
  per-expert bias, adjusted elsewhere to balance load, shifts the selection.
  Readings: the bias enters the selection only, not the gate value; the
  selection key is fl32(sigmoid(l_e) + b_e) with the specified binary32
  sigmoid; equal keys are ordered by the lower expert index; slot order is
  key descending; the gate of a selected expert is its sigmoid score,
  optionally normalised over the K selected scores (flag; parity unpinned
  against the pages, which do not say).

SOFTMAX_GROUPED  [PANGU-MOGE]: experts are split into G equal groups; one
  global softmax over all E experts gives the scores; each group keeps its K'
  best experts, all others score 0.  Readings: selection compares logits
  (softmax is strictly increasing in the logit, so the order is the same and
  no exp rounding can create ties); equal logits go to the lower index; slot
  order is group-major, then key descending; the kept scores are not
  renormalised.  The dense top-2 softmax router is the case G = 1, K' = 2.
"""

import numpy as np

from .specmath import spec_sigmoid

F32 = np.float32


def _topk_desc_lower_index(keys, k):
    """Indices of the k largest keys per row, largest first, ties -> lower
    index.  A stable ascending sort of -key keeps equal keys in index order."""
    order = np.argsort(-keys, axis=1, kind="stable")
    return order[:, :k]


def route_sigmoid_bias(logits, bias, K, normalize=True):
    """-> (topk_idx int32 [T, K], topk_gate float32 [T, K])."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 0 < K <= E:
        raise ValueError("need 0 < K <= E")
    s = spec_sigmoid(logits)
    b = np.zeros(E, np.float32) if bias is None else np.asarray(bias, np.float32)
    key = (s + b[None, :]).astype(np.float32)
    idx = _topk_desc_lower_index(key, K).astype(np.int32)
    gate = np.take_along_axis(s, idx, axis=1).astype(np.float32)
    if normalize:
        total = np.zeros(T, np.float32)
        for k in range(K):                       # slot order, binary32
            total = (total + gate[:, k]).astype(np.float32)
        gate = (gate / total[:, None]).astype(np.float32)
    return idx, gate


def route_softmax_grouped(logits, n_groups, k_per_group):
    """-> (topk_idx int32 [T, G*K'], topk_gate float32 [T, G*K'])."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    G, Kp = n_groups, k_per_group
    if G <= 0 or E % G or not 0 < Kp <= E // G:
        raise ValueError("need E % G == 0 and 0 < K' <= E/G")
    l64 = logits.astype(np.float64)
    z = np.exp(l64 - l64.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)                   # float64 softmax
    per = E // G
    idx = np.empty((T, G * Kp), np.int32)
    for g in range(G):
        local = _topk_desc_lower_index(logits[:, g * per:(g + 1) * per], Kp)
        idx[:, g * Kp:(g + 1) * Kp] = local + g * per
    gate = np.take_along_axis(p, idx.astype(np.int64), axis=1).astype(np.float32)
    return idx, gate


def imbalance_score(topk_idx, E, n_groups):
    """Imbalance Score over groups (reading; [PANGU-MOGE] states IS = 0 but
    does not define it): (max_g L_g - min_g L_g) / mean_g L_g with L_g the
    number of picks landing in group g.  It is 0 iff every group carries the
    same load."""
    per = E // n_groups
    loads = np.bincount(np.asarray(topk_idx).ravel() // per, minlength=n_groups)
    return float(loads.max() - loads.min()) / float(loads.mean())
