"""Router projection and the aux-loss-free balancing bias update (oracle;
test infrastructure only).

[DSV3-MOE]: each token's affinity to an expert comes from its router score,
and a per-expert bias term, adjusted to balance the load, shifts the top-K
selection (no auxiliary loss).  The pages say neither how the scores are
computed nor how the bias is adjusted.  Readings taken here:

* Router projection: logits[t, e] = sum_h x[t, h] * W_r[e, h] with the
  layer input x (bf16) and a float32 router weight W_r [E, H] (the gating
  path kept in higher precision than the FP8 expert GEMMs); the oracle is
  that sum, exactly, in float64.
* Bias update, once per training step from the step's per-expert loads
  (the grouped-row counts of the permutation): an expert above the mean load
  has its bias lowered by a fixed step gamma, one below raised by gamma, one
  exactly at the mean left alone:
      b_e <- fl32(b_e - gamma * sign(load_e - mean)),  mean = (T * K) / E.
  The comparison with the mean is exact (integers: load_e * E against
  T * K); the update is one binary32 addition of +-gamma.
"""

import numpy as np

F32 = np.float32


def router_logits(x, w_router):
    """x [T, H] (bf16 values as float32), w_router f32 [E, H] -> float64
    [T, E] = x . W_r^T, and its magnitude sum |x| . |W_r|^T."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w_router, np.float64)
    return x @ w.T, np.abs(x) @ np.abs(w).T


def bias_update(bias, offsets, gamma):
    """bias f32 [E], offsets [E+1] (expert row offsets of the step), gamma
    f32 -> the updated bias (float32)."""
    b = np.asarray(bias, F32)
    off = np.asarray(offsets, np.int64)
    E = len(off) - 1
    load = np.diff(off)
    total = off[-1] - off[0]
    # sign(load_e - total / E), decided on integers
    s = np.sign(load * E - total)
    step = (F32(gamma) * s.astype(F32)).astype(F32)          # exactly +-gamma or 0
    return (b - step).astype(F32)
