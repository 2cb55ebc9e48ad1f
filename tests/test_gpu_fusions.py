"""The fused stages against the oracle and against their unfused forms:
routing with the permutation's index maps in one launch
(moe_route_permute), and the down projection with the combine in its
epilogue (grouped_gemm_fp8_combine).  Fusing moves work between launches
(the Pangu page's system optimisation section, operator fusion); it must
not change a bit of any output:

  * moe_route_permute: top-K ids, gates, expert offsets, dst_row and
    src_token equal the oracle's routing and stable permutation (DeepSeek-V3
    page section 2.1, Pangu page MoGE section) bit for bit (grouped-softmax
    gates within one float32 ulp of the oracle's float64 value, like
    moe_route), and equal moe_route + moe_permute bit for bit;
  * grouped_gemm_fp8_combine: c equals grouped_gemm_fp8_blockscaled's c bit
    for bit (and the oracle GEMM within the 1e-4 tolerance), y equals
    moe_combine on that c bit for bit (moe_combine itself is pinned against
    the oracle's binary32 replay in the kernel tests);
  * both keep counters in their workspace between calls: after every call
    they must be back to zero (and no ranking wait may have run out), also
    when one workspace serves calls of different shapes.
"""

import numpy as np
import pytest
import torch

import oracle as O
import routed_experts_fp8_amd as R
from helpers import assert_gemm_close, bf16_bits, dev, np_, to_dev

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(131)
F32 = np.float32
HEADER = 256            # bytes of moe_route_permute's workspace header
CHUNK = 256             # tokens per ranking workgroup


def _rp_counts_zero(ws, T, E):
    """The workspace header (ticket, arrival counters, ready flag and the
    wait-timeout word) is back to zero; the rest is scratch."""
    b = np_(ws)
    assert not b[:HEADER].any(), f"header not reset (T={T}, E={E}): {b[:20].view(np.int32)}"


def _route_case(T, E, K, mode, G=1, Kp=None, normalize=True, bias=True, ties=False):
    logits = RNG.standard_normal((T, E)).astype(F32)
    if ties and T:
        logits[::4, 1] = logits[::4, 0]
        logits[:3] = 0.0
    b = (RNG.standard_normal(E) * 0.01).astype(F32) if (bias and mode == "sigmoid_bias") else None
    return logits, b


ROUTE_CASES = [
    # T, E, K, mode, G, K', normalize, bias
    (0, 64, 8, "sigmoid_bias", 1, None, True, True),
    (1, 8, 2, "sigmoid_bias", 1, None, True, True),
    (15, 16, 4, "sigmoid_bias", 1, None, False, True),
    (16, 64, 8, "sigmoid_bias", 1, None, True, False),
    (17, 64, 8, "sigmoid_bias", 1, None, True, True),
    (255, 256, 8, "sigmoid_bias", 1, None, True, True),
    (256, 256, 8, "sigmoid_bias", 1, None, True, True),
    (257, 256, 8, "sigmoid_bias", 1, None, True, True),
    (1000, 1024, 13, "sigmoid_bias", 1, None, True, True),
    (700, 16, 16, "sigmoid_bias", 1, None, False, True),
    (4096, 256, 8, "sigmoid_bias", 1, None, True, True),      # DeepSeek-V3-shaped routing
    (500, 64, 8, "softmax_grouped", 8, 1, False, False),
    (77, 24, 12, "softmax_grouped", 4, 3, False, False),
    (64, 1024, 16, "softmax_grouped", 8, 2, False, False),
    (4096, 64, 8, "softmax_grouped", 8, 1, False, False),     # MoGE-shaped routing
]


def _check_route_permute(logits, bias, K, mode, G, Kp, normalize, ws):
    T, E = logits.shape
    out = R.moe_route_permute(to_dev(logits), None if bias is None else to_dev(bias), K, mode, n_groups=G,
                              k_per_group=Kp, normalize=normalize, workspace=ws)
    torch.cuda.synchronize()
    if mode == "sigmoid_bias":
        io, go = O.route_sigmoid_bias(logits, bias, K, normalize)
        assert np.array_equal(np_(out["topk_gate"]), go)
    else:
        io, go = O.route_softmax_grouped(logits, G, Kp)
        assert np.all(np.abs(np_(out["topk_gate"]) - go) <= np.spacing(np.abs(go)))
    assert np.array_equal(np_(out["topk_idx"]), io)
    po = O.permute(io, E)
    for k in ("offsets", "dst_row", "src_token"):
        assert np.array_equal(np_(out[k]), po[k]), k
    # the unfused launches give the same bits
    idx2, gate2 = R.moe_route(to_dev(logits), None if bias is None else to_dev(bias), K, mode, n_groups=G,
                              k_per_group=Kp, normalize=normalize)
    p2 = R.moe_permute(idx2, E)
    assert torch.equal(out["topk_idx"], idx2)
    assert torch.equal(out["topk_gate"].view(torch.int32), gate2.view(torch.int32))
    for k in ("offsets", "dst_row", "src_token"):
        assert torch.equal(out[k], p2[k]), k
    _rp_counts_zero(ws, T, E)


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: f"T{c[0]}_E{c[1]}_K{c[2]}_{c[3]}")
def test_route_permute_matches_oracle_and_unfused(case):
    T, E, K, mode, G, Kp, normalize, bias = case
    logits, b = _route_case(T, E, K, mode, G, Kp, normalize, bias, ties=True)
    ws = torch.zeros(R.moe_route_permute_workspace_size(T, K, E), dtype=torch.uint8, device=dev())
    _check_route_permute(logits, b, K, mode, G, Kp, normalize, ws)
    # a second call on the same workspace
    _check_route_permute(logits, b, K, mode, G, Kp, normalize, ws)


def test_route_permute_workspace_reused_across_shapes():
    """One workspace, sized for the largest call, serves a sequence of calls
    of different T, E and K (the counters left by each call are zero)."""
    ws = torch.zeros(R.moe_route_permute_workspace_size(4096, 8, 1024), dtype=torch.uint8, device=dev())
    for case in [ROUTE_CASES[i] for i in (10, 1, 8, 0, 11, 5, 13, 10)]:
        T, E, K, mode, G, Kp, normalize, bias = case
        logits, b = _route_case(T, E, K, mode, G, Kp, normalize, bias)
        _check_route_permute(logits, b, K, mode, G, Kp, normalize, ws)


def test_route_permute_concentrated_and_empty_experts():
    """Every token on the same two experts (all other experts empty)."""
    T, E, K = 600, 64, 2
    logits = np.full((T, E), -5.0, F32)
    logits[:, 5] = 3.0
    logits[:, 63] = 2.0
    logits[::3, 7] = 4.0
    ws = torch.zeros(R.moe_route_permute_workspace_size(T, K, E), dtype=torch.uint8, device=dev())
    _check_route_permute(logits, None, K, "sigmoid_bias", 1, None, True, ws)


# ------------------------------------------------------------------ down projection + combine


def _combine_problem(T, E, topk, N, Kd, shared, skew=0.05):
    p = np.exp(-skew * np.arange(E))
    p /= p.sum()
    idx = np.stack([RNG.choice(E, topk, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    perm = R.moe_permute(to_dev(idx), E)
    M = T * topk
    a = RNG.standard_normal((M, Kd)).astype(F32)
    aq, as_ = O.quant_act_1x128(a)
    bq, bs = O.quant_weight_128x128((RNG.standard_normal((E, N, Kd)) * 0.02).astype(F32))
    gate = RNG.uniform(0, 1, (T, topk)).astype(F32)
    S = RNG.standard_normal((T, N)).astype(F32) if shared else None
    return dict(aq=aq, as_=as_, bq=bq, bs=bs, gate=gate, S=S, perm=perm, idx=idx)


def _run_combine(p, counters):
    aq, as_, bq, bs = (to_dev(p[k]) for k in ("aq", "as_", "bq", "bs"))
    perm = p["perm"]
    gate = to_dev(p["gate"])
    S = None if p["S"] is None else to_dev(p["S"])
    c_ref = R.grouped_gemm_fp8_blockscaled(aq, as_, bq, bs, perm["offsets"])
    y_ref = R.moe_combine(c_ref, perm["dst_row"], gate, S)
    c, y = R.grouped_gemm_fp8_combine(aq, as_, bq, bs, perm["offsets"], perm["src_token"], perm["dst_row"], gate,
                                      S, counters=counters)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int32), c_ref.view(torch.int32)), "c differs from the unfused GEMM"
    assert np.array_equal(bf16_bits(y), bf16_bits(y_ref)), "y differs from the unfused combine"
    assert not counters.any(), "arrival counters not reset"
    return c


COMBINE_CASES = [
    # T, E, topk, N, K (reduction), shared
    (1, 4, 1, 128, 128, False),
    (37, 8, 2, 384, 256, True),          # a half n-tile (N = 384)
    (300, 16, 4, 512, 640, True),
    (257, 64, 8, 256, 2048, True),
    (200, 32, 10, 256, 256, True),       # topk > 8: two slot batches
    (500, 8, 8, 256, 4224, False),       # one tile per workgroup (K above the persistent limit)
    (1024, 256, 8, 1024, 512, True),     # many small groups, some empty
]


@pytest.mark.parametrize("case", COMBINE_CASES, ids=lambda c: "T{}_E{}_k{}_N{}_K{}_{}".format(*c))
def test_gemm_combine_matches_unfused_and_oracle(case):
    T, E, topk, N, Kd, shared = case
    p = _combine_problem(T, E, topk, N, Kd, shared)
    ctr = torch.zeros(max(R.grouped_gemm_fp8_combine_workspace_size(T, N) // 4, 1), dtype=torch.int32,
                      device=dev())
    c = _run_combine(p, ctr)
    c2 = _run_combine(p, ctr)                       # same counters again
    assert torch.equal(c.view(torch.int32), c2.view(torch.int32))
    if T * topk * N * Kd <= 300 * 4 * 512 * 640:
        off = np_(p["perm"]["offsets"])
        C, Mag = O.grouped_gemm(p["aq"], p["as_"], p["bq"], p["bs"], off)
        assert_gemm_close(np_(c), C, Mag, what="combine GEMM")


def test_gemm_combine_counters_reused_across_shapes():
    big = (1024, 256, 8, 1024, 512, True)
    ctr = torch.zeros(R.grouped_gemm_fp8_combine_workspace_size(big[0], big[3]) // 4, dtype=torch.int32,
                      device=dev())
    for case in (big, COMBINE_CASES[1], COMBINE_CASES[4], big, COMBINE_CASES[0]):
        _run_combine(_combine_problem(*case), ctr)


def test_gemm_combine_skewed_load():
    """One expert takes most rows (several m-tiles of one group), others
    none: the arrival counters see tiles of very different lengths."""
    p = _combine_problem(900, 32, 4, 512, 256, True, skew=1.5)
    counts = np.bincount(p["idx"].ravel(), minlength=32)
    assert counts.max() > 600 and (counts == 0).any()
    ctr = torch.zeros(R.grouped_gemm_fp8_combine_workspace_size(900, 512) // 4, dtype=torch.int32, device=dev())
    _run_combine(p, ctr)
