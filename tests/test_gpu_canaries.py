"""Guard bands and canaries around every output of the library's kernels, at
ragged shapes (partial tiles, empty groups, one-row groups, a half weight
tile, K = 1 routing, padded weight-gradient operands).

Each kernel runs twice, into outputs pre-filled with 0x00 and with 0xFF,
each between 4 KiB guard bands of the same byte.  Every element the entry
point documents as written must come out identical in both runs (an
element left unwritten keeps its fill and differs), the documented
unwritten regions must keep their fill, and no guard byte may change (no
write past either end of a buffer).  DeepSeek-V3 page section 2.1: no
token is dropped, so every grouped row exists and is written."""

import numpy as np
import pytest
import torch

import oracle as O
import routed_experts_fp8_amd as R
from helpers import Guarded, dev, rand_offsets, to_dev

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(97)
F32 = np.float32


def _run_twice(outs, call):
    """outs: {name: (shape, dtype)}; call(bufs) runs the kernel into the
    given tensors.  Returns ({name: bytes of the 0x00 run}, {.. 0xFF run})."""
    res = []
    for fill in (0x00, 0xFF):
        g = {k: Guarded(s, dt, fill) for k, (s, dt) in outs.items()}
        call({k: v.t for k, v in g.items()})
        torch.cuda.synchronize()
        for k, v in g.items():
            assert v.bands_intact(), f"{k}: a guard band changed (fill {fill:#x})"
        res.append({k: v.bytes() for k, v in g.items()})
    return res


def _all_written(outs, call):
    a, b = _run_twice(outs, call)
    for k in outs:
        assert np.array_equal(a[k], b[k]), f"{k}: elements left unwritten"
    return a


def _gemm_operands(sizes, N, K):
    M = int(sum(sizes))
    a = RNG.standard_normal((M, K)).astype(F32)
    aq, as_ = O.quant_act_1x128(a)
    bq, bs = O.quant_weight_128x128((RNG.standard_normal((len(sizes), N, K)) * 0.02).astype(F32))
    return [to_dev(v) for v in (aq, as_, bq, bs, rand_offsets(RNG, sizes))], M


SIZES = [5, 0, 17, 1, 300, 161, 0, 33]
LARGE = [1000, 0, 700, 3]          # several full m-tiles per group


@pytest.mark.parametrize("sizes", [SIZES, LARGE])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,K", [(384, 256), (256, 4224)])
def test_gemm_output_bands(sizes, dtype, N, K):
    """N = 384: the last 256-row weight tile is half past N; K = 4224: one
    tile per workgroup (above the persistent walk's limit)."""
    args, M = _gemm_operands(sizes, N, K)
    _all_written({"c": ((M, N), dtype)}, lambda o: R.grouped_gemm_fp8_blockscaled(*args, c=o["c"]))
    perm = RNG.permutation(M).astype(np.int32)
    src_q, src_s = torch.empty_like(args[0]), torch.empty_like(args[1])
    src_q[torch.from_numpy(perm).long().to(dev())] = args[0]
    src_s[torch.from_numpy(perm).long().to(dev())] = args[1]
    _all_written({"c": ((M, N), dtype)}, lambda o: R.grouped_gemm_fp8_blockscaled_gather(
        src_q, src_s, to_dev(perm), *args[2:], c=o["c"]))


@pytest.mark.parametrize("sizes", [SIZES, LARGE])
@pytest.mark.parametrize("K", [256, 4224])
def test_fused_swiglu_output_bands(sizes, K):
    I = 384
    args, M = _gemm_operands(sizes, 2 * I, K)
    _all_written({"hq": ((M, I), torch.uint8), "hs": ((M, I // 128), torch.float32)},
                 lambda o: R.grouped_gemm_fp8_swiglu(*args, hq=o["hq"], hs=o["hs"]))
    c1 = R.grouped_gemm_fp8_blockscaled(*args)
    _all_written({"hq": ((M, I), torch.uint8), "hs": ((M, I // 128), torch.float32)},
                 lambda o: R.swiglu(c1, hq=o["hq"], hs=o["hs"]))


def test_route_permute_combine_bands():
    T, E, K, H = 333, 40, 6, 264
    logits = to_dev(RNG.standard_normal((T, E)).astype(F32))
    bias = to_dev((RNG.standard_normal(E) * 0.01).astype(F32))
    o = _all_written({"idx": ((T, K), torch.int32), "gate": ((T, K), torch.float32)},
                     lambda o: R.moe_route(logits, bias, K, topk_idx=o["idx"], topk_gate=o["gate"]))
    idx = to_dev(o["idx"].view(np.int32).reshape(T, K))
    _all_written({"idx": ((T, 1), torch.int32), "gate": ((T, 1), torch.float32)},
                 lambda o: R.moe_route(logits, None, 1, topk_idx=o["idx"], topk_gate=o["gate"]))
    lg = to_dev(RNG.standard_normal((T, 48)).astype(F32))
    _all_written({"idx": ((T, 8), torch.int32), "gate": ((T, 8), torch.float32)},
                 lambda o: R.moe_route(lg, None, 8, "softmax_grouped", n_groups=8, k_per_group=1,
                                       topk_idx=o["idx"], topk_gate=o["gate"]))
    Hq = 384
    xq, xs = R.quant_act_1x128_e4m3(to_dev(RNG.standard_normal((T, Hq)).astype(F32)))
    outs = {"offsets": ((E + 1,), torch.int32), "dst_row": ((T, K), torch.int32),
            "src_token": ((T * K,), torch.int32), "aq": ((T * K, Hq), torch.uint8),
            "as": ((T * K, Hq // 128), torch.float32)}
    p = _all_written(outs, lambda o: R.moe_permute(idx, E, xq, xs, out=o))
    dst = to_dev(p["dst_row"].view(np.int32).reshape(T, K))
    gate = to_dev(RNG.uniform(0, 1, (T, K)).astype(F32))
    y_perm = to_dev(RNG.standard_normal((T * K, H)).astype(F32))
    shared = to_dev(RNG.standard_normal((T, H)).astype(F32))
    for sh in (shared, None):
        _all_written({"y": ((T, H), torch.bfloat16)},
                     lambda o: R.moe_combine(y_perm, dst, gate, sh, out=o["y"]))


def test_fused_stage_bands():
    """moe_route_permute writes every element of its five outputs; the down
    projection with the fused combine writes every element of c and y."""
    T, E, K = 333, 40, 6
    logits = to_dev(RNG.standard_normal((T, E)).astype(F32))
    bias = to_dev((RNG.standard_normal(E) * 0.01).astype(F32))
    ws = torch.zeros(R.moe_route_permute_workspace_size(T, K, E), dtype=torch.uint8, device=dev())
    outs = {"topk_idx": ((T, K), torch.int32), "topk_gate": ((T, K), torch.float32),
            "offsets": ((E + 1,), torch.int32), "dst_row": ((T, K), torch.int32),
            "src_token": ((T * K,), torch.int32)}
    o = _all_written(outs, lambda o: R.moe_route_permute(logits, bias, K, workspace=ws, out=o))
    idx = to_dev(o["topk_idx"].view(np.int32).reshape(T, K))
    perm = R.moe_permute(idx, E)
    N, Kd = 384, 256                                    # a half n-tile
    aq, as_ = O.quant_act_1x128(RNG.standard_normal((T * K, Kd)).astype(F32))
    bq, bs = O.quant_weight_128x128((RNG.standard_normal((E, N, Kd)) * 0.02).astype(F32))
    gate = to_dev(RNG.uniform(0, 1, (T, K)).astype(F32))
    shared = to_dev(RNG.standard_normal((T, N)).astype(F32))
    ctr = torch.zeros(R.grouped_gemm_fp8_combine_workspace_size(T, N) // 4, dtype=torch.int32, device=dev())
    _all_written({"c": ((T * K, N), torch.float32), "y": ((T, N), torch.bfloat16)},
                 lambda o: R.grouped_gemm_fp8_combine(to_dev(aq), to_dev(as_), to_dev(bq), to_dev(bs),
                                                      perm["offsets"], perm["src_token"], perm["dst_row"], gate,
                                                      shared, c=o["c"], y=o["y"], counters=ctr))
    assert not ctr.any()


def test_quantiser_and_transpose_bands():
    x = to_dev(RNG.standard_normal((77, 640)).astype(F32))
    _all_written({"q": ((77, 640), torch.uint8), "s": ((77, 5), torch.float32)},
                 lambda o: R.quant_act_1x128_e4m3(x, q=o["q"], scale=o["s"]))
    w = to_dev((RNG.standard_normal((3, 256, 384)) * 0.02).astype(F32)).to(torch.bfloat16)
    outs = {"q": ((3, 256, 384), torch.uint8), "s": ((3, 2, 3), torch.float32)}
    _all_written(outs, lambda o: R.quant_weight_128x128_e4m3(w, q=o["q"], scale=o["s"]))
    outs.update(qt=((3, 384, 256), torch.uint8), st=((3, 3, 2), torch.float32))
    r = _all_written(outs, lambda o: R.quant_weight_128x128_e4m3_t(w, q=o["q"], scale=o["s"], qt=o["qt"],
                                                                   scale_t=o["st"]))
    q = to_dev(r["q"].reshape(3, 256, 384))
    s = to_dev(r["s"].view(np.float32).reshape(3, 2, 3))
    _all_written({"qt": ((3, 384, 256), torch.uint8), "st": ((3, 3, 2), torch.float32)},
                 lambda o: R.fp8_block_transpose(q, s, qt=o["qt"], scale_t=o["st"]))


def test_backward_kernel_bands():
    T, K, H, E, I = 61, 4, 256, 16, 384
    M = T * K
    dy = to_dev(RNG.standard_normal((T, H)).astype(F32)).to(torch.bfloat16)
    y_perm = to_dev(RNG.standard_normal((M, H)).astype(F32))
    dst = to_dev(RNG.permutation(M).astype(np.int32).reshape(T, K))
    gate = to_dev(RNG.uniform(0, 1, (T, K)).astype(F32))
    _all_written({"dq": ((M, H), torch.uint8), "ds": ((M, H // 128), torch.float32),
                  "dg": ((T, K), torch.float32), "gr": ((M,), torch.float32)},
                 lambda o: R.moe_combine_backward(dy, y_perm, dst, gate, dq=o["dq"], ds=o["ds"],
                                                  d_gate=o["dg"], gate_row=o["gr"]))
    gu = to_dev((RNG.standard_normal((M, 2 * I)) * 3).astype(F32))
    dh = to_dev(RNG.standard_normal((M, I)).astype(F32))
    _all_written({"dq": ((M, 2 * I), torch.uint8), "ds": ((M, 2 * I // 128), torch.float32),
                  "d": ((M, 2 * I), torch.float32)},
                 lambda o: R.swiglu_backward(gu, dh, dq=o["dq"], ds=o["ds"], d=o["d"]))
    logits = to_dev(RNG.standard_normal((T, E)).astype(F32))
    idx, _ = R.moe_route(logits, None, K)
    dgate = to_dev(RNG.standard_normal((T, K)).astype(F32))
    _all_written({"dl": ((T, E), torch.float32)},
                 lambda o: R.moe_route_backward(logits, idx, dgate, d_logits=o["dl"]))


def test_wgrad_operand_padding_and_output_bands():
    """The 128x1 quantiser writes expert g's rows then zero codes up to its
    padded end, and nothing past P_G (those columns keep their fill); the
    weight-gradient GEMM writes every element of every expert's gradient,
    zeros for an expert without rows."""
    sizes = [0, 1, 127, 129, 0, 300, 5]
    off = rand_offsets(RNG, sizes)
    M, C, G = int(off[-1]), 256, len(sizes)
    ld = R.moe_wgrad_padded_rows(M, G) + 256                 # a stride beyond the smallest one
    x = to_dev(RNG.standard_normal((M, C)).astype(F32))
    pg = O.padded_offsets(off)
    P = int(pg[-1])
    outs = {"qt": ((C, ld), torch.uint8), "st": ((ld // 128, C), torch.float32), "p": ((G + 1,), torch.int32)}
    a, b = _run_twice(outs, lambda o: R.quant_act_128x1_grouped_e4m3(
        x, to_dev(off), ld=ld, qt=o["qt"], st=o["st"], padded_offsets=o["p"]))
    qa, qb = a["qt"].reshape(C, ld), b["qt"].reshape(C, ld)
    assert np.array_equal(qa[:, :P], qb[:, :P])                       # every padded row written
    assert (qa[:, P:] == 0x00).all() and (qb[:, P:] == 0xFF).all()    # nothing past P_G
    for g in range(G):                                                 # padding rows are +0 codes
        assert (qa[:, int(pg[g]) + sizes[g]:int(pg[g + 1])] == 0).all()
    sa, sb = a["st"].reshape(ld // 128, C * 4), b["st"].reshape(ld // 128, C * 4)
    assert np.array_equal(sa[:P // 128], sb[:P // 128])
    assert (sa[P // 128:] == 0x00).all() and (sb[P // 128:] == 0xFF).all()
    assert np.array_equal(a["p"], b["p"]) and np.array_equal(a["p"].view(np.int32), pg)
    qt, st, p = R.quant_act_128x1_grouped_e4m3(x, to_dev(off), ld=ld)
    y = to_dev(RNG.standard_normal((M, 384)).astype(F32))
    qt2, st2, _ = R.quant_act_128x1_grouped_e4m3(y, to_dev(off), ld=ld)
    for dtype in (torch.float32, torch.bfloat16):
        _all_written({"c": ((G, C, 384), dtype)},
                     lambda o: R.grouped_wgrad_fp8(qt, st, qt2, st2, p, c=o["c"]))
