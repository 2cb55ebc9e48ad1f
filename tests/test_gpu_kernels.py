"""Per-kernel parity of the HIP library against the CPU oracle, through the
C ABI, on seeded inputs that span several tiles, ragged tails and the edge
cases of each step.  Bit-exact for codes, scales, indices, permutations and
transposes; GEMMs within 2^-10 of the oracle's magnitude sum; combine
bit-exact against the documented binary32 order and within 1 bf16 ulp of
the float64 value."""

import numpy as np
import pytest
import torch

import oracle as O
import routed_experts_fp8_amd as R
from helpers import (assert_gemm_close, bf16_bits, bf16_ulp_distance, check_hidden, dev,
                     gemm_model_bound, np_, rand_offsets, to_dev)

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(2024)


# ------------------------------------------------------------------ quantisers


def _act_inputs(rows, cols, rng):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (rows, 1))).astype(np.float32)
    if rows >= 4:
        x[0] = 0.0                                   # amax == 0 tile
        x[1, :128] = -0.0
        x[2] = np.float32(448) * np.exp2(rng.integers(-5, 5, cols)).astype(np.float32)  # exact codes
        x[3, 5::7] = 1e-30                           # tiny values next to normal ones
    return x


@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 640), (300, 7168)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quant_act_bitexact(rows, cols, dtype):
    x = to_dev(_act_inputs(rows, cols, RNG)).to(dtype)
    q, s = R.quant_act_1x128_e4m3(x)
    qo, so = O.quant_act_1x128(np_(x))
    assert np.array_equal(np_(q), qo)
    assert np.array_equal(np_(s), so)


def _encoder_sweep():
    """Values that exercise every rounding decision of the encoder: every
    float32 within +-4 ulp of each E4M3 value and each midpoint, both signs,
    and every bf16 value, all in [-448, 448]."""
    pos = O.e4m3_values()
    centers = np.concatenate([pos, (pos[:-1] + pos[1:]) / 2]).astype(np.float32)
    v = (centers.view(np.int32)[:, None] + np.arange(-4, 5, dtype=np.int32)[None, :]).ravel()
    v = v[v >= 0].view(np.float32)
    bf = (np.arange(0, 1 << 15, dtype=np.uint32) << 16).view(np.float32)
    v = np.concatenate([v, bf[np.isfinite(bf)]])
    v = v[v <= 448.0]
    return np.concatenate([v, -v])


def test_quant_encoder_sweep_bitexact():
    """Rows with one element equal to 448 have scale exactly 1, so the codes
    of the other 127 are the encoder's direct output."""
    v = _encoder_sweep()
    n = len(v)
    rows = (n + 126) // 127
    x = np.zeros((rows, 128), np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(rows * 127, np.float32)
    flat[:n] = v
    x[:, 1:] = flat.reshape(rows, 127)
    q, s = R.quant_act_1x128_e4m3(to_dev(x))
    assert np.all(np_(s) == 1.0)
    assert np.array_equal(np_(q)[:, 1:].ravel()[:n], O.e4m3_encode(v))


@pytest.mark.parametrize("G,rows,cols", [(1, 128, 128), (3, 256, 384)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quant_weight_bitexact(G, rows, cols, dtype):
    w = (RNG.standard_normal((G, rows, cols)) * 0.02).astype(np.float32)
    w[0, :128, :128] = 0.0                               # zero block
    w[-1, -1, -1] = 448.0 * 2 ** -7                      # exact-scale block
    wt = to_dev(w).to(dtype)
    q, s = R.quant_weight_128x128_e4m3(wt)
    qo, so = O.quant_weight_128x128(np_(wt))
    assert np.array_equal(np_(q), qo)
    assert np.array_equal(np_(s), so)


def test_quant_tiny_and_mixed_scales_bitexact():
    """Scales far below 2^-100 (amax ~1e-33 and below, float32 subnormal
    inputs included) next to ordinary ones in the same wavefront and block
    grid: every code and scale still equals the oracle's (quotients taken by
    direct division where the reciprocal of the scale would overflow)."""
    rows = 64
    x = (RNG.standard_normal((rows, 512)) * np.float32(0.3)).astype(np.float32)
    x[::3, :128] *= np.float32(1e-33)                       # s ~ 1e-36 in every third row's first tile
    x[1::4, 256:384] = (RNG.standard_normal((16, 128)) * np.float32(1e-41)).astype(np.float32)  # subnormal inputs
    x[2, 384] = np.float32(-0.0)
    q, sc = R.quant_act_1x128_e4m3(to_dev(x))
    qo, so = O.quant_act_1x128(x)
    assert np.array_equal(np_(q), qo) and np.array_equal(np_(sc), so)
    assert (so < 2.0 ** -100).any() and (so > 2.0 ** -20).any()
    w = (RNG.standard_normal((2, 256, 384)) * 0.02).astype(np.float32)
    w[0, :128, 128:256] *= np.float32(1e-33)
    w[1, 128:, :128] = (RNG.standard_normal((128, 128)) * np.float32(1e-40)).astype(np.float32)
    qw, sw = R.quant_weight_128x128_e4m3(to_dev(w))
    qwo, swo = O.quant_weight_128x128(w)
    assert np.array_equal(np_(qw), qwo) and np.array_equal(np_(sw), swo)
    assert (swo < 2.0 ** -100).any()


# ------------------------------------------------------------------ transpose


@pytest.mark.parametrize("G,rows,cols", [(1, 128, 128), (3, 256, 640), (2, 512, 128)])
def test_block_transpose_bitexact(G, rows, cols):
    q = RNG.integers(0, 256, (G, rows, cols)).astype(np.uint8)
    s = RNG.standard_normal((G, rows // 128, cols // 128)).astype(np.float32)
    qt, st = R.fp8_block_transpose(to_dev(q), to_dev(s))
    qo, so = O.block_transpose(q, s)
    assert np.array_equal(np_(qt), qo) and np.array_equal(np_(st), so)
    q2, s2 = R.fp8_block_transpose(qt, st)
    assert np.array_equal(np_(q2), q) and np.array_equal(np_(s2), s)


@pytest.mark.parametrize("G,rows,cols", [(1, 128, 128), (3, 256, 640), (2, 512, 128)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quant_weight_with_transposed_copy(G, rows, cols, dtype):
    """The weight quantisation writing the block-transposed copy in the same
    pass: the forward codes as without it, the copy equal to the oracle's
    transpose of the oracle's codes and to the separate transpose kernel."""
    w = (RNG.standard_normal((G, rows, cols)) * 0.02).astype(np.float32)
    w[0, :128, :128] = 0.0
    wt = to_dev(w).to(dtype)
    q, s, qt, st = R.quant_weight_128x128_e4m3_t(wt)
    qo, so = O.quant_weight_128x128(np_(wt))
    assert np.array_equal(np_(q), qo) and np.array_equal(np_(s), so)
    qto, sto = O.block_transpose(qo, so)
    assert np.array_equal(np_(qt), qto) and np.array_equal(np_(st), sto)
    qt2, st2 = R.fp8_block_transpose(q, s)
    assert torch.equal(qt, qt2) and torch.equal(st, st2)


def test_block_transpose_equals_requantised_transpose():
    w = (RNG.standard_normal((2, 256, 384)) * 0.006).astype(np.float32)
    q, s = R.quant_weight_128x128_e4m3(to_dev(w))
    qt, st = R.fp8_block_transpose(q, s)
    qo, so = O.quant_weight_128x128(np.ascontiguousarray(w.transpose(0, 2, 1)))
    assert np.array_equal(np_(qt), qo) and np.array_equal(np_(st), so)


# ------------------------------------------------------------------ routing


@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (300, 64, 8), (257, 256, 8), (50, 1000, 13), (20, 8, 8),
                                   (33, 130, 130)])
@pytest.mark.parametrize("normalize", [True, False])
def test_route_sigmoid_bitexact(T, E, K, normalize):
    logits = RNG.standard_normal((T, E)).astype(np.float32)
    bias = (RNG.standard_normal(E) * 0.01).astype(np.float32)
    idx, gate = R.moe_route(to_dev(logits), to_dev(bias), K, "sigmoid_bias", normalize=normalize)
    io, go = O.route_sigmoid_bias(logits, bias, K, normalize)
    assert np.array_equal(np_(idx), io)
    assert np.array_equal(np_(gate), go)


def test_route_sigmoid_ties_and_no_bias():
    T, E, K = 200, 96, 8
    logits = RNG.choice(np.array([-2.0, -0.5, 0.0, 0.5, 3.0], np.float32), (T, E))
    logits[:10] = 0.0                                  # all-equal rows -> experts 0..K-1
    idx, gate = R.moe_route(to_dev(logits), None, K, "sigmoid_bias")
    io, go = O.route_sigmoid_bias(logits, None, K)
    assert np.array_equal(np_(idx), io) and np.array_equal(np_(gate), go)
    assert np.array_equal(np_(idx)[:10], np.tile(np.arange(K), (10, 1)))


def test_sigmoid_spec_dense_sweep():
    """With K = E and no normalisation every gate is sigmoid(logit): sweep
    ~4M logits across [-90, 90] (the clamp included) bit for bit."""
    E = 1024
    vals = np.concatenate([np.linspace(-90, 90, 3_000_000, dtype=np.float32),
                           RNG.standard_normal(1_000_000).astype(np.float32)])
    T = (len(vals) + E - 1) // E
    logits = np.zeros(T * E, np.float32)
    logits[:len(vals)] = vals
    logits = logits.reshape(T, E)
    idx, gate = R.moe_route(to_dev(logits), None, E, "sigmoid_bias", normalize=False)
    idx = np_(idx).astype(np.int64)
    expect = O.spec_sigmoid(np.take_along_axis(logits, idx, axis=1))
    assert np.array_equal(np_(gate), expect)


@pytest.mark.parametrize("T,E,G,Kp", [(256, 8, 1, 2), (500, 64, 8, 1), (77, 24, 4, 3), (64, 1024, 8, 2)])
def test_route_grouped(T, E, G, Kp):
    logits = RNG.standard_normal((T, E)).astype(np.float32)
    logits[::5, 1] = logits[::5, 0]                     # exact ties
    idx, gate = R.moe_route(to_dev(logits), None, G * Kp, "softmax_grouped", n_groups=G, k_per_group=Kp)
    io, go = O.route_softmax_grouped(logits, G, Kp)
    assert np.array_equal(np_(idx), io)
    g = np_(gate)
    ulp = np.spacing(np.abs(go))
    assert np.all(np.abs(g - go) <= ulp), np.max(np.abs(g - go) / ulp)
    assert O.imbalance_score(np_(idx), E, G) == 0.0 if G > 1 else True


# ------------------------------------------------------------------ permutation


def _rand_idx(T, E, K, rng, skew=0.0):
    p = np.exp(-skew * np.arange(E))
    p /= p.sum()
    return np.stack([rng.choice(E, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)


@pytest.mark.parametrize("T,E,K,H", [(1, 4, 2, 128), (255, 64, 8, 256), (256, 8, 2, 512), (257, 256, 8, 384),
                                     (1000, 1024, 4, 128), (700, 16, 16, 128),
                                     # many 256-token blocks: the scan splits each expert's blocks
                                     # into runs (E = 128: 8 runs; E = 7: 128 runs, most empty;
                                     # E = 1024: one run)
                                     (20000, 128, 8, 128), (5000, 7, 3, 128), (3000, 1024, 4, 128)])
def test_permute_bitexact(T, E, K, H):
    idx = _rand_idx(T, E, K, RNG, skew=0.05)
    xq = RNG.integers(0, 256, (T, H)).astype(np.uint8)
    xs = RNG.standard_normal((T, H // 128)).astype(np.float32)
    out = R.moe_permute(to_dev(idx), E, to_dev(xq), to_dev(xs))
    po = O.permute(idx, E, xq, xs)
    for k in ("offsets", "dst_row", "src_token", "aq", "as"):
        assert np.array_equal(np_(out[k]), po[k]), k


def test_permute_empty_and_concentrated():
    T, E, K = 600, 64, 2
    idx = np.stack([np.array([5, 63])] * T).astype(np.int32)
    idx[::3] = [7, 5]
    out = R.moe_permute(to_dev(idx), E)
    po = O.permute(idx, E)
    for k in ("offsets", "dst_row", "src_token"):
        assert np.array_equal(np_(out[k]), po[k]), k
    out0 = R.moe_permute(torch.zeros((0, K), dtype=torch.int32, device=dev()), E)
    assert np.all(np_(out0["offsets"]) == 0)


# ------------------------------------------------------------------ grouped GEMM


def _gemm_problem(sizes, N, K, rng, integer=False):
    M = int(sum(sizes))
    G = len(sizes)
    if integer:
        a = rng.integers(-8, 9, (M, K)).astype(np.float32)
        b = rng.integers(-8, 9, (G, N, K)).astype(np.float32)
        aq, bq = O.e4m3_encode(a), O.e4m3_encode(b)
        as_ = np.ones((M, K // 128), np.float32)
        bs = np.ones((G, N // 128, K // 128), np.float32)
    else:
        a = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-4, 4, (M, 1)))).astype(np.float32)
        b = (rng.standard_normal((G, N, K)) * 0.02).astype(np.float32)
        aq, as_ = O.quant_act_1x128(a)
        bq, bs = O.quant_weight_128x128(b)
    return aq, as_, bq, bs, rand_offsets(rng, sizes)


GEMM_CASES = [
    ([5, 0, 17, 1], 256, 384),
    ([0, 16, 15, 129, 128, 300, 0], 384, 640),
    ([64], 128, 128),
    ([1] * 40, 128, 256),
    ([257, 3], 512, 1024),
]


@pytest.mark.parametrize("sizes,N,K", GEMM_CASES)
def test_grouped_gemm_f32(sizes, N, K):
    aq, as_, bq, bs, off = _gemm_problem(sizes, N, K, RNG)
    c = R.grouped_gemm_fp8_blockscaled(to_dev(aq), to_dev(as_), to_dev(bq), to_dev(bs), to_dev(off))
    C, Mag = O.grouped_gemm(aq, as_, bq, bs, off)
    assert_gemm_close(np_(c), C, Mag, what=f"gemm {sizes} N={N} K={K}")


@pytest.mark.parametrize("sizes,N,K", GEMM_CASES[:3])
def test_grouped_gemm_bf16_is_rounded_f32(sizes, N, K):
    aq, as_, bq, bs, off = _gemm_problem(sizes, N, K, RNG)
    args = [to_dev(v) for v in (aq, as_, bq, bs, off)]
    c32 = R.grouped_gemm_fp8_blockscaled(*args)
    c16 = R.grouped_gemm_fp8_blockscaled(*args, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_bits(c16), bf16_bits(c32.to(torch.bfloat16)))


def _random_codes(rng, shape):
    """E4M3 codes of magnitude 2^-3 .. 2^4 with random signs (no NaN)."""
    return (rng.integers(0x20, 0x58, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)


@pytest.mark.parametrize("K", [128, 384])
def test_grouped_gemm_many_tiles_short_k(K):
    """800 tiles with K of one or three 128-chunks: each workgroup runs
    several tiles back to back, its load stream crossing tile boundaries
    (up to two tiles ahead at K = 128), with ragged one-row m-tiles.
    Operands are random codes and scales (the GEMM's contract)."""
    sizes = [161, 1, 40, 100] * 40
    G, M, N = len(sizes), sum(sizes), 1024
    aq, bq = _random_codes(RNG, (M, K)), _random_codes(RNG, (G, N, K))
    as_ = RNG.uniform(0.5, 2.0, (M, K // 128)).astype(np.float32)
    bs = RNG.uniform(0.5, 2.0, (G, N // 128, K // 128)).astype(np.float32)
    off = rand_offsets(RNG, sizes)
    args = [to_dev(v) for v in (aq, as_, bq, bs, off)]
    c = R.grouped_gemm_fp8_blockscaled(*args)
    C, Mag = O.grouped_gemm(aq, as_, bq, bs, off)
    # codes over 7 binades at one or three chunks: the truncation model's clause
    assert_gemm_close(np_(c), C, Mag, what=f"short K={K}", model=gemm_model_bound(aq, as_, bq, bs, off))
    # fused SwiGLU over the same tile stream (I = 512: 4 tiles per m-tile)
    hq, hs = R.grouped_gemm_fp8_swiglu(*args)
    hq2, hs2 = R.swiglu(c)
    assert np.array_equal(np_(hq), np_(hq2)) and np.array_equal(np_(hs), np_(hs2))
    # the same operand gathered from a shuffled source through a row index:
    # identical bits, tile switches now reloading gathered row offsets
    perm = RNG.permutation(M)
    src_q, src_s = np.empty_like(aq), np.empty_like(as_)
    src_q[perm], src_s[perm] = aq, as_
    a_row = to_dev(perm.astype(np.int32))
    cg = R.grouped_gemm_fp8_blockscaled_gather(to_dev(src_q), to_dev(src_s), a_row, args[2], args[3], args[4])
    assert torch.equal(cg, c)
    hg, hsg = R.grouped_gemm_fp8_swiglu(to_dev(src_q), to_dev(src_s), args[2], args[3], args[4], a_row=a_row)
    assert torch.equal(hg, hq) and torch.equal(hsg, hs)


@pytest.mark.parametrize("K", [384, 7168])
def test_grouped_gemm_row_gather(K):
    """Rows gathered through an index with repeats (several grouped rows read
    one source row, as tokens do across their top-K experts): equal to the
    GEMM on the explicitly gathered operand, and within tolerance of the
    oracle on it.  K = 7168 runs one tile per workgroup, K = 384 the
    persistent tile walk."""
    sizes = [5, 0, 17, 1, 300, 161]
    G, M, N, A = len(sizes), sum(sizes), 256, 97
    src_q, src_s, bq, bs, off = _gemm_problem([A] + [0] * (G - 1), N, K, RNG)
    a_row_np = RNG.integers(0, A, M).astype(np.int32)
    off = rand_offsets(RNG, sizes)
    aq, as_ = src_q[a_row_np], src_s[a_row_np]
    w = [to_dev(v) for v in (bq, bs, off)]
    c = R.grouped_gemm_fp8_blockscaled_gather(to_dev(src_q), to_dev(src_s), to_dev(a_row_np), *w)
    assert torch.equal(c, R.grouped_gemm_fp8_blockscaled(to_dev(aq), to_dev(as_), *w))
    C, Mag = O.grouped_gemm(aq, as_, bq, bs, off)
    assert_gemm_close(np_(c), C, Mag, what=f"row gather K={K}")
    if K == 384:
        bq2, bs2 = O.quant_weight_128x128((RNG.standard_normal((G, 2 * N, K)) * 0.02).astype(np.float32))
        w2 = [to_dev(v) for v in (bq2, bs2, off)]
        hq, hs = R.grouped_gemm_fp8_swiglu(to_dev(src_q), to_dev(src_s), *w2, a_row=to_dev(a_row_np))
        hq2, hs2 = R.grouped_gemm_fp8_swiglu(to_dev(aq), to_dev(as_), *w2)
        assert torch.equal(hq, hq2) and torch.equal(hs, hs2)


def _random_problem(sizes, N, K, rng):
    """Random codes and scales (the GEMM's contract takes any)."""
    G, M = len(sizes), int(sum(sizes))
    aq, bq = _random_codes(rng, (M, K)), _random_codes(rng, (G, N, K))
    as_ = rng.uniform(0.5, 2.0, (M, K // 128)).astype(np.float32)
    bs = rng.uniform(0.5, 2.0, (G, N // 128, K // 128)).astype(np.float32)
    return aq, as_, bq, bs, rand_offsets(rng, sizes)


def test_grouped_gemm_at_the_limits():
    """The two size limits of the grouped GEMM: 1024 groups (every
    workgroup's tile table then scans 1024 group offsets, two per thread),
    mostly empty or 1-3 rows with a few long and ragged ones; and K = 65536
    (512 chunks, one tile per workgroup).  Both against the oracle, the
    fused SwiGLU against the unfused GEMM + standalone SwiGLU."""
    sizes = list(RNG.integers(0, 4, 1024))
    sizes[7], sizes[500], sizes[1023] = 161, 300, 17
    aq, as_, bq, bs, off = _random_problem(sizes, 256, 256, RNG)
    args = [to_dev(v) for v in (aq, as_, bq, bs, off)]
    c = R.grouped_gemm_fp8_blockscaled(*args)
    C, Mag = O.grouped_gemm(aq, as_, bq, bs, off)
    assert_gemm_close(np_(c), C, Mag, what="1024 groups, K=256",
                      model=gemm_model_bound(aq, as_, bq, bs, off))
    hq, hs = R.grouped_gemm_fp8_swiglu(*args)
    hq2, hs2 = R.swiglu(c)
    assert torch.equal(hq, hq2) and torch.equal(hs, hs2)
    aq, as_, bq, bs, off = _random_problem([3, 0, 17], 128, 65536, RNG)
    c = R.grouped_gemm_fp8_blockscaled(*[to_dev(v) for v in (aq, as_, bq, bs, off)])
    C, Mag = O.grouped_gemm(aq, as_, bq, bs, off)
    assert_gemm_close(np_(c), C, Mag, what="K=65536")


def test_grouped_gemm_exact_integers():
    """Integer codes with unit scales: every partial sum is an integer below
    2^24, so the float32 result must equal the exact integer product."""
    aq, as_, bq, bs, off = _gemm_problem([3, 70, 0, 33], 256, 1024, RNG, integer=True)
    c = R.grouped_gemm_fp8_blockscaled(to_dev(aq), to_dev(as_), to_dev(bq), to_dev(bs), to_dev(off))
    C, _ = O.grouped_gemm(aq, as_, bq, bs, off)
    assert np.array_equal(np_(c).astype(np.float64), C)


def test_grouped_gemm_fused_swiglu():
    I, H = 256, 384
    sizes = [0, 16, 15, 129, 64, 300, 1]
    aq, as_, bq, bs, off = _gemm_problem(sizes, 2 * I, H, RNG)
    args = [to_dev(v) for v in (aq, as_, bq, bs, off)]
    hq, hs = R.grouped_gemm_fp8_swiglu(*args)
    # (1) same as the unfused GEMM followed by the standalone SwiGLU kernel
    c1 = R.grouped_gemm_fp8_blockscaled(*args)
    hq2, hs2 = R.swiglu(c1)
    assert np.array_equal(np_(hq), np_(hq2)) and np.array_equal(np_(hs), np_(hs2))
    # (2) against the oracle: the GEMM is within tolerance, so h codes agree
    # except next to rounding boundaries, where they may differ by one step
    C1, Mag1 = O.grouped_gemm(aq, as_, bq, bs, off)
    hqo, hso, h = O.swiglu_quant(C1.astype(np.float32))
    frac, _ = check_hidden(np_(hq), np_(hs), C1, Mag1, hqo)
    assert frac < 0.01


@pytest.mark.parametrize("M,I", [(1, 128), (300, 256), (77, 2048)])
def test_swiglu_bitexact(M, I):
    gu = (RNG.standard_normal((M, 2 * I)) * 3).astype(np.float32)
    gu[0, :I] = 0.0
    hq, hs = R.swiglu(to_dev(gu))
    hqo, hso, _ = O.swiglu_quant(gu)
    assert np.array_equal(np_(hq), hqo) and np.array_equal(np_(hs), hso)


# ------------------------------------------------------------------ combine


@pytest.mark.parametrize("T,K,H,shared", [(1, 1, 128, False), (100, 8, 512, True), (33, 2, 7168, True)])
def test_combine(T, K, H, shared):
    y = RNG.standard_normal((T * K, H)).astype(np.float32)
    dst = RNG.permutation(T * K).reshape(T, K).astype(np.int32)
    gate = RNG.uniform(0, 1, (T, K)).astype(np.float32)
    S = RNG.standard_normal((T, H)).astype(np.float32) if shared else None
    out = R.moe_combine(to_dev(y), to_dev(dst), to_dev(gate), None if S is None else to_dev(S))
    _, bits_replay = O.combine_fp32_replay(y, dst, gate, S)
    assert np.array_equal(bf16_bits(out), bits_replay)
    # against the exact sum: one bf16 ulp, widened under cancellation by the
    # float32 accumulation bound (K products and K adds, plus the shared add,
    # each within 2^-24 of the running magnitude sum)
    ref, bits_ref = O.combine_ref(y.astype(np.float64), dst, gate, S)
    d = bf16_ulp_distance(bf16_bits(out), bits_ref)
    mag = sum(np.abs(gate[:, k:k + 1].astype(np.float64) * y[dst[:, k]]) for k in range(K))
    if S is not None:
        mag = mag + np.abs(S)
    got = np_(out.float()).astype(np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) * 2 ** 16
    far = d > 1
    assert np.all(np.abs(got - ref)[far] <= ulp[far] + (2 * K + 1) * 2.0 ** -24 * mag[far])
    assert far.mean() < 1e-3


@pytest.mark.parametrize("K", [640, 4224])
def test_grouped_gemm_large_groups(K):
    """Groups of hundreds of rows, several m-tiles each (K = 640: the
    persistent tile walk; K = 4224: one tile per workgroup): ragged groups
    (a 3-row one, an empty one), a half weight tile (N = 384), against the
    oracle; bf16 output equal to the rounded float32 output; row gather;
    the fused SwiGLU equal to the unfused GEMM + SwiGLU."""
    sizes = [1000, 0, 700, 3]
    aq, as_, bq, bs, off = _gemm_problem(sizes, 384, K, RNG)
    args = [to_dev(v) for v in (aq, as_, bq, bs, off)]
    c = R.grouped_gemm_fp8_blockscaled(*args)
    C, Mag = O.grouped_gemm(aq, as_, bq, bs, off)
    assert_gemm_close(np_(c), C, Mag, what=f"large groups K={K}")
    c16 = R.grouped_gemm_fp8_blockscaled(*args, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_bits(c16), bf16_bits(c.to(torch.bfloat16)))
    M = int(off[-1])
    perm = RNG.permutation(M)
    src_q, src_s = np.empty_like(aq), np.empty_like(as_)
    src_q[perm], src_s[perm] = aq, as_
    cg = R.grouped_gemm_fp8_blockscaled_gather(to_dev(src_q), to_dev(src_s), to_dev(perm.astype(np.int32)),
                                               *args[2:])
    assert torch.equal(cg, c)
    I = 256
    aq2, as2, bq2, bs2, off2 = _gemm_problem([900, 5, 700], 2 * I, K, RNG)
    args2 = [to_dev(v) for v in (aq2, as2, bq2, bs2, off2)]
    hq, hs = R.grouped_gemm_fp8_swiglu(*args2)
    c1 = R.grouped_gemm_fp8_blockscaled(*args2)
    hq2, hs2 = R.swiglu(c1)
    assert torch.equal(hq, hq2) and torch.equal(hs, hs2)
    C1, Mag1 = O.grouped_gemm(aq2, as2, bq2, bs2, off2)
    assert_gemm_close(np_(c1), C1, Mag1, what=f"large groups gate|up K={K}")
