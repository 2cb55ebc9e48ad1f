"""moe_permute_noalloc (the library's static scratch instead of a caller
workspace) against moe_permute (caller workspace), through the C ABI: two
calls in a row on the same GPU, the second with a smaller problem (the
scratch keeps the first call's contents), then the largest problem the
scratch admits; every output bit-identical, including the gathered rows.
The permutation is the stable counting sort of the DeepSeek-V3 page's
no-token-dropping dispatch (section 2.1)."""

import numpy as np
import pytest
import torch

import routed_experts_fp8_amd as R
from helpers import dev, to_dev

pytestmark = pytest.mark.gpu


def _case(T, E, K, H, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    x = rng.standard_normal((T, H)).astype(np.float32)
    xq, xs = R.quant_act_1x128_e4m3(to_dev(x))
    return to_dev(idx), xq, xs


def _same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("gather", [True, False])
def test_permute_noalloc_matches_workspace_entry(gather):
    for T, E, K, H, seed in ((3000, 256, 8, 256, 1), (517, 64, 6, 128, 2), (1, 3, 3, 128, 3)):
        idx, xq, xs = _case(T, E, K, H, seed)
        args = (xq, xs) if gather else (None, None)
        ref = R.moe_permute(idx, E, *args)
        got = R.moe_permute_noalloc(idx, E, *args)
        torch.cuda.synchronize()
        _same(got, ref)


def test_permute_noalloc_at_the_scratch_limit():
    # 8 nblk E + 256 <= 4 MiB: 2047 blocks of 256 tokens at E = 256
    T, E, K = 2047 * 256, 256, 2
    rng = np.random.default_rng(5)
    idx = torch.from_numpy(rng.integers(0, E - 1, (T, 1)).astype(np.int32)).to(dev())
    idx = torch.cat([idx, (idx + 1) % E], dim=1).contiguous()          # two distinct experts per token
    ref = R.moe_permute(idx, E)
    got = R.moe_permute_noalloc(idx, E)
    torch.cuda.synchronize()
    _same(got, ref)
    assert R.moe_permute_workspace_size(T, K, E) <= 4 << 20 < R.moe_permute_workspace_size(T + 256, K, E)
