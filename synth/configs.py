"""Workload table: the five layer shapes exercised by tests and the bench.

Shapes follow the pages' models: a DeepSeek-V3-shaped layer (256 routed
experts + 1 shared, top-8 sigmoid routing with a balancing bias), a
Pangu-style MoGE layer (64 experts in 8 groups, global softmax, top-1 per
group), a skewed-load layer, a tiny layer for exhaustive checks, and the
backward-side block transpose + dgrad on the DeepSeek-V3 expert weights.
"""

CONFIGS = {
    # tiny layer: dense top-2 softmax router == grouped mode with G = 1, K' = 2
    "tiny": dict(
        name="tiny_t256_h512_e8_top2softmax_i256",
        T=256, H=512, E=8, I=256, K=2,
        route=dict(mode="softmax_grouped", n_groups=1, k_per_group=2),
        shared_I=None, x_dtype="f32", w_dtype="f32", w_std=0.02, bias_std=None,
        zipf_beta=None),
    # DeepSeek-V3-shaped layer
    "dsv3": dict(
        name="dsv3_t4096_h7168_e256_top8sigmoid_i2048_shared1",
        T=4096, H=7168, E=256, I=2048, K=8,
        route=dict(mode="sigmoid_bias", K=8, normalize=True),
        shared_I=2048, x_dtype="bf16", w_dtype="bf16", w_std=0.006, bias_std=0.01,
        zipf_beta=None),
    # MoGE group-balanced routing
    "moge": dict(
        name="moge_t8192_h5120_e64_g8_top1pergroup_i1408",
        T=8192, H=5120, E=64, I=1408, K=8,
        route=dict(mode="softmax_grouped", n_groups=8, k_per_group=1),
        shared_I=None, x_dtype="bf16", w_dtype="bf16", w_std=0.02, bias_std=None,
        zipf_beta=None),
    # skewed per-expert load from Zipf-like logit offsets
    "skewed": dict(
        name="skewed_t16384_h2048_e128_top8sigmoid_i768",
        T=16384, H=2048, E=128, I=768, K=8,
        route=dict(mode="sigmoid_bias", K=8, normalize=True),
        shared_I=None, x_dtype="bf16", w_dtype="bf16", w_std=0.02, bias_std=None,
        zipf_beta=0.2),
    # backward side: transpose of all experts' block-quantised 2048x7168 gate
    # projection, then dX = dY . W per expert with the dsv3 routing
    "bwd": dict(
        name="bwd_dsv3_transpose_e256_2048x7168_dgrad_m32768",
        T=4096, H=7168, E=256, I=2048, K=8,
        route=dict(mode="sigmoid_bias", K=8, normalize=True),
        shared_I=None, x_dtype="bf16", w_dtype="bf16", w_std=0.006, bias_std=0.01,
        zipf_beta=None),
}


def get_config(key):
    return dict(CONFIGS[key])
