"""CPU oracle for the routed-expert FP8 MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this package.  The product path (the HIP library and its Python binding)
never calls it, and it shares no code, constants or helpers with that path.

Everything here is plain numpy, written so that each function can be checked
against the pages by eye:

* floating-point results that the method defines exactly (dequantised dot
  products, the combine) are computed in float64;
* steps whose *result is an integer decided by floating point* (an FP8 code,
  a top-K selection) are taken in IEEE binary32, in the same precision the
  GPU kernels use, with numpy float32 ufuncs (one rounding per operation, no
  contraction).

Sources, cited in every function by these keys:

[KANANA-FP8]  "Kakao Kanana-2 pre-training deep dive" (devday.kr), the
              paragraph on FP8 Tensor-Core training: activations quantised in
              1x128 tiles and weights in 128x128 blocks (the DeepSeek-V3
              fine-grained scheme); one MoE quantisation kernel covering every
              expert's weights and activations instead of a per-expert loop;
              only the forward FP8 weights are stored and the backward pass
              transposes the block-quantised weights.
[DSV3-MOE]    "DeepSeek-V3 technical report summary" (theinnovators.zone),
              section 2.1 "Model architecture", DeepSeekMoE bullets: shared
              and routed experts are separate; a sigmoid affinity score is
              followed by top-K expert selection; a per-expert bias term is
              adjusted to balance load without an auxiliary loss; no tokens
              are dropped.
[DSV3-FP8]    same page, section 2.2, "FP8 mixed-precision training" bullets:
              most GEMMs run in FP8; 1x128 tile / 128x128 block quantisation;
              accumulation is promoted to higher precision.
[PANGU-MOGE]  "Huawei releases open-weight models trained on Ascend"
              (amuse.peoplentools.com), section introducing Mixture of Grouped
              Experts: experts split into equal-size groups, each token picks
              a fixed number of experts in every group, scores come from one
              global softmax and unselected experts score 0, which makes the
              Imbalance Score 0 by construction.

``oracle.native`` holds plain C forms of the weight quantiser, the E4M3
encoder, the GEMM rows and the sigmoid (``oracle_c.c``), for full-size
checks; they restate the numpy definitions step for step and are held to
them bit for bit by ``tests/test_oracle_native.py``.

Readings of points the pages leave open (format, rounding, tie-break, gate
normalisation, SwiGLU) are stated at the function that takes them.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, invariants or library routines, except the
input-side readings listed as "parity unpinned" in the module that holds
them (gate normalisation flag, shared-expert size).
"""

from .codec import (E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_encode_bruteforce,
                    bf16_round, e4m3_values)
from .specmath import spec_exp, spec_sigmoid, spec_silu
from .quant import quant_act_1x128, quant_weight_128x128, dequant_act, dequant_weight
from .route import route_sigmoid_bias, route_softmax_grouped, imbalance_score
from .permute import permute
from .gemm import grouped_gemm, grouped_gemm_rows
from .swiglu import swiglu_quant
from .combine import combine_ref, combine_fp32_replay
from .backward import (combine_backward, swiglu_backward, route_backward_sigmoid,
                       route_backward_softmax, layer_backward)
from .transpose import block_transpose
from .wgrad import padded_offsets, grouped_rows, quant_act_128x1_grouped, wgrad_gemm, layer_wgrad
from .router import router_logits, bias_update
from .layer import layer_forward, layer_forward_dense

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "e4m3_encode_bruteforce", "bf16_round",
    "e4m3_values", "spec_exp", "spec_sigmoid", "spec_silu", "quant_act_1x128",
    "quant_weight_128x128", "dequant_act", "dequant_weight", "route_sigmoid_bias",
    "route_softmax_grouped", "imbalance_score", "permute", "grouped_gemm",
    "grouped_gemm_rows", "swiglu_quant", "combine_ref", "combine_fp32_replay",
    "block_transpose", "layer_forward", "layer_forward_dense", "combine_backward",
    "swiglu_backward", "route_backward_sigmoid", "route_backward_softmax", "layer_backward",
    "padded_offsets", "grouped_rows", "quant_act_128x1_grouped", "wgrad_gemm", "layer_wgrad",
    "router_logits", "bias_update",
]
