"""The routed-expert FP8 MoE FFN layer forward, as a sequence of library
calls (no host synchronisation inside).

Dataflow ([DSV3-MOE] shared + routed experts, sigmoid top-K with bias, no
dropping; [PANGU-MOGE] grouped softmax routing; [DSV3-FP8] / [KANANA-FP8]
fine-grained FP8):

  quant_act_1x128_e4m3(x) -> moe_route -> moe_permute (index maps) ->
  grouped_gemm_fp8_swiglu (expert-grouped rows gathered from x's FP8 codes
  through src_token; gate|up GEMM, SwiGLU and 1x128 quantisation fused) ->
  grouped_gemm_fp8_blockscaled (down projection, float32) -> moe_combine
  (gate-weighted sum + shared expert, bf16).

The shared expert (the same two GEMMs, one group over the unpermuted
tokens) runs on a side stream from the quantisation on and joins before the
combine.

Weights are quantised ahead of the forward (``quantize_weights``), as in
training where quantisation runs once per optimizer step for all experts.
"""

import torch

from . import _lib as L


def quantize_weights(w13, w2, sw13=None, sw2=None):
    """All experts' 128x128-block FP8 weights in one launch per matrix."""
    q = {}
    q["w13q"], q["w13s"] = L.quant_weight_128x128_e4m3(w13)
    q["w2q"], q["w2s"] = L.quant_weight_128x128_e4m3(w2)
    if sw13 is not None:
        q["sw13q"], q["sw13s"] = L.quant_weight_128x128_e4m3(sw13)
        q["sw2q"], q["sw2s"] = L.quant_weight_128x128_e4m3(sw2)
    return q


class MoEForward:
    """Preallocated buffers for one layer shape; ``__call__`` enqueues the
    whole forward on the current stream and returns y (bf16 [T, H])."""

    def __init__(self, T, H, E, I, route, weights, device, fused=True, shared_I=None, overlap_shared=True):
        self.T, self.H, self.E, self.I = T, H, E, I
        self.route = dict(route)
        self.K = route["K"] if route["mode"] == "sigmoid_bias" else route["n_groups"] * route["k_per_group"]
        self.w = weights
        self.fused = fused
        self.shared_I = shared_I
        K, M = self.K, T * self.K
        dev = device
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.buf = dict(
            idx=e((T, K), torch.int32), gate=e((T, K), torch.float32),
            xq=e((T, H), torch.uint8), xs=e((T, H // 128), torch.float32),
            offsets=e((E + 1,), torch.int32), dst_row=e((T, K), torch.int32),
            src_token=e((M,), torch.int32),
            hq=e((M, I), torch.uint8), hs=e((M, I // 128), torch.float32),
            c2=e((M, H), torch.float32), y=e((T, H), torch.bfloat16),
            ws=e((L.moe_permute_workspace_size(T, K, E),), torch.uint8),
            one_group=torch.tensor([0, T], dtype=torch.int32, device=dev),
        )
        if not fused:
            self.buf["c1"] = e((M, 2 * I), torch.float32)
        # The shared expert only needs x's FP8 codes, so it can run on a side
        # stream beside the permutation and the routed GEMMs: its GEMMs are
        # dense and compute-heavy while the routed ones stream weights from
        # HBM, and the two fill each other's idle units.
        self.side = torch.cuda.Stream(device=dev) if (shared_I and overlap_shared) else None
        if shared_I:
            self.buf.update(shq=e((T, shared_I), torch.uint8), shs=e((T, shared_I // 128), torch.float32),
                            sc2=e((T, H), torch.float32))
            if not fused:
                self.buf["sc1"] = e((T, 2 * shared_I), torch.float32)

    def _ffn(self, aq, as_, offsets, w13q, w13s, w2q, w2s, hq, hs, c2, c1, mark, a_row=None):
        if self.fused:
            L.grouped_gemm_fp8_swiglu(aq, as_, w13q, w13s, offsets, hq=hq, hs=hs, a_row=a_row)
        else:
            L.grouped_gemm_fp8_blockscaled(aq, as_, w13q, w13s, offsets, c=c1, a_row=a_row)
            L.swiglu(c1, hq=hq, hs=hs)
        mark("gemm1")
        L.grouped_gemm_fp8_blockscaled(hq, hs, w2q, w2s, offsets, c=c2)
        mark("gemm2")

    def __call__(self, x, logits, bias=None, on_stage=None):
        """Enqueue the forward.  on_stage(name), if given, is called after each
        stage is enqueued on the caller's stream (the bench records a HIP event
        there).  With the shared expert on the side stream its GEMMs are not
        marked; "shared_join" marks the caller's stream waiting for them."""
        mark = on_stage or (lambda name: None)
        b, w, r = self.buf, self.w, self.route
        shared = None

        def route():
            if r["mode"] == "sigmoid_bias":
                L.moe_route(logits, bias, self.K, "sigmoid_bias", normalize=r.get("normalize", True),
                            topk_idx=b["idx"], topk_gate=b["gate"])
            else:
                L.moe_route(logits, None, self.K, "softmax_grouped", n_groups=r["n_groups"],
                            k_per_group=r["k_per_group"], topk_idx=b["idx"], topk_gate=b["gate"])
            mark("route")

        def quant():
            L.quant_act_1x128_e4m3(x, q=b["xq"], scale=b["xs"])
            mark("quant_act")

        def fork():  # shared expert on the side stream
            nonlocal shared
            if self.shared_I and self.side is not None:
                self.side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(self.side):
                    self._ffn(b["xq"], b["xs"], b["one_group"], w["sw13q"], w["sw13s"], w["sw2q"], w["sw2s"],
                              b["shq"], b["shs"], b["sc2"], b.get("sc1"), lambda n: None)
                shared = b["sc2"]

        def permute():
            # index maps only: GEMM1 gathers its rows from x's codes through
            # src_token, so no permuted copy of the activations is written
            L.moe_permute(b["idx"], self.E, workspace=b["ws"],
                          out=dict(offsets=b["offsets"], dst_row=b["dst_row"], src_token=b["src_token"]))
            mark("permute")

        # The shared expert needs only x's codes: it is forked first, and the
        # routing, permutation and routed GEMM1 fill the CUs its last partial
        # wave of workgroups leaves idle.
        quant()
        fork()
        route()
        permute()
        self._ffn(b["xq"], b["xs"], b["offsets"], w["w13q"], w["w13s"], w["w2q"], w["w2s"],
                  b["hq"], b["hs"], b["c2"], b.get("c1"), mark, a_row=b["src_token"])
        if self.shared_I and self.side is None:
            self._ffn(b["xq"], b["xs"], b["one_group"], w["sw13q"], w["sw13s"], w["sw2q"], w["sw2s"],
                      b["shq"], b["shs"], b["sc2"], b.get("sc1"), lambda n: mark("shared_" + n))
            shared = b["sc2"]
        elif self.side is not None:
            torch.cuda.current_stream().wait_stream(self.side)
            mark("shared_join")
        L.moe_combine(b["c2"], b["dst_row"], b["gate"], shared, out=b["y"])
        mark("combine")
        return b["y"]
