"""The routed-expert FP8 MoE FFN layer as sequences of library calls (no
host synchronisation inside): weight quantisation, the forward
(``MoEForward``), the input-side backward (``MoEBackward``) and the FP8
weight gradients (``MoEWeightGrad``).

Forward dataflow ([DSV3-MOE] shared + routed experts, sigmoid top-K with
bias, no dropping; [PANGU-MOGE] grouped softmax routing; [DSV3-FP8] /
[KANANA-FP8] fine-grained FP8):

  quant_act_1x128_e4m3(x) -> moe_route -> moe_permute (index maps) ->
  grouped_gemm_fp8_swiglu (expert-grouped rows gathered from x's FP8 codes
  through src_token; gate|up GEMM, SwiGLU and 1x128 quantisation fused) ->
  grouped_gemm_fp8_blockscaled (down projection, float32) -> moe_combine
  (gate-weighted sum + shared expert, bf16).

The shared expert (the same two GEMMs, one group over the unpermuted
tokens) runs on a side stream from the quantisation on and joins before the
combine.

Weights are quantised ahead of the forward (``quantize_weights``), as in
training where quantisation runs once per optimizer step for all experts;
the same launches can write the block-transposed copies the backward uses.
"""

import torch

from . import _lib as L


def quantize_weights(w13, w2, sw13=None, sw2=None, transposed=False):
    """All experts' 128x128-block FP8 weights in one launch per matrix.  With
    transposed=True the same launches also write the block-transposed copies
    the backward uses ([KANANA-FP8]) -> (weights, transposed weights), the
    latter in the layout of transpose_weights."""
    q, t = {}, {}
    mats = [("w13", w13), ("w2", w2)] + ([("sw13", sw13), ("sw2", sw2)] if sw13 is not None else [])
    for k, m in mats:
        r = L.quant_weight_128x128_e4m3_t(m) if transposed else L.quant_weight_128x128_e4m3(m)
        q[k + "q"], q[k + "s"] = r[0], r[1]
        if transposed:
            t[k + "tq"], t[k + "ts"] = r[2], r[3]
    return (q, t) if transposed else q


class MoEForward:
    """Preallocated buffers for one layer shape; ``__call__`` enqueues the
    whole forward on the current stream and returns y (bf16 [T, H])."""

    def __init__(self, T, H, E, I, route, weights, device, fused=True, shared_I=None, overlap_shared=True,
                 router_weight=None, fuse_route_permute=False, fuse_combine=False):
        self.T, self.H, self.E, self.I = T, H, E, I
        self.route = dict(route)
        self.K = route["K"] if route["mode"] == "sigmoid_bias" else route["n_groups"] * route["k_per_group"]
        self.w = weights
        self.fused = fused
        self.shared_I = shared_I
        # Routing + the permutation's index maps in one launch
        # (moe_route_permute) and the combine inside the down projection's
        # epilogue (grouped_gemm_fp8_combine): bit-identical to the separate
        # launches, and off by default because both measure slower on
        # MI355X.  Workgroups that hand data to workgroups on other XCDs need
        # a device-scope release (a write-back of the XCD's L2) per
        # workgroup or tile, which costs more than the kernel boundaries it
        # removes, and the combine's row gathers stall the GEMM tile
        # pipeline, while the separate combine streams at about 5 TB/s.
        self.fuse_route_permute = fuse_route_permute
        self.fuse_combine = fuse_combine
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
            # both keep counters between calls and must start zero-filled
            rp_ws=torch.zeros((L.moe_route_permute_workspace_size(T, K, E),), dtype=torch.uint8, device=dev),
            combine_ctr=torch.zeros((max(L.grouped_gemm_fp8_combine_workspace_size(T, H) // 4, 1),),
                                    dtype=torch.int32, device=dev),
            one_group=torch.tensor([0, T], dtype=torch.int32, device=dev),
        )
        if not fused:
            self.buf["c1"] = e((M, 2 * I), torch.float32)
        # optional router projection (float32 [E, H]): logits = x . W_r^T
        self.wr = router_weight
        if router_weight is not None:
            self.buf["logits"] = e((T, E), torch.float32)
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

    def _gemm1(self, aq, as_, offsets, w13q, w13s, hq, hs, c1, a_row=None):
        if self.fused:
            L.grouped_gemm_fp8_swiglu(aq, as_, w13q, w13s, offsets, hq=hq, hs=hs, a_row=a_row)
        else:
            if a_row is None:
                L.grouped_gemm_fp8_blockscaled(aq, as_, w13q, w13s, offsets, c=c1)
            else:
                L.grouped_gemm_fp8_blockscaled_gather(aq, as_, a_row, w13q, w13s, offsets, c=c1)
            L.swiglu(c1, hq=hq, hs=hs)

    def _ffn(self, aq, as_, offsets, w13q, w13s, w2q, w2s, hq, hs, c2, c1, mark, a_row=None):
        self._gemm1(aq, as_, offsets, w13q, w13s, hq, hs, c1, a_row=a_row)
        mark("gemm1")
        L.grouped_gemm_fp8_blockscaled(hq, hs, w2q, w2s, offsets, c=c2)
        mark("gemm2")

    def __call__(self, x, logits=None, bias=None, on_stage=None):
        """Enqueue the forward.  logits: the router logits [T, E], or None to
        compute them from x with the router weight given at construction.
        on_stage(name), if given, is called after each stage is enqueued on
        the caller's stream (the bench records a HIP event there).  With the
        shared expert on the side stream its GEMMs are not marked;
        "shared_join" marks the caller's stream waiting for them."""
        mark = on_stage or (lambda name: None)
        b, w, r = self.buf, self.w, self.route
        shared = None
        if logits is None:
            if self.wr is None:
                raise ValueError("no logits given and no router weight")
            logits = L.moe_router_logits(x, self.wr, logits=b["logits"])
            mark("router")

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

        def route_permute():
            mode = r["mode"]
            L.moe_route_permute(logits, bias if mode == "sigmoid_bias" else None, self.K, mode,
                                n_groups=r.get("n_groups", 1), k_per_group=r.get("k_per_group"),
                                normalize=r.get("normalize", True), workspace=b["rp_ws"],
                                out=dict(topk_idx=b["idx"], topk_gate=b["gate"], offsets=b["offsets"],
                                         dst_row=b["dst_row"], src_token=b["src_token"]))
            mark("route_permute")

        def join_shared():
            nonlocal shared
            if self.shared_I and self.side is None:
                self._ffn(b["xq"], b["xs"], b["one_group"], w["sw13q"], w["sw13s"], w["sw2q"], w["sw2s"],
                          b["shq"], b["shs"], b["sc2"], b.get("sc1"), lambda n: mark("shared_" + n))
                shared = b["sc2"]
            elif self.side is not None:
                torch.cuda.current_stream().wait_stream(self.side)
                mark("shared_join")

        # The shared expert needs only x's codes: it is forked first, and the
        # routing, permutation and routed GEMM1 fill the CUs its last partial
        # wave of workgroups leaves idle.
        quant()
        fork()
        if self.fuse_route_permute:
            route_permute()
        else:
            route()
            permute()
        self._gemm1(b["xq"], b["xs"], b["offsets"], w["w13q"], w["w13s"], b["hq"], b["hs"], b.get("c1"),
                    a_row=b["src_token"])
        mark("gemm1")
        if self.fuse_combine:
            # the epilogue reads the shared expert's output: join first
            join_shared()
            L.grouped_gemm_fp8_combine(b["hq"], b["hs"], w["w2q"], w["w2s"], b["offsets"], b["src_token"],
                                       b["dst_row"], b["gate"], shared, c=b["c2"], y=b["y"],
                                       counters=b["combine_ctr"])
            mark("gemm2_combine")
            return b["y"]
        L.grouped_gemm_fp8_blockscaled(b["hq"], b["hs"], w["w2q"], w["w2s"], b["offsets"], c=b["c2"])
        mark("gemm2")
        join_shared()
        L.moe_combine(b["c2"], b["dst_row"], b["gate"], shared, out=b["y"])
        mark("combine")
        return b["y"]

    def update_bias(self, bias, gamma):
        """Aux-loss-free balancing after a step: bias[e] -= gamma * sign(load_e
        - mean load), with the loads of the last forward's routing (in place,
        on the current stream)."""
        return L.moe_bias_update(self.buf["offsets"], gamma, bias)


def transpose_weights(w):
    """Block-transposed FP8 weights for the input-side backward ([KANANA-FP8]:
    the backward uses the transposed forward weights, not a second
    quantisation).  Like the weight quantisation, once per optimizer step."""
    t = {}
    t["w13tq"], t["w13ts"] = L.fp8_block_transpose(w["w13q"], w["w13s"])   # [E, H, 2I]
    t["w2tq"], t["w2ts"] = L.fp8_block_transpose(w["w2q"], w["w2s"])       # [E, I, H]
    if "sw13q" in w:
        t["sw13tq"], t["sw13ts"] = L.fp8_block_transpose(w["sw13q"], w["sw13s"])
        t["sw2tq"], t["sw2ts"] = L.fp8_block_transpose(w["sw2q"], w["sw2s"])
    return t


class MoEBackward:
    """Input-side backward of a MoEForward (dx and the router-logit gradient),
    enqueued on the current stream (the shared expert's chain on the
    forward's side stream):

      moe_combine_backward (dC2 quantised, d_gate) -> down dgrad GEMM on W2^T
      -> swiglu_backward on the forward's gate|up output -> gate|up dgrad GEMM
      on W13^T -> un-permute sum (moe_combine with unit gates, plus the shared
      expert's dx) -> moe_route_backward.

    The forward must keep its float32 gate|up output (MoEForward(fused=False)).
    With ``weight_grad=True`` the backward also keeps what the weight
    gradients need (each grouped row's gate and the unquantised [dg | du]);
    ``MoEWeightGrad`` consumes them.
    """

    def __init__(self, fwd, wt, weight_grad=False):
        if fwd.fused:
            raise ValueError("the backward needs the gate|up output: build the forward with fused=False")
        self.f, self.wt = fwd, wt
        T, H, E, I, K = fwd.T, fwd.H, fwd.E, fwd.I, fwd.K
        M = T * K
        dev = fwd.buf["xq"].device
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        self.buf = dict(dc2q=e((M, H), torch.uint8), dc2s=e((M, H // 128), torch.float32),
                        d_gate=e((T, K), torch.float32), dh=e((M, I), torch.float32),
                        dq1=e((M, 2 * I), torch.uint8), ds1=e((M, 2 * I // 128), torch.float32),
                        dxp=e((M, H), torch.float32), ones=torch.ones((T, K), dtype=torch.float32, device=dev),
                        dx=e((T, H), torch.bfloat16), d_logits=e((T, E), torch.float32))
        self.weight_grad = weight_grad
        if weight_grad:
            self.buf.update(gate_row=e((M,), torch.float32), d1=e((M, 2 * I), torch.float32))
            if fwd.shared_I:
                self.buf["d1s"] = e((T, 2 * fwd.shared_I), torch.float32)
        if fwd.shared_I:
            Is = fwd.shared_I
            self.buf.update(dyq=e((T, H), torch.uint8), dys=e((T, H // 128), torch.float32),
                            dhs=e((T, Is), torch.float32), dq1s=e((T, 2 * Is), torch.uint8),
                            ds1s=e((T, 2 * Is // 128), torch.float32), dxs=e((T, H), torch.float32))

    def __call__(self, dy, logits, on_stage=None):
        """dy bf16 [T, H], logits f32 [T, E] (the forward's) -> (dx bf16 [T, H],
        d_logits f32 [T, E])."""
        mark = on_stage or (lambda name: None)
        f, fb, b, wt = self.f, self.f.buf, self.buf, self.wt
        shared = None
        if f.shared_I:
            def shared_chain():
                L.quant_act_1x128_e4m3(dy, q=b["dyq"], scale=b["dys"])
                L.grouped_gemm_fp8_blockscaled(b["dyq"], b["dys"], wt["sw2tq"], wt["sw2ts"], fb["one_group"],
                                               c=b["dhs"])
                L.swiglu_backward(fb["sc1"], b["dhs"], dq=b["dq1s"], ds=b["ds1s"], d=b.get("d1s"))
                L.grouped_gemm_fp8_blockscaled(b["dq1s"], b["ds1s"], wt["sw13tq"], wt["sw13ts"], fb["one_group"],
                                               c=b["dxs"])
            if f.side is not None:
                f.side.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(f.side):
                    shared_chain()
            else:
                shared_chain()
            shared = b["dxs"]
        L.moe_combine_backward(dy, fb["c2"], fb["dst_row"], fb["gate"], dq=b["dc2q"], ds=b["dc2s"],
                               d_gate=b["d_gate"], gate_row=b.get("gate_row"))
        mark("combine_backward")
        L.grouped_gemm_fp8_blockscaled(b["dc2q"], b["dc2s"], wt["w2tq"], wt["w2ts"], fb["offsets"], c=b["dh"])
        mark("down_dgrad")
        L.swiglu_backward(fb["c1"], b["dh"], dq=b["dq1"], ds=b["ds1"], d=b.get("d1"))
        mark("swiglu_backward")
        L.grouped_gemm_fp8_blockscaled(b["dq1"], b["ds1"], wt["w13tq"], wt["w13ts"], fb["offsets"], c=b["dxp"])
        mark("gate_up_dgrad")
        if f.shared_I and f.side is not None:
            torch.cuda.current_stream().wait_stream(f.side)
            mark("shared_join")
        L.moe_combine(b["dxp"], fb["dst_row"], b["ones"], shared, out=b["dx"])
        mark("unpermute_sum")
        r = f.route
        L.moe_route_backward(logits, fb["idx"], b["d_gate"], mode=r["mode"], normalize=r.get("normalize", True),
                             d_logits=b["d_logits"])
        mark("route_backward")
        return b["dx"], b["d_logits"]


class MoEWeightGrad:
    """FP8 weight gradients of the expert projections after a MoEBackward
    built with ``weight_grad=True`` ([DSV3-FP8]: backward GEMMs in FP8).

    For each projection out = in . W^T the two operands are re-quantised in
    128x1 tiles along the token dimension, per expert (zero-padded to whole
    tiles), stored transposed, and multiplied per expert:
      down:    dOut = gate * dy (grouped rows; dy gathered through src_token,
               times each row's gate), In = h = silu(g) * u of the forward's
               gate|up output                      -> dw2  [E, H, I]
      gate|up: dOut = [dg | du] of the SwiGLU backward, In = x (gathered)
                                                   -> dw13 [E, 2I, H]
    and the same for the shared expert (one group over all tokens; dOut of
    its down projection is dy itself).  ``__call__(x, dy)`` enqueues
    everything on the current stream and returns the gradient dict;
    ``accumulate=True`` adds into the previous call's gradients.
    """

    def __init__(self, bwd, out_dtype=torch.float32):
        if not bwd.weight_grad:
            raise ValueError("build the MoEBackward with weight_grad=True")
        f = bwd.f
        self.b, self.f = bwd, f
        T, H, E, I, K = f.T, f.H, f.E, f.I, f.K
        M = T * K
        dev = f.buf["xq"].device
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)
        ld = L.moe_wgrad_padded_rows(M, E)
        self.ld = ld
        self.buf = dict(poff=e((E + 1,), torch.int32),
                        dc2t=e((H, ld), torch.uint8), dc2ts=e((ld // 128, H), torch.float32),
                        ht=e((I, ld), torch.uint8), hts=e((ld // 128, I), torch.float32),
                        d1t=e((2 * I, ld), torch.uint8), d1ts=e((ld // 128, 2 * I), torch.float32),
                        xt=e((H, ld), torch.uint8), xts=e((ld // 128, H), torch.float32),
                        dw2=e((E, H, I), out_dtype), dw13=e((E, 2 * I, H), out_dtype))
        if f.shared_I:
            Is = f.shared_I
            lds = L.moe_wgrad_padded_rows(T, 1)
            self.lds = lds
            self.buf.update(spoff=e((2,), torch.int32),
                            sdyt=e((H, lds), torch.uint8), sdyts=e((lds // 128, H), torch.float32),
                            sht=e((Is, lds), torch.uint8), shts=e((lds // 128, Is), torch.float32),
                            sd1t=e((2 * Is, lds), torch.uint8), sd1ts=e((lds // 128, 2 * Is), torch.float32),
                            sxt=e((H, lds), torch.uint8), sxts=e((lds // 128, H), torch.float32),
                            sdw2=e((1, H, Is), out_dtype), sdw13=e((1, 2 * Is, H), out_dtype))

    def __call__(self, x, dy, accumulate=False, on_stage=None):
        mark = on_stage or (lambda name: None)
        f, fb, bb, b = self.f, self.f.buf, self.b.buf, self.buf
        off, src, ld = fb["offsets"], fb["src_token"], self.ld
        M = src.shape[0]
        L.quant_act_128x1_grouped_e4m3(dy, off, M=M, row_index=src, row_scale=bb["gate_row"], ld=ld,
                                       qt=b["dc2t"], st=b["dc2ts"], padded_offsets=b["poff"])
        L.quant_act_128x1_grouped_e4m3(fb["c1"], off, swiglu_input=True, ld=ld, qt=b["ht"], st=b["hts"],
                                       padded_offsets=b["poff"])
        mark("quant_down_operands")
        L.grouped_wgrad_fp8(b["dc2t"], b["dc2ts"], b["ht"], b["hts"], b["poff"], c=b["dw2"], accumulate=accumulate)
        mark("down_wgrad")
        L.quant_act_128x1_grouped_e4m3(bb["d1"], off, ld=ld, qt=b["d1t"], st=b["d1ts"], padded_offsets=b["poff"])
        L.quant_act_128x1_grouped_e4m3(x, off, M=M, row_index=src, ld=ld, qt=b["xt"], st=b["xts"],
                                       padded_offsets=b["poff"])
        mark("quant_gate_up_operands")
        L.grouped_wgrad_fp8(b["d1t"], b["d1ts"], b["xt"], b["xts"], b["poff"], c=b["dw13"],
                            accumulate=accumulate)
        mark("gate_up_wgrad")
        out = dict(dw2=b["dw2"], dw13=b["dw13"])
        if f.shared_I:
            one, lds = fb["one_group"], self.lds
            L.quant_act_128x1_grouped_e4m3(dy, one, ld=lds, qt=b["sdyt"], st=b["sdyts"], padded_offsets=b["spoff"])
            L.quant_act_128x1_grouped_e4m3(fb["sc1"], one, swiglu_input=True, ld=lds, qt=b["sht"], st=b["shts"],
                                           padded_offsets=b["spoff"])
            L.grouped_wgrad_fp8(b["sdyt"], b["sdyts"], b["sht"], b["shts"], b["spoff"], c=b["sdw2"],
                                accumulate=accumulate)
            L.quant_act_128x1_grouped_e4m3(bb["d1s"], one, ld=lds, qt=b["sd1t"], st=b["sd1ts"],
                                           padded_offsets=b["spoff"])
            L.quant_act_128x1_grouped_e4m3(x, one, ld=lds, qt=b["sxt"], st=b["sxts"], padded_offsets=b["spoff"])
            L.grouped_wgrad_fp8(b["sd1t"], b["sd1ts"], b["sxt"], b["sxts"], b["spoff"], c=b["sdw13"],
                                accumulate=accumulate)
            mark("shared_wgrad")
            out.update(shared_dw2=b["sdw2"], shared_dw13=b["sdw13"])
        return out
