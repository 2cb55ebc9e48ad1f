#!/usr/bin/env python3
"""Benchmark of the routed-expert FP8 MoE layer forward on one MI355X.

One step = one forward of the whole layer over one batch (routing, 1x128
activation quantisation, permutation, fused gate|up GEMM + SwiGLU + FP8
quantisation, down GEMM, shared expert, combine) on the DeepSeek-V3-shaped
workload: T=4096 tokens, hidden 7168, 256 routed experts (top-8 sigmoid with
bias) + 1 shared expert, SwiGLU inter 2048.  Weights are block-quantised to
FP8 before the timed region (as in training, once per optimizer step); that
pass, the backward-side block transpose, the dgrad GEMM, the input-side
layer backward (with its stages) and the other routing workloads are timed
separately and reported under "extra".  Inputs are seeded synthetic tensors
resident in HBM before timing starts.

Prints ONE JSON line (see the keys below).  Per-kernel times come from HIP
events recorded on the stream the library launches on, inside the timed
region.  The CPU baseline times the oracle (test infrastructure) on a
bounded sample of the same workload and scales it to the full layer.

Besides the contract keys the line carries the per-step median and minimum
(from per-step events), a cold-cache run (a 1 GiB buffer written before
each step, outside the step's events, so inputs are not served from the
L2s or the Infinity Cache) and the GPU clocks as the SMI tool reports them.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
                      [--section layer|backward|train]
"""

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA, TFLOP/s
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense FP32 matrix, TFLOP/s
METRIC = "MoE-layer fwd tokens/s + FP8 grouped-GEMM TFLOP/s (% MFMA peak), 1 GPU"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="dsv3")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true")
    p.add_argument("--section", choices=["layer", "backward", "train", "wgrad"], default="layer",
                   help="layer: the forward bench line (default); backward: time only the input-side "
                        "backward + weight gradients of the same workload, K steps after W warm-ups "
                        "(for per-kernel profiles); train: a whole training step of the layer (weight "
                        "quantisation and transpose, forward, backward, weight gradients, bias update); "
                        "wgrad: only the routed weight-gradient GEMMs (down and gate|up, float32 and "
                        "bf16 output) on operands prepared once, for per-kernel profiles and counters; "
                        "the last three print their own JSON line")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def gpu_clocks():
    """Current GPU clocks read from the driver's sysfs tables (no child
    process: under a profiler that preloads itself, a spawned tool would be
    an exec from a process that has set up the GPU).  {domain: MHz} of the
    level marked current in pp_dpm_sclk / pp_dpm_mclk / pp_dpm_fclk of the
    first card that has them, or None."""
    import glob
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        out = {}
        for dom in ("sclk", "mclk", "fclk", "socclk"):
            try:
                lines = open(os.path.join(dev, f"pp_dpm_{dom}")).read().splitlines()
            except OSError:
                continue
            for ln in lines:
                if ln.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*[Mm][Hh]z", ln)
                    if m:
                        out[dom] = int(m.group(1))
        if out:
            return out
    return None


def cold_steps(step, n, torch):
    """Median and minimum of n single steps, each after writing a 1 GiB
    buffer (outside the step's events): the inputs then come from HBM, not
    from the L2s or the 256 MB Infinity Cache."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    times = []
    for i in range(n):
        flush.fill_(float(i))
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del flush
    return dict(steps=n, median_ms=statistics.median(times), min_ms=min(times), flush_bytes=1 << 30)


def copy_rate(torch, nbytes=1 << 30, reps=10):
    """A plain device copy (torch's copy kernel) of nbytes: read + write
    bytes per second, the device's measured streaming ceiling beside 8 TB/s."""
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ms = time_op(lambda: b.copy_(a), reps, torch)
    del a, b
    return dict(copy_bytes=nbytes, ms=ms, GBps=2 * nbytes / ms / 1e6)


def dense_fp8_gemm_rate(torch, n=8192, reps=20):
    """A plain dense FP8 GEMM from the vendor library (torch._scaled_mm, one
    scale per tensor) at n x n x n: the device's measured matrix-core rate
    for FP8 beside the 5.0 PFLOP/s datasheet figure.  Context only; the
    layer's GEMMs are the library's own kernels (block scales need the
    per-chunk promotion)."""
    try:
        a = torch.randn(n, n, device="cuda").to(torch.float8_e4m3fn)
        b = torch.randn(n, n, device="cuda").to(torch.float8_e4m3fn)
        one = torch.tensor(1.0, device="cuda")
        ms = time_op(lambda: torch._scaled_mm(a, b.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16),
                     reps, torch)
    except (RuntimeError, AttributeError, TypeError) as ex:
        return dict(error=repr(ex)[:200])
    return dict(m=n, n=n, k=n, ms=ms, TFLOPs=2 * n ** 3 / ms / 1e9,
                frac_mfma=2 * n ** 3 / ms / 1e9 / FP8_PEAK_TFLOPS)


def mfma_probe_rate(torch, R, iters=20000, reps=5):
    """The library's matrix-core probe: 8 independent chains of FP8 matrix
    instructions per wave on register operands, no memory traffic, at the
    grouped GEMM's occupancy (one 8-wave workgroup per compute unit, 2 waves
    per SIMD) and at 8 waves per SIMD: the device's own FP8 ceiling beside
    the 5.0 PFLOP/s datasheet figure."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {}
    for tag, per_cu in (("2_waves_per_simd", 1), ("8_waves_per_simd", 4)):
        blocks = cus * per_cu
        buf = torch.empty(blocks * 64 * 8, dtype=torch.float32, device="cuda")
        fl = R.moe_probe_mfma_fp8(iters, blocks, 8, out=buf)[1]
        ms = time_op(lambda: R.moe_probe_mfma_fp8(iters, blocks, 8, out=buf), reps, torch)
        out[tag] = dict(blocks=blocks, waves_per_block=8, ms=ms, TFLOPs=fl / ms / 1e9,
                        frac_mfma=fl / ms / 1e9 / FP8_PEAK_TFLOPS)
    return out


def wgrad_bytes(E, H, I, wg):
    """Algorithmic bytes of the down and gate|up weight-gradient launches:
    float32 gradients written once, the two 128x1 operands read once over
    the padded rows the experts own (P_E, from the last call), and their
    tile scales."""
    pg = int(wg.buf["poff"][-1].item())
    b2 = 4 * E * H * I + (H + I) * pg + 4 * (H + I) * (pg // 128)
    b13 = 4 * E * 2 * I * H + (2 * I + H) * pg + 4 * (2 * I + H) * (pg // 128)
    return b2, b13


def gemm1_bytes(T, K, H, E, I):
    """Algorithmic HBM bytes of the fused gate|up launch: activation codes and
    scales, every expert's gate|up codes and block scales, h codes and scales."""
    M = T * K
    return (M * H + M * (H // 128) * 4 + E * 2 * I * H + E * (2 * I // 128) * (H // 128) * 4
            + M * I + M * (I // 128) * 4)


def gemm_flops(M, N, K):
    return 2.0 * M * N * K


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(name, kernel_src, workload):
    """HBM traffic measured by rocprofv3 counters for this kernel, if the
    committed measurement was taken on the current kernel source and on the
    workload being timed."""
    f = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(f):
        return None
    rec = json.load(open(f))
    if rec.get("kernel_source_sha256_16") != source_hash(kernel_src) or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def time_op(fn, reps, torch):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    fn()
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(reps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    return sum(evs[i].elapsed_time(evs[i + 1]) for i in range(reps)) / reps


def extra_rows(cfg, d, fwd, torch, R, synth, reps=5):
    """Weight quantisation of all experts, and the backward-side block
    transpose + dY quantisation + dgrad GEMM on the dsv3 expert shapes."""
    out = {}
    T, H, E, I = cfg["T"], cfg["H"], cfg["E"], cfg["I"]
    w13, w2 = d["w13"], d["w2"]
    q13 = torch.empty(w13.shape, dtype=torch.uint8, device=w13.device)
    s13 = torch.empty((E, 2 * I // 128, H // 128), dtype=torch.float32, device=w13.device)
    ms = time_op(lambda: R.quant_weight_128x128_e4m3(w13, q=q13, scale=s13), reps, torch)
    nbytes = w13.numel() * 3 + s13.numel() * 4
    out["quant_weight_128x128_w13_all_experts"] = dict(
        ms=ms, GBps=nbytes / ms / 1e6, frac_hbm=nbytes / ms / 1e6 / HBM_PEAK_GBS, bytes=nbytes)
    del q13, s13
    # backward side: gate projection of every expert, stored [2048, 7168]
    bcfg = dict(synth.get_config("bwd"), I=I // 2)       # [E, 2 * (I/2), H] = [E, 2048, 7168]
    wg = synth.expert_weights(bcfg, "w13", w13.device, seed=1)
    wq, ws = R.quant_weight_128x128_e4m3(wg)
    del wg
    qt = torch.empty((E, H, I), dtype=torch.uint8, device=wq.device)
    st = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device=wq.device)
    ms = time_op(lambda: R.fp8_block_transpose(wq, ws, qt=qt, scale_t=st), reps, torch)
    nbytes = 2 * (wq.numel() + ws.numel() * 4)
    out["fp8_block_transpose_e256_2048x7168"] = dict(
        ms=ms, GBps=nbytes / ms / 1e6, frac_hbm=nbytes / ms / 1e6 / HBM_PEAK_GBS, bytes=nbytes)
    M = T * cfg["K"]
    dy = synth.output_grad(M, I, wq.device, seed=0)
    dyq = torch.empty((M, I), dtype=torch.uint8, device=wq.device)
    dys = torch.empty((M, I // 128), dtype=torch.float32, device=wq.device)
    ms_q = time_op(lambda: R.quant_act_1x128_e4m3(dy, q=dyq, scale=dys), reps, torch)
    nbytes = dy.numel() * 3 + dys.numel() * 4
    out["quant_act_1x128_dY"] = dict(ms=ms_q, GBps=nbytes / ms_q / 1e6,
                                     frac_hbm=nbytes / ms_q / 1e6 / HBM_PEAK_GBS, bytes=nbytes)
    # the layer's down projection with bf16 output (same main loop; its bytes
    # drop by the halved output)
    bb = fwd.buf
    c2_bf16 = torch.empty((M, H), dtype=torch.bfloat16, device=wq.device)
    ms = time_op(lambda: R.grouped_gemm_fp8_blockscaled(bb["hq"], bb["hs"], fwd.w["w2q"], fwd.w["w2s"],
                                                          bb["offsets"], c=c2_bf16), reps, torch)
    fl = gemm_flops(M, H, I)
    nbytes = M * I + M * (I // 128) * 4 + fwd.w["w2q"].numel() + fwd.w["w2s"].numel() * 4 + M * H * 2
    out["gemm2_down_bf16_out"] = dict(ms=ms, TFLOPs=fl / ms / 1e9, frac_mfma=fl / ms / 1e9 / FP8_PEAK_TFLOPS,
                                      GBps=nbytes / ms / 1e6, frac_hbm=nbytes / ms / 1e6 / HBM_PEAK_GBS,
                                      bytes=nbytes, flops=fl)
    del c2_bf16
    dx = torch.empty((M, H), dtype=torch.float32, device=wq.device)
    offsets = fwd.buf["offsets"]
    ms = time_op(lambda: R.grouped_gemm_fp8_blockscaled(dyq, dys, qt, st, offsets, c=dx), reps, torch)
    fl = gemm_flops(M, H, I)
    nbytes = M * I + M * (I // 128) * 4 + qt.numel() + st.numel() * 4 + M * H * 4
    out["dgrad_grouped_gemm_m32768_n7168_k2048"] = dict(
        ms=ms, TFLOPs=fl / ms / 1e9, frac_mfma=fl / ms / 1e9 / FP8_PEAK_TFLOPS, GBps=nbytes / ms / 1e6,
        frac_hbm=nbytes / ms / 1e6 / HBM_PEAK_GBS, bytes=nbytes, flops=fl)
    return out


def staged(fn, reps, torch):
    """Mean time of fn(on_stage) and of each stage between its marks, from
    HIP events recorded on the launching stream."""
    marks = []

    def on_stage(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        marks[-1].append((name, e))

    fn(None)
    torch.cuda.synchronize()
    for _ in range(reps):
        s = torch.cuda.Event(enable_timing=True)
        s.record()
        marks.append([("start", s)])
        fn(on_stage)
    torch.cuda.synchronize()
    stages = {}
    for step in marks:
        for (_, a), (name, b) in zip(step[:-1], step[1:]):
            stages[name] = stages.get(name, 0.0) + a.elapsed_time(b) / reps
    total = sum(step[0][1].elapsed_time(step[-1][1]) for step in marks) / reps
    return total, stages


def router_rows(cfg, d, fwd, torch, R, synth, reps=5):
    """Router projection (float32 matrix cores) and one balancing bias update
    on the same workload."""
    T, H, E = cfg["T"], cfg["H"], cfg["E"]
    wr = synth.router_weight(cfg, d["x"].device, seed=0)
    lg = torch.empty((T, E), dtype=torch.float32, device=d["x"].device)
    ms = time_op(lambda: R.moe_router_logits(d["x"], wr, logits=lg), reps, torch)
    fl = gemm_flops(T, E, H)
    bias = torch.zeros(E, dtype=torch.float32, device=d["x"].device)
    ms_b = time_op(lambda: R.moe_bias_update(fwd.buf["offsets"], 1e-3, bias), reps, torch)
    return dict(router_logits=dict(ms=ms, TFLOPs=fl / ms / 1e9, frac_fp32_mfma=fl / ms / 1e9 / FP32_MFMA_PEAK_TFLOPS,
                                   flops=fl),
                bias_update_us=ms_b * 1e3)


def fusion_rows(cfg, d, w, torch, R, reps=20):
    """The layer forward with the single-launch routing + permutation
    (moe_route_permute) and the combine fused into the down projection
    (grouped_gemm_fp8_combine), each on and off, on the timed workload: the
    layer time of every combination (y is bit-identical in all four) and the
    stage times of the two extremes."""
    T, H, E, I = cfg["T"], cfg["H"], cfg["E"], cfg["I"]
    dev = d["x"].device
    out = {}
    ref = None
    for frp in (False, True):
        for fc in (False, True):
            f = R.MoEForward(T, H, E, I, cfg["route"], w, dev, fused=True, shared_I=cfg.get("shared_I"),
                             fuse_route_permute=frp, fuse_combine=fc)
            y = f(d["x"], d["logits"], d["bias"])
            torch.cuda.synchronize()
            same = True if ref is None else bool(torch.equal(y.view(torch.int16), ref))
            if ref is None:
                ref = y.view(torch.int16).clone()
            ms = time_op(lambda: f(d["x"], d["logits"], d["bias"]), reps, torch)
            row = dict(layer_ms=ms, y_bit_identical=same)
            if frp == fc:
                _, st = staged(lambda m: f(d["x"], d["logits"], d["bias"], on_stage=m), 5, torch)
                row["stage_ms"] = st
            out[f"route_permute_{'fused' if frp else 'separate'}__combine_{'fused' if fc else 'separate'}"] = row
            del f
    return out


def graph_rows(torch, R, synth, reps=50):
    """The layer forward eager vs replayed from a captured HIP graph on the
    small layers, where kernel launches, not the kernels, set the step time:
    the tiny workload (T=256, H=512, 8 experts, top-2 softmax) and a small
    shared-expert layer (T=200, H=512, 16 experts top-4 + shared, whose
    capture holds the side stream's fork and join)."""
    tiny = synth.get_config("tiny")
    shared = dict(tiny, T=200, E=16, K=4, I=256, shared_I=256, bias_std=0.01,
                  route=dict(mode="sigmoid_bias", K=4, normalize=True), x_dtype="bf16", w_dtype="bf16")
    out = {}
    for key, cfg, label in (("tiny", tiny, tiny["name"]),
                            ("shared_layer", shared, "T=200, H=512, 16 experts top-4 + shared")):
        r = graph_row(cfg, torch, R, synth, reps)
        r["workload"] = label
        r["eager_tokens_per_s"] = cfg["T"] / (r["eager_ms"] / 1e3)
        r["graph_tokens_per_s"] = cfg["T"] / (r["graph_replay_ms"] / 1e3)
        out[key] = r
    return out


def graph_row(cfg, torch, R, synth, reps):
    dev = torch.device("cuda:0")
    d = synth.layer_inputs(cfg, dev, seed=0)
    w = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"))
    fwd = R.MoEForward(cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["route"], w, dev,
                       shared_I=cfg.get("shared_I"))
    eager = time_op(lambda: fwd(d["x"], d["logits"], d["bias"]), reps, torch)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd(d["x"], d["logits"], d["bias"])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(d["x"], d["logits"], d["bias"])
    graph = time_op(g.replay, reps, torch)
    return dict(eager_ms=eager, graph_replay_ms=graph)


def backward_rows(cfg, d, w, torch, R, synth, reps=5):
    """Input-side layer backward on the same workload: the forward that keeps
    its float32 gate|up output, the block transpose of every expert's
    weights (once per optimizer step), and the backward chain with its
    stages (combine backward, down dgrad, SwiGLU backward, gate|up dgrad,
    un-permute sum, router backward)."""
    T, H, E, I, K = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["K"]
    M = T * K
    dev = d["x"].device
    ms_t = time_op(lambda: R.transpose_weights(w), 2, torch)
    wt = R.transpose_weights(w)
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev, fused=False, shared_I=cfg.get("shared_I"))
    fwd_ms = time_op(lambda: fwd(d["x"], d["logits"], d["bias"]), reps, torch)
    dy = synth.output_grad(T, H, dev, seed=4)
    bwd = R.MoEBackward(fwd, wt)
    total, st = staged(lambda mark: bwd(dy, d["logits"], on_stage=mark), reps, torch)
    f_down = gemm_flops(M, I, H)
    f_gu = gemm_flops(M, H, 2 * I)
    out = dict(
        backward_ms=total, tokens_per_s=T / (total / 1e3), forward_keep_c1_ms=fwd_ms,
        stages_ms=st, transpose_weights_all_ms=ms_t,
        down_dgrad=dict(ms=st["down_dgrad"], TFLOPs=f_down / st["down_dgrad"] / 1e9,
                        frac_mfma=f_down / st["down_dgrad"] / 1e9 / FP8_PEAK_TFLOPS),
        gate_up_dgrad=dict(ms=st["gate_up_dgrad"], TFLOPs=f_gu / st["gate_up_dgrad"] / 1e9,
                           frac_mfma=f_gu / st["gate_up_dgrad"] / 1e9 / FP8_PEAK_TFLOPS))
    # weight gradients (128x1 operands + grouped wgrad GEMMs), float32 out
    bwd = R.MoEBackward(fwd, wt, weight_grad=True)
    bwd(dy, d["logits"])
    wg = R.MoEWeightGrad(bwd)
    total_w, st_w = staged(lambda mark: wg(d["x"], dy, on_stage=mark), reps, torch)
    ld = wg.ld
    b2, b13 = wgrad_bytes(E, H, I, wg)
    rows = {}
    for name, stage, nbytes, fl in (("down_wgrad", "down_wgrad", b2, gemm_flops(M, H, I)),
                                    ("gate_up_wgrad", "gate_up_wgrad", b13, gemm_flops(M, 2 * I, H))):
        ms = st_w[stage]
        rows[name] = dict(ms=ms, GBps=nbytes / ms / 1e6, frac_hbm=nbytes / ms / 1e6 / HBM_PEAK_GBS, bytes=nbytes,
                          TFLOPs=fl / ms / 1e9, frac_mfma=fl / ms / 1e9 / FP8_PEAK_TFLOPS)
    # the same gate|up weight gradient with bf16 output
    wb = wg.buf
    dwb = torch.empty((E, 2 * I, H), dtype=torch.bfloat16, device=dev)
    ms = time_op(lambda: R.grouped_wgrad_fp8(wb["d1t"], wb["d1ts"], wb["xt"], wb["xts"], wb["poff"], c=dwb),
                 reps, torch)
    nb = b13 - 2 * E * 2 * I * H
    rows["gate_up_wgrad_bf16_out"] = dict(ms=ms, GBps=nb / ms / 1e6, frac_hbm=nb / ms / 1e6 / HBM_PEAK_GBS,
                                          bytes=nb)
    out["weight_grad"] = dict(ms=total_w, stages_ms=st_w, padded_rows=ld, **rows)
    del bwd, wg, dwb, fwd, wt
    torch.cuda.empty_cache()
    return out


def other_workload_rows(torch, R, synth, names=("moge", "skewed"), reps=5):
    """GEMM1 (gate|up + SwiGLU, gathered rows) and GEMM2 throughput and the
    whole layer forward on the other routing workloads, whose GEMM1 sits
    above the MFMA ridge (compute-bound).  Same kernels and launch as the
    layer; context rows, not the headline."""
    out = {}
    dev = torch.device("cuda:0")
    for name in names:
        cfg = synth.get_config(name)
        T, H, E, I, K = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["K"]
        d = synth.layer_inputs(cfg, dev, seed=0)
        w = R.quantize_weights(d["w13"], d["w2"])
        del d["w13"], d["w2"]
        fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev, fused=True)
        layer_ms = time_op(lambda: fwd(d["x"], d["logits"], d["bias"]), reps, torch)
        b = fwd.buf
        g1 = time_op(lambda: R.grouped_gemm_fp8_swiglu(b["xq"], b["xs"], w["w13q"], w["w13s"], b["offsets"],
                                                         hq=b["hq"], hs=b["hs"], a_row=b["src_token"]), reps, torch)
        g2 = time_op(lambda: R.grouped_gemm_fp8_blockscaled(b["hq"], b["hs"], w["w2q"], w["w2s"], b["offsets"],
                                                              c=b["c2"]), reps, torch)
        M = T * K
        f1, f2 = gemm_flops(M, 2 * I, H), gemm_flops(M, H, I)
        out[cfg["name"]] = dict(
            layer_ms=layer_ms, tokens_per_s=T / (layer_ms / 1e3),
            gemm1_swiglu=dict(ms=g1, TFLOPs=f1 / g1 / 1e9, frac_mfma=f1 / g1 / 1e9 / FP8_PEAK_TFLOPS),
            gemm2=dict(ms=g2, TFLOPs=f2 / g2 / 1e9, frac_mfma=f2 / g2 / 1e9 / FP8_PEAK_TFLOPS))
        del fwd, w, d, b
        torch.cuda.empty_cache()
    return out


def cpu_baseline(cfg, d, n_experts=12, shared_tokens=1024, combine_tokens=2048):
    """The oracle as it stands, on a bounded sample of the workload, scaled to
    the full layer: routing, activation quantisation and permutation of all
    tokens; the routed-expert FFN (GEMM1, SwiGLU + quantisation, GEMM2) for
    `n_experts` experts with all their rows; the shared expert for
    `shared_tokens` tokens; the combine for `combine_tokens` tokens."""
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_info
    T, H, E, I, K = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["K"]
    shared_tokens, combine_tokens = min(shared_tokens, T), min(combine_tokens, T)
    x = d["x"].float().cpu().numpy()
    logits = d["logits"].cpu().numpy()
    bias = d["bias"].cpu().numpy() if d["bias"] is not None else None
    t = {}
    rc = cfg["route"]
    t0 = time.perf_counter()
    if rc["mode"] == "sigmoid_bias":
        idx, gate = O.route_sigmoid_bias(logits, bias, K, rc.get("normalize", True))
    else:
        idx, gate = O.route_softmax_grouped(logits, rc["n_groups"], rc["k_per_group"])
    t["route"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    xq, xs = O.quant_act_1x128(x)
    t["quant_act"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    perm = O.permute(idx, E, xq, xs)
    t["permute"] = time.perf_counter() - t0
    counts = np.diff(perm["offsets"])
    order = np.argsort(counts)
    experts = [int(e) for e in order[len(order) // 2: len(order) // 2 + n_experts]]   # median loads
    t_exp = 0.0
    rows_done = 0
    for e in experts:
        w13q, w13s = O.quant_weight_128x128(d["w13"][e:e + 1].float().cpu().numpy())   # untimed prep
        w2q, w2s = O.quant_weight_128x128(d["w2"][e:e + 1].float().cpu().numpy())
        r0, r1 = perm["offsets"][e], perm["offsets"][e + 1]
        off = np.array([0, r1 - r0], np.int32)
        t0 = time.perf_counter()
        c1, _ = O.grouped_gemm(perm["aq"][r0:r1], perm["as"][r0:r1], w13q, w13s, off, with_mag=False)
        hq, hs, _ = O.swiglu_quant(c1.astype(np.float32))
        O.grouped_gemm(hq, hs, w2q, w2s, off, with_mag=False)
        t_exp += time.perf_counter() - t0
        rows_done += int(r1 - r0)
    t_sh = 0.0
    if cfg.get("shared_I"):
        sw13q, sw13s = O.quant_weight_128x128(d["sw13"].float().cpu().numpy())
        sw2q, sw2s = O.quant_weight_128x128(d["sw2"].float().cpu().numpy())
        off = np.array([0, shared_tokens], np.int32)
        t0 = time.perf_counter()
        c1, _ = O.grouped_gemm(xq[:shared_tokens], xs[:shared_tokens], sw13q, sw13s, off, with_mag=False)
        hq, hs, _ = O.swiglu_quant(c1.astype(np.float32))
        O.grouped_gemm(hq, hs, sw2q, sw2s, off, with_mag=False)
        t_sh = time.perf_counter() - t0
    yperm = np.zeros((combine_tokens * K, H))
    dst = np.arange(combine_tokens * K).reshape(combine_tokens, K)
    t0 = time.perf_counter()
    O.combine_ref(yperm, dst, gate[:combine_tokens], np.zeros((combine_tokens, H)))
    t_comb = time.perf_counter() - t0
    total = (t["route"] + t["quant_act"] + t["permute"] + t_exp * (T * K) / max(rows_done, 1)
             + t_sh * T / shared_tokens + t_comb * T / combine_tokens)
    sampled = sum(t.values()) + t_exp + t_sh + t_comb
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return dict(value=T / total, unit="tokens/s", cores=threads, kind="oracle",
                sample=(f"oracle layer forward on the {cfg['name']} workload: routing, activation "
                        f"quantisation and permutation of all {T} tokens; routed-expert FFN for "
                        f"{len(experts)} median-load experts ({rows_done} of {T * K} rows, scaled by rows); "
                        + (f"shared expert for {shared_tokens} tokens and " if cfg.get("shared_I") else "")
                        + f"combine for {combine_tokens} "
                        f"tokens (scaled by tokens); {sampled:.1f} s of CPU work measured, "
                        f"{total:.1f} s estimated for the full layer"),
                seconds_full_layer_estimate=total)


def backward_section(args, cfg, d, w, torch, R, synth):
    """K timed steps of the input-side backward followed by the FP8 weight
    gradients (float32), with per-stage HIP events; one JSON line."""
    T, H, E, I, K = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["K"]
    dev = d["x"].device
    wt = R.transpose_weights(w)
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev, fused=False, shared_I=cfg.get("shared_I"))
    fwd(d["x"], d["logits"], d["bias"])
    dy = synth.output_grad(T, H, dev, seed=4)
    bwd = R.MoEBackward(fwd, wt, weight_grad=True)
    wg = R.MoEWeightGrad(bwd)

    def step(mark):
        bwd(dy, d["logits"], on_stage=mark)
        wg(d["x"], dy, on_stage=mark)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    total, st = staged(step, args.steps, torch)
    line = {"metric": "MoE-layer input-side backward + FP8 weight gradients, tokens/s, 1 GPU",
            "value": T / (total / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": total, "higher_is_better": True, "dtype": "fp8_e4m3",
            "data": "synthetic", "config": {"workload": cfg["name"]}, "stages_ms": st}
    print(json.dumps(line), flush=True)


def wgrad_section(args, cfg, d, w, torch, R, synth):
    """K timed steps of the routed weight-gradient GEMMs alone: dW2 and dW13
    with float32 and with bf16 output, on the 128x1-quantised operands of one
    backward pass (prepared once, untimed); one JSON line with each launch's
    time and algorithmic bytes."""
    T, H, E, I = cfg["T"], cfg["H"], cfg["E"], cfg["I"]
    dev = d["x"].device
    wt = R.transpose_weights(w)
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev, fused=False, shared_I=cfg.get("shared_I"))
    fwd(d["x"], d["logits"], d["bias"])
    dy = synth.output_grad(T, H, dev, seed=4)
    bwd = R.MoEBackward(fwd, wt, weight_grad=True)
    bwd(dy, d["logits"])
    wg = R.MoEWeightGrad(bwd)
    wg(d["x"], dy)
    del wt
    wb = wg.buf
    b2, b13 = wgrad_bytes(E, H, I, wg)
    launches = {}
    for name, (a, sa, b, sb), shape, nbytes in (
            ("down", (wb["dc2t"], wb["dc2ts"], wb["ht"], wb["hts"]), (E, H, I), b2),
            ("gate_up", (wb["d1t"], wb["d1ts"], wb["xt"], wb["xts"]), (E, 2 * I, H), b13)):
        for dt, tag in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
            c = torch.empty(shape, dtype=dt, device=dev)
            out_bytes = shape[0] * shape[1] * shape[2] * (4 if dt == torch.float32 else 2)
            launches[f"{name}_wgrad_{tag}"] = (lambda a=a, sa=sa, b=b, sb=sb, c=c: R.grouped_wgrad_fp8(
                a, sa, b, sb, wb["poff"], c=c), nbytes - 4 * shape[0] * shape[1] * shape[2] + out_bytes)
    for _ in range(args.warmup):
        for fn, _ in launches.values():
            fn()
    torch.cuda.synchronize()
    rows = {}
    for k, (fn, nbytes) in launches.items():
        ms = time_op(fn, args.steps, torch)
        rows[k] = dict(ms=ms, bytes=nbytes, GBps=nbytes / ms / 1e6, frac_hbm=nbytes / ms / 1e6 / HBM_PEAK_GBS)
    line = {"metric": "routed FP8 weight-gradient GEMMs, GB/s (algorithmic bytes), 1 GPU", "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "dtype": "fp8_e4m3", "data": "synthetic",
            "config": {"workload": cfg["name"], "padded_rows": wg.ld}, "launches": rows}
    print(json.dumps(line), flush=True)


def cpu_baseline_train(cfg, d, dy, n_experts=2):
    """The oracle's training step on a bounded sample, scaled to the layer:
    routing, activation quantisation and permutation of all tokens; for
    `n_experts` median-load experts, their weights quantised and transposed,
    the forward rows (GEMM1, SwiGLU, GEMM2), the combine gradient, both dgrad
    GEMMs, the SwiGLU backward and both FP8 weight gradients (scaled by
    experts); the bias update."""
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_info
    T, H, E, I, K = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["K"]
    x = d["x"].float().cpu().numpy()
    logits = d["logits"].cpu().numpy()
    bias = d["bias"].cpu().numpy()
    dyn = dy.float().cpu().numpy()
    t0 = time.perf_counter()
    idx, gate = O.route_sigmoid_bias(logits, bias, K, True)
    perm = O.permute(idx, E)
    t_all = time.perf_counter() - t0
    off, src, dst = perm["offsets"], perm["src_token"], perm["dst_row"]
    gate_row = np.zeros(T * K, np.float32)
    gate_row[dst.ravel()] = gate.ravel()
    order = np.argsort(np.diff(off))
    experts = [int(e) for e in order[len(order) // 2: len(order) // 2 + n_experts]]
    t_exp = 0.0
    for e in experts:
        w13 = d["w13"][e:e + 1].float().cpu().numpy()
        w2 = d["w2"][e:e + 1].float().cpu().numpy()
        rows = np.arange(off[e], off[e + 1])
        one = np.array([0, len(rows)], np.int32)
        t0 = time.perf_counter()
        q13, s13 = O.quant_weight_128x128(w13)
        q2, s2 = O.quant_weight_128x128(w2)
        q13t, s13t = O.block_transpose(q13, s13)
        q2t, s2t = O.block_transpose(q2, s2)
        aq, as_ = O.quant_act_1x128(x[src[rows]])
        c1, _ = O.grouped_gemm(aq, as_, q13, s13, one, with_mag=False)
        hq, hs, h = O.swiglu_quant(c1.astype(np.float32))
        O.grouped_gemm(hq, hs, q2, s2, one, with_mag=False)
        dc2 = (gate_row[rows][:, None] * dyn[src[rows]]).astype(np.float32)
        dc2q, dc2s = O.quant_act_1x128(dc2)
        dh, _ = O.grouped_gemm(dc2q, dc2s, q2t, s2t, one, with_mag=False)
        dq1, ds1, d1 = O.swiglu_backward(c1.astype(np.float32), dh.astype(np.float32))
        O.grouped_gemm(dq1, ds1, q13t, s13t, one, with_mag=False)
        a2, s_a2, p = O.quant_act_128x1_grouped(dc2, one)
        b2, s_b2, _ = O.quant_act_128x1_grouped(h, one)
        O.wgrad_gemm(a2, s_a2, b2, s_b2, p, with_mag=False)
        a1, s_a1, _ = O.quant_act_128x1_grouped(d1, one)
        b1, s_b1, _ = O.quant_act_128x1_grouped(x[src[rows]], one)
        O.wgrad_gemm(a1, s_a1, b1, s_b1, p, with_mag=False)
        t_exp += time.perf_counter() - t0
    t0 = time.perf_counter()
    O.bias_update(bias, off, np.float32(1e-3))
    t_all += time.perf_counter() - t0
    total = t_all + t_exp * E / n_experts
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return dict(value=T / total, unit="tokens/s", cores=threads, kind="oracle",
                sample=(f"oracle training step on the {cfg['name']} workload: routing, permutation and bias "
                        f"update of all {T} tokens; weights, forward rows, backward rows and weight gradients of "
                        f"{n_experts} median-load experts, scaled by experts (shared expert and combine not "
                        f"included); {t_all + t_exp:.1f} s measured, {total:.0f} s estimated for the step"))


def train_section(args, cfg, d, torch, R, synth):
    """K timed training steps of the layer: every expert's weights quantised
    from the bf16 masters and block-transposed (once per optimizer step, as
    the pages' all-experts quantisation kernel does), the forward keeping its
    float32 gate|up output, the input-side backward, the FP8 weight gradients
    (float32) and one balancing bias update.  One JSON line."""
    T, H, E, I, K = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["K"]
    dev = d["x"].device
    w = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"))
    wt = R.transpose_weights(w)
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev, fused=False, shared_I=cfg.get("shared_I"))
    fwd(d["x"], d["logits"], d["bias"])
    dy = synth.output_grad(T, H, dev, seed=4)
    bwd = R.MoEBackward(fwd, wt, weight_grad=True)
    wg = R.MoEWeightGrad(bwd)
    bias = d["bias"].clone()

    def step(mark):
        m = mark or (lambda name: None)
        # every expert's weights quantised, the backward's transposed copies
        # written by the same launches (into the same buffers every step)
        for k in ("w13", "w2", "sw13", "sw2"):
            if k in d:
                R.quant_weight_128x128_e4m3_t(d[k], q=w[k + "q"], scale=w[k + "s"], qt=wt[k + "tq"],
                                              scale_t=wt[k + "ts"])
        m("quantize_and_transpose_weights")
        fwd(d["x"], d["logits"], bias)
        m("forward")
        bwd(dy, d["logits"], on_stage=mark)     # its own stages
        wg(d["x"], dy, on_stage=mark)
        fwd.update_bias(bias, 1e-3)
        m("bias_update")

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    total, detail = staged(step, args.steps, torch)
    bwd_keys = ("combine_backward", "down_dgrad", "swiglu_backward", "gate_up_dgrad", "shared_join",
                "unpermute_sum", "route_backward")
    wg_keys = ("quant_down_operands", "down_wgrad", "quant_gate_up_operands", "gate_up_wgrad", "shared_wgrad")
    st = {"quantize_and_transpose_weights": detail["quantize_and_transpose_weights"],
          "forward": detail["forward"],
          "backward": sum(detail.get(k, 0.0) for k in bwd_keys),
          "weight_gradients": sum(detail.get(k, 0.0) for k in wg_keys),
          "bias_update": detail["bias_update"]}
    # the step's longest single launch: the routed gate|up weight gradient
    _, b13 = wgrad_bytes(E, H, I, wg)
    ms_w = detail["gate_up_wgrad"]
    roofline = dict(bound="hbm", achieved=b13 / ms_w / 1e6, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=b13 / ms_w / 1e6 / HBM_PEAK_GBS, traffic=None,
                    kernel="grouped_wgrad_fp8 (routed gate|up weight gradient, float32)",
                    algorithmic_bytes_per_launch=b13)
    cpu = None if args.no_cpu_baseline else cpu_baseline_train(cfg, d, dy)
    line = {"metric": "MoE-layer training step (FP8 weights, forward, backward, FP8 weight gradients), tokens/s, 1 GPU",
            "value": T / (total / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": total, "higher_is_better": True, "dtype": "fp8_e4m3",
            "data": "synthetic", "config": {"workload": cfg["name"]}, "stages_ms": st,
            "stages_detail_ms": detail, "roofline": roofline, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the expert-parallel multi-GPU path is not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch
    import routed_experts_fp8_amd as R
    import synth

    cfg = synth.get_config(args.config)
    dev = torch.device("cuda:0")
    T, H, E, I, K = cfg["T"], cfg["H"], cfg["E"], cfg["I"], cfg["K"]
    log(f"generating {cfg['name']} inputs on the GPU")
    d = synth.layer_inputs(cfg, dev, seed=0)
    w = R.quantize_weights(d["w13"], d["w2"], d.get("sw13"), d.get("sw2"))
    if args.section == "backward":
        backward_section(args, cfg, d, w, torch, R, synth)
        return
    if args.section == "wgrad":
        wgrad_section(args, cfg, d, w, torch, R, synth)
        return
    if args.section == "train":
        del w
        train_section(args, cfg, d, torch, R, synth)
        return
    fwd = R.MoEForward(T, H, E, I, cfg["route"], w, dev, fused=True, shared_I=cfg.get("shared_I"))
    torch.cuda.synchronize()
    log("warmup")
    for _ in range(args.warmup):
        fwd(d["x"], d["logits"], d["bias"])
    torch.cuda.synchronize()
    log("cold-cache steps")
    cold = cold_steps(lambda: fwd(d["x"], d["logits"], d["bias"]), 10, torch)
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    marks = []
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    def on_stage(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        marks[-1].append((name, e))

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        s = torch.cuda.Event(enable_timing=True)
        s.record()
        marks.append([("start", s)])
        fwd(d["x"], d["logits"], d["bias"], on_stage=on_stage)
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_per_step = start.elapsed_time(end) / args.steps
    step_ms = [marks[i][0][1].elapsed_time(marks[i + 1][0][1]) for i in range(len(marks) - 1)]
    step_ms.append(marks[-1][0][1].elapsed_time(end))
    stage_ms = {}
    for step in marks:
        for (_, a), (name, b) in zip(step[:-1], step[1:]):
            stage_ms[name] = stage_ms.get(name, 0.0) + a.elapsed_time(b) / args.steps

    tokens_per_s = T / (ms_per_step / 1e3)
    M = T * K
    g1_ms = stage_ms["gemm1"]
    g2_ms = stage_ms["gemm2"]
    g1_flops = gemm_flops(M, 2 * I, H)
    g2_flops = gemm_flops(M, H, I)
    g1_bytes = gemm1_bytes(T, K, H, E, I)
    g1_gbs = g1_bytes / g1_ms / 1e6
    gemm = dict(
        gemm1_swiglu=dict(ms=g1_ms, TFLOPs=g1_flops / g1_ms / 1e9,
                          frac_mfma=g1_flops / g1_ms / 1e9 / FP8_PEAK_TFLOPS, GBps=g1_gbs,
                          frac_hbm=g1_gbs / HBM_PEAK_GBS, flops=g1_flops, bytes=g1_bytes),
        gemm2=dict(ms=g2_ms, TFLOPs=g2_flops / g2_ms / 1e9,
                   frac_mfma=g2_flops / g2_ms / 1e9 / FP8_PEAK_TFLOPS),
    )
    all_gemm_ms = g1_ms + g2_ms
    all_gemm_flops = g1_flops + g2_flops
    if cfg.get("shared_I"):
        Is = cfg["shared_I"]
        sf1, sf2 = gemm_flops(T, 2 * Is, H), gemm_flops(T, H, Is)
        if "shared_gemm1" in stage_ms:  # shared expert in line on the main stream
            gemm["shared_gemm1_swiglu"] = dict(ms=stage_ms["shared_gemm1"],
                                               TFLOPs=sf1 / stage_ms["shared_gemm1"] / 1e9)
            gemm["shared_gemm2"] = dict(ms=stage_ms["shared_gemm2"], TFLOPs=sf2 / stage_ms["shared_gemm2"] / 1e9)
            all_gemm_ms += stage_ms["shared_gemm1"] + stage_ms["shared_gemm2"]
        else:  # on the side stream, overlapped with routing, permutation and the
            # routed GEMMs: the GEMM phase runs from the end of quant_act to the join
            gemm["shared_expert"] = dict(overlapped=True, flops=sf1 + sf2,
                                         join_wait_ms=stage_ms.get("shared_join", 0.0))
            all_gemm_ms += stage_ms.get("shared_join", 0.0) + stage_ms["permute"] + stage_ms["route"]
        all_gemm_flops += sf1 + sf2
    gemm["all_grouped_gemms"] = dict(ms=all_gemm_ms, TFLOPs=all_gemm_flops / all_gemm_ms / 1e9,
                                     frac_mfma=all_gemm_flops / all_gemm_ms / 1e9 / FP8_PEAK_TFLOPS)

    traffic = measured_traffic("gemm1_swiglu_dsv3", os.path.join(ROOT, "routed_experts_fp8_amd", "csrc",
                                                                  "gemm.hip"), cfg["name"])
    # the launch's bound from its arithmetic intensity: HBM below the ridge
    # point (peak flop/s over peak bytes/s = 625 flop/B), the FP8 matrix
    # cores above it (the compute-bound MoGE and skewed-load shapes)
    kernel = "grouped_gemm_fp8_swiglu (routed gate|up GEMM + SwiGLU + quant)"
    if g1_flops / g1_bytes <= FP8_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS:
        roofline = dict(bound="hbm", achieved=g1_gbs, peak=HBM_PEAK_GBS, unit="GB/s", frac=g1_gbs / HBM_PEAK_GBS,
                        traffic=traffic, kernel=kernel, algorithmic_bytes_per_launch=g1_bytes)
    else:
        g1_tf = g1_flops / g1_ms / 1e9
        roofline = dict(bound="mfma", achieved=g1_tf, peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=g1_tf / FP8_PEAK_TFLOPS, traffic=traffic, kernel=kernel,
                        algorithmic_flops_per_launch=g1_flops, algorithmic_bytes_per_launch=g1_bytes)

    extra = None
    if not args.no_extra:
        log("extra rows: weight quantisation, block transpose, dgrad")
        extra = extra_rows(cfg, d, fwd, torch, R, synth)
        log("router projection and bias update")
        extra["router"] = router_rows(cfg, d, fwd, torch, R, synth)
        log("input-side backward")
        extra["backward"] = backward_rows(cfg, d, w, torch, R, synth)
        log("fused stages on and off")
        extra["stage_fusions"] = fusion_rows(cfg, d, w, torch, R)
        log("small layer: eager vs HIP graph replay")
        extra["graph"] = graph_rows(torch, R, synth)
        log("other workloads: MoGE and skewed-load layers")
        extra["other_workloads"] = other_workload_rows(torch, R, synth)
        log("measured streaming ceiling: a plain 1 GiB device copy")
        extra["measured_copy"] = copy_rate(torch)
        log("measured FP8 matrix rate: a dense vendor-library FP8 GEMM")
        extra["measured_dense_fp8_gemm"] = dense_fp8_gemm_rate(torch)
        log("measured FP8 matrix-core ceiling: the library's register-only probe")
        extra["measured_mfma_fp8_probe"] = mfma_probe_rate(torch, R)
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, bounded sample)")
        cpu = cpu_baseline(cfg, d)

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_median": statistics.median(step_ms),
        "ms_per_step_min": min(step_ms),
        "wall_ms_per_step": wall_ms,
        "cold_cache": cold,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) activations and router logits, N(0,0.006) bf16 weights)",
        "config": {"workload": cfg["name"], "T": T, "hidden": H, "experts": E, "top_k": K,
                   "inter": I, "shared_inter": cfg.get("shared_I"), "route": cfg["route"]["mode"]},
        "gemm_tflops": gemm["all_grouped_gemms"]["TFLOPs"],
        "gemm_frac_mfma_peak": gemm["all_grouped_gemms"]["frac_mfma"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages_ms": stage_ms,
        "gemm": gemm,
        "gpu": {"name": torch.cuda.get_device_name(0), "clocks": gpu_clocks()},
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
