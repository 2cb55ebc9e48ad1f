"""ctypes binding of libmoefp8.so: one Python function per C entry point,
same names, argument marshalling only (shape/dtype/device checks, output
allocation when no `out` is given, the current torch stream).  Every step
of the computation runs in the library's HIP kernels; there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoefp8.so")

MOE_OK = 0
MOE_F32, MOE_BF16 = 0, 1
ROUTE_SIGMOID_BIAS, ROUTE_SOFTMAX_GROUPED = 0, 1

_c_void_p = ctypes.c_void_p
_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_last_error_detail": (ctypes.c_char_p, []),
    "moe_route": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                         _c_void_p, _c_void_p, _c_void_p]),
    "moe_sigmoid_f32": (_i32, [_c_void_p, _i64, _c_void_p, _c_void_p]),
    "moe_permute_workspace_size": (_i32, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "moe_permute": (_i32, [_c_void_p, _i32, _i32, _i32, _c_void_p, _c_void_p, _i32, _c_void_p,
                           _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_route_permute_workspace_size": (_i32, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "moe_route_permute": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _c_void_p,
                                 _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _sz, _c_void_p]),
    "moe_permute_noalloc": (_i32, [_c_void_p, _i32, _i32, _i32, _c_void_p, _c_void_p, _i32, _c_void_p,
                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "quant_act_1x128_e4m3": (_i32, [_c_void_p, _i32, _i64, _i32, _c_void_p, _c_void_p, _c_void_p]),
    "quant_weight_128x128_e4m3": (_i32, [_c_void_p, _i32, _i32, _i32, _i32, _c_void_p, _c_void_p,
                                         _c_void_p]),
    "quant_weight_128x128_e4m3_t": (_i32, [_c_void_p, _i32, _i32, _i32, _i32, _c_void_p, _c_void_p,
                                           _c_void_p, _c_void_p, _c_void_p]),
    "grouped_gemm_fp8_blockscaled": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32,
                                            _i64, _i32, _i32, _c_void_p, _i32, _c_void_p]),
    "grouped_gemm_fp8_blockscaled_gather": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p,
                                                   _c_void_p, _c_void_p, _i32, _i64, _i32, _i32, _c_void_p,
                                                   _i32, _c_void_p]),
    "grouped_gemm_fp8_swiglu": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _c_void_p,
                                       _c_void_p, _i32, _i64, _i32, _i32, _c_void_p, _c_void_p, _c_void_p]),
    "grouped_gemm_fp8_combine_workspace_size": (_i32, [_i32, _i32, ctypes.POINTER(_sz)]),
    "grouped_gemm_fp8_combine": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64, _i32,
                                        _i32, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32,
                                        _c_void_p, _c_void_p, _sz, _c_void_p]),
    "swiglu": (_i32, [_c_void_p, _i64, _i32, _c_void_p, _c_void_p, _c_void_p]),
    "moe_combine": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _c_void_p,
                           _c_void_p]),
    "fp8_block_transpose": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i32, _c_void_p, _c_void_p,
                                   _c_void_p]),
    "moe_combine_backward": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                    _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "swiglu_backward": (_i32, [_c_void_p, _c_void_p, _i64, _i32, _c_void_p, _c_void_p, _c_void_p,
                               _c_void_p]),
    "moe_route_backward": (_i32, [_c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32, _i32, _i32,
                                  _c_void_p, _c_void_p]),
    "moe_wgrad_padded_rows": (_i32, [_i64, _i32, ctypes.POINTER(_i64)]),
    "quant_act_128x1_grouped_e4m3": (_i32, [_c_void_p, _i32, _i32, _i64, _i32, _c_void_p, _c_void_p,
                                            _c_void_p, _i32, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                            _c_void_p]),
    "grouped_wgrad_fp8": (_i32, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i32, _i32,
                                 _i64, _c_void_p, _i32, _i32, _c_void_p]),
    "moe_router_logits": (_i32, [_c_void_p, _c_void_p, _i32, _i32, _i32, _c_void_p, _c_void_p]),
    "moe_bias_update": (_i32, [_c_void_p, _i32, ctypes.c_float, _c_void_p, _c_void_p]),
    "moe_probe_mfma_fp8": (_i32, [ctypes.c_uint8, _i64, _i32, _i32, _c_void_p, ctypes.POINTER(ctypes.c_double),
                                  _c_void_p]),
}


class MoeError(RuntimeError):
    """A non-OK status from libmoefp8."""

    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({detail})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python routed_experts_fp8_amd/build.py` (or __graft_entry__.build()) "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(s):
    return lib.moe_status_string(int(s)).decode()


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status, lib.moe_last_error_detail().decode())


def _p(t):
    return None if t is None else _c_void_p(t.data_ptr())


def _stream():
    return _c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        # work is enqueued on the current device's stream
        raise ValueError(f"{name} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _out(out, name, shape, dtype, device):
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return _need(out, name, dtype, shape)


def _even(n, name):
    if n % 2:
        raise ValueError(f"{name} must be even (a gate half and an up half), got {n}")
    return n // 2


def _dtype_code(t):
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


# ---------------------------------------------------------------------------


def moe_route(logits, bias, K, mode="sigmoid_bias", n_groups=1, k_per_group=None, normalize=True,
              topk_idx=None, topk_gate=None):
    """-> (topk_idx int32 [T, K], topk_gate float32 [T, K])."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    m = ROUTE_SIGMOID_BIAS if mode == "sigmoid_bias" else ROUTE_SOFTMAX_GROUPED
    if m == ROUTE_SOFTMAX_GROUPED:
        k_per_group = K // n_groups if k_per_group is None else k_per_group
        normalize = False
    idx = _out(topk_idx, "topk_idx", (T, K), torch.int32, logits.device)
    gate = _out(topk_gate, "topk_gate", (T, K), torch.float32, logits.device)
    _check("moe_route", lib.moe_route(_p(logits), _p(bias), T, E, K, n_groups,
                                      k_per_group or K, m, int(bool(normalize)), _p(idx), _p(gate),
                                      _stream()))
    return idx, gate


def moe_sigmoid_f32(x, y=None):
    """y = sigmoid(x) elementwise (float32, any shape), the routing's binary32
    sigmoid."""
    _need(x, "x", torch.float32)
    y = _out(y, "y", tuple(x.shape), torch.float32, x.device)
    _check("moe_sigmoid_f32", lib.moe_sigmoid_f32(_p(x), x.numel(), _p(y), _stream()))
    return y


def moe_permute_workspace_size(T, K, E):
    n = _sz(0)
    _check("moe_permute_workspace_size", lib.moe_permute_workspace_size(T, K, E, ctypes.byref(n)))
    return n.value


def _permute_outputs(topk_idx, E, xq, xs, out):
    _need(topk_idx, "topk_idx", torch.int32)
    T, K = topk_idx.shape
    dev = topk_idx.device
    out = dict(out or {})
    H = 0
    if xq is not None:
        _need(xq, "xq", torch.uint8)
        H = xq.shape[1]
        _need(xs, "xs", torch.float32, (T, H // 128))
        if xq.shape[0] != T:
            raise ValueError("xq rows must equal T")
    res = {
        "offsets": _out(out.get("offsets"), "offsets", (E + 1,), torch.int32, dev),
        "dst_row": _out(out.get("dst_row"), "dst_row", (T, K), torch.int32, dev),
        "src_token": _out(out.get("src_token"), "src_token", (T * K,), torch.int32, dev),
    }
    if xq is not None:
        res["aq"] = _out(out.get("aq"), "aq", (T * K, H), torch.uint8, dev)
        res["as"] = _out(out.get("as"), "as", (T * K, H // 128), torch.float32, dev)
    return T, K, H, res


def moe_permute(topk_idx, E, xq=None, xs=None, out=None, workspace=None):
    """-> dict(offsets [E+1], dst_row [T, K], src_token [T*K], aq, as)."""
    T, K, H, res = _permute_outputs(topk_idx, E, xq, xs, out)
    need = moe_permute_workspace_size(T, K, E)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=topk_idx.device)
    _need(workspace, "workspace", torch.uint8)
    _check("moe_permute", lib.moe_permute(
        _p(topk_idx), T, K, E, _p(xq), _p(xs), H, _p(res["offsets"]), _p(res["dst_row"]),
        _p(res["src_token"]), _p(res.get("aq")), _p(res.get("as")), _p(workspace),
        workspace.numel(), _stream()))
    return res


def moe_permute_noalloc(topk_idx, E, xq=None, xs=None, out=None):
    """moe_permute with the library's static scratch instead of a workspace
    (the library allocates nothing; pass every output in ``out`` to allocate
    nothing here either)."""
    T, K, H, res = _permute_outputs(topk_idx, E, xq, xs, out)
    _check("moe_permute_noalloc", lib.moe_permute_noalloc(
        _p(topk_idx), T, K, E, _p(xq), _p(xs), H, _p(res["offsets"]), _p(res["dst_row"]),
        _p(res["src_token"]), _p(res.get("aq")), _p(res.get("as")), _stream()))
    return res


def moe_route_permute_workspace_size(T, K, E):
    n = _sz(0)
    _check("moe_route_permute_workspace_size", lib.moe_route_permute_workspace_size(T, K, E, ctypes.byref(n)))
    return n.value


def moe_route_permute(logits, bias, K, mode="sigmoid_bias", n_groups=1, k_per_group=None, normalize=True,
                      workspace=None, out=None):
    """moe_route and moe_permute's index maps in one launch -> dict(topk_idx,
    topk_gate, offsets, dst_row, src_token).  The first 256 bytes of
    ``workspace`` (uint8) must be zero before its first use (every call
    leaves them zero); without one a zero-filled workspace is allocated for
    this call."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    if bias is not None:
        _need(bias, "bias", torch.float32, (E,))
    m = ROUTE_SIGMOID_BIAS if mode == "sigmoid_bias" else ROUTE_SOFTMAX_GROUPED
    if m == ROUTE_SOFTMAX_GROUPED:
        k_per_group = K // n_groups if k_per_group is None else k_per_group
        normalize = False
    dev = logits.device
    out = dict(out or {})
    res = {
        "topk_idx": _out(out.get("topk_idx"), "topk_idx", (T, K), torch.int32, dev),
        "topk_gate": _out(out.get("topk_gate"), "topk_gate", (T, K), torch.float32, dev),
        "offsets": _out(out.get("offsets"), "offsets", (E + 1,), torch.int32, dev),
        "dst_row": _out(out.get("dst_row"), "dst_row", (T, K), torch.int32, dev),
        "src_token": _out(out.get("src_token"), "src_token", (T * K,), torch.int32, dev),
    }
    if workspace is None:
        workspace = torch.zeros(moe_route_permute_workspace_size(T, K, E), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8)
    _check("moe_route_permute", lib.moe_route_permute(
        _p(logits), _p(bias), T, E, K, n_groups, k_per_group or K, m, int(bool(normalize)), _p(res["topk_idx"]),
        _p(res["topk_gate"]), _p(res["offsets"]), _p(res["dst_row"]), _p(res["src_token"]), _p(workspace),
        workspace.numel(), _stream()))
    return res


def quant_act_1x128_e4m3(x, q=None, scale=None):
    """x float32/bf16 [rows, cols] -> (codes uint8 [rows, cols], scales f32 [rows, cols/128])."""
    code = _dtype_code(x)
    _need(x, "x", x.dtype)
    rows, cols = x.shape
    q = _out(q, "q", (rows, cols), torch.uint8, x.device)
    scale = _out(scale, "scale", (rows, cols // 128), torch.float32, x.device)
    _check("quant_act_1x128_e4m3", lib.quant_act_1x128_e4m3(_p(x), code, rows, cols, _p(q),
                                                            _p(scale), _stream()))
    return q, scale


def quant_weight_128x128_e4m3(w, q=None, scale=None):
    """w float32/bf16 [G, rows, cols] -> (codes [G, rows, cols], scales [G, rows/128, cols/128])."""
    code = _dtype_code(w)
    _need(w, "w", w.dtype)
    G, rows, cols = w.shape
    q = _out(q, "q", (G, rows, cols), torch.uint8, w.device)
    scale = _out(scale, "scale", (G, rows // 128, cols // 128), torch.float32, w.device)
    _check("quant_weight_128x128_e4m3", lib.quant_weight_128x128_e4m3(
        _p(w), code, G, rows, cols, _p(q), _p(scale), _stream()))
    return q, scale


def quant_weight_128x128_e4m3_t(w, q=None, scale=None, qt=None, scale_t=None):
    """As quant_weight_128x128_e4m3, plus the block-transposed codes
    [G, cols, rows] and scales [G, cols/128, rows/128] from the same pass
    -> (q, scale, qt, scale_t)."""
    code = _dtype_code(w)
    _need(w, "w", w.dtype)
    G, rows, cols = w.shape
    q = _out(q, "q", (G, rows, cols), torch.uint8, w.device)
    scale = _out(scale, "scale", (G, rows // 128, cols // 128), torch.float32, w.device)
    qt = _out(qt, "qt", (G, cols, rows), torch.uint8, w.device)
    scale_t = _out(scale_t, "scale_t", (G, cols // 128, rows // 128), torch.float32, w.device)
    _check("quant_weight_128x128_e4m3_t", lib.quant_weight_128x128_e4m3_t(
        _p(w), code, G, rows, cols, _p(q), _p(scale), _p(qt), _p(scale_t), _stream()))
    return q, scale, qt, scale_t


def _gemm_operands(aq, as_, bq, bs, offsets, a_row):
    _need(aq, "aq", torch.uint8)
    A, K = aq.shape
    _need(as_, "as", torch.float32, (A, K // 128))
    if a_row is not None:
        _need(a_row, "a_row", torch.int32)
        if a_row.dim() != 1:
            raise ValueError("a_row must be 1-D [M]")
    M = A if a_row is None else a_row.shape[0]
    _need(bq, "bq", torch.uint8)
    G, N, K2 = bq.shape
    if K2 != K:
        raise ValueError(f"bq reduction dim {K2} != aq's {K}")
    _need(bs, "bs", torch.float32, (G, N // 128, K // 128))
    _need(offsets, "group_offsets", torch.int32, (G + 1,))
    return M, K, G, N, A


def _c_out(c, out_dtype, M, N, device):
    if c is not None and c.dtype in (torch.float32, torch.bfloat16):
        out_dtype = c.dtype                       # a given output buffer sets the type
    return _out(c, "c", (M, N), out_dtype, device)


def grouped_gemm_fp8_blockscaled(aq, as_, bq, bs, offsets, out_dtype=torch.float32, c=None):
    """C[M, N] = per-group A . B_g^T with block scales (float32 or bf16 output;
    the type of ``c`` when given, else ``out_dtype``)."""
    M, K, G, N, A = _gemm_operands(aq, as_, bq, bs, offsets, None)
    c = _c_out(c, out_dtype, M, N, aq.device)
    _check("grouped_gemm_fp8_blockscaled", lib.grouped_gemm_fp8_blockscaled(
        _p(aq), _p(as_), _p(bq), _p(bs), _p(offsets), G, M, N, K, _p(c), _dtype_code(c), _stream()))
    return c


def grouped_gemm_fp8_blockscaled_gather(aq, as_, a_row, bq, bs, offsets, out_dtype=torch.float32, c=None):
    """As grouped_gemm_fp8_blockscaled with row m of A read from aq[a_row[m]]
    (a_row int32 [M]; aq / as in token order)."""
    if a_row is None:
        raise ValueError("a_row is required")
    M, K, G, N, A = _gemm_operands(aq, as_, bq, bs, offsets, a_row)
    c = _c_out(c, out_dtype, M, N, aq.device)
    _check("grouped_gemm_fp8_blockscaled_gather", lib.grouped_gemm_fp8_blockscaled_gather(
        _p(aq), _p(as_), _p(a_row), A, _p(bq), _p(bs), _p(offsets), G, M, N, K, _p(c), _dtype_code(c),
        _stream()))
    return c


def grouped_gemm_fp8_swiglu(aq, as_, bq, bs, offsets, hq=None, hs=None, a_row=None):
    """Gate|up GEMM with fused SwiGLU + 1x128 quantisation -> (hq [M, I], hs [M, I/128]).
    a_row (int32 [M]), if given, gathers row m of A from aq[a_row[m]]."""
    M, K, G, N, A = _gemm_operands(aq, as_, bq, bs, offsets, a_row)
    I = _even(N, "bq rows per group (2I)")
    hq = _out(hq, "hq", (M, I), torch.uint8, aq.device)
    hs = _out(hs, "hs", (M, I // 128), torch.float32, aq.device)
    _check("grouped_gemm_fp8_swiglu", lib.grouped_gemm_fp8_swiglu(
        _p(aq), _p(as_), _p(a_row), A, _p(bq), _p(bs), _p(offsets), G, M, I, K, _p(hq), _p(hs), _stream()))
    return hq, hs


def grouped_gemm_fp8_combine_workspace_size(T, N):
    n = _sz(0)
    _check("grouped_gemm_fp8_combine_workspace_size",
           lib.grouped_gemm_fp8_combine_workspace_size(T, N, ctypes.byref(n)))
    return n.value


def grouped_gemm_fp8_combine(aq, as_, bq, bs, offsets, src_token, dst_row, topk_gate, shared=None, c=None,
                             y=None, counters=None):
    """The down projection with the combine fused into its epilogue ->
    (c f32 [M, N], y bf16 [T, N]), both identical to grouped_gemm_fp8_blockscaled
    followed by moe_combine.  ``counters`` (int32) must have been zero-filled
    before its first use (every call leaves it zero-filled); without it a
    zero-filled one is allocated for this call."""
    M, K, G, N, A = _gemm_operands(aq, as_, bq, bs, offsets, None)
    _need(dst_row, "dst_row", torch.int32)
    T, topk = dst_row.shape
    _need(src_token, "src_token", torch.int32, (M,))
    _need(topk_gate, "topk_gate", torch.float32, (T, topk))
    if shared is not None:
        _need(shared, "shared", torch.float32, (T, N))
    c = _out(c, "c", (M, N), torch.float32, aq.device)
    y = _out(y, "y", (T, N), torch.bfloat16, aq.device)
    need = grouped_gemm_fp8_combine_workspace_size(T, N)
    if counters is None:
        counters = torch.zeros(max(need // 4, 1), dtype=torch.int32, device=aq.device)
    _need(counters, "counters", torch.int32)
    _check("grouped_gemm_fp8_combine", lib.grouped_gemm_fp8_combine(
        _p(aq), _p(as_), _p(bq), _p(bs), _p(offsets), G, M, N, K, _p(c), _p(src_token), _p(dst_row),
        _p(topk_gate), _p(shared), T, topk, _p(y), _p(counters), counters.numel() * 4, _stream()))
    return c, y


def swiglu(gate_up, hq=None, hs=None):
    """gate_up float32 [M, 2I] -> (hq uint8 [M, I], hs float32 [M, I/128])."""
    _need(gate_up, "gate_up", torch.float32)
    M, twoI = gate_up.shape
    I = _even(twoI, "gate_up columns (2I)")
    hq = _out(hq, "hq", (M, I), torch.uint8, gate_up.device)
    hs = _out(hs, "hs", (M, I // 128), torch.float32, gate_up.device)
    _check("swiglu", lib.swiglu(_p(gate_up), M, I, _p(hq), _p(hs), _stream()))
    return hq, hs


def moe_combine(y_perm, dst_row, topk_gate, shared=None, out=None):
    """-> y bf16 [T, H] = sum_k gate * y_perm[dst_row] (+ shared)."""
    _need(y_perm, "y_perm", torch.float32)
    _need(dst_row, "dst_row", torch.int32)
    T, K = dst_row.shape
    H = y_perm.shape[1]
    _need(topk_gate, "topk_gate", torch.float32, (T, K))
    if y_perm.shape[0] != T * K:
        raise ValueError("y_perm must have T*K rows")
    if shared is not None:
        _need(shared, "shared", torch.float32, (T, H))
    out = _out(out, "out", (T, H), torch.bfloat16, y_perm.device)
    _check("moe_combine", lib.moe_combine(_p(y_perm), _p(dst_row), _p(topk_gate), _p(shared), T, K,
                                          H, _p(out), _stream()))
    return out


def fp8_block_transpose(q, scale, qt=None, scale_t=None):
    """(q [G, R, C], s [G, R/128, C/128]) -> (q^T [G, C, R], s^T [G, C/128, R/128])."""
    _need(q, "q", torch.uint8)
    G, R, C = q.shape
    _need(scale, "scale", torch.float32, (G, R // 128, C // 128))
    qt = _out(qt, "qt", (G, C, R), torch.uint8, q.device)
    scale_t = _out(scale_t, "scale_t", (G, C // 128, R // 128), torch.float32, q.device)
    _check("fp8_block_transpose", lib.fp8_block_transpose(_p(q), _p(scale), G, R, C, _p(qt),
                                                          _p(scale_t), _stream()))
    return qt, scale_t


def moe_combine_backward(dy, y_perm, dst_row, topk_gate, dq=None, ds=None, d_gate=None, gate_row=None):
    """dy bf16 [T, H], y_perm f32 [T*K, H] -> (dq u8 [T*K, H], ds f32 [T*K, H/128],
    d_gate f32 [T, K]): the combine's gradient, quantised for the down dgrad.
    gate_row (f32 [T*K], optional) receives each grouped row's gate."""
    _need(dy, "dy", torch.bfloat16)
    _need(y_perm, "y_perm", torch.float32)
    _need(dst_row, "dst_row", torch.int32)
    T, K = dst_row.shape
    H = dy.shape[1]
    if dy.shape[0] != T or y_perm.shape != (T * K, H):
        raise ValueError("dy must be [T, H] and y_perm [T*K, H]")
    _need(topk_gate, "topk_gate", torch.float32, (T, K))
    dq = _out(dq, "dq", (T * K, H), torch.uint8, dy.device)
    ds = _out(ds, "ds", (T * K, H // 128), torch.float32, dy.device)
    d_gate = _out(d_gate, "d_gate", (T, K), torch.float32, dy.device)
    if gate_row is not None:
        _need(gate_row, "gate_row", torch.float32, (T * K,))
    _check("moe_combine_backward", lib.moe_combine_backward(
        _p(dy), _p(y_perm), _p(dst_row), _p(topk_gate), T, K, H, _p(dq), _p(ds), _p(d_gate), _p(gate_row),
        _stream()))
    return dq, ds, d_gate


def swiglu_backward(gate_up, dh, dq=None, ds=None, d=None):
    """gate_up f32 [M, 2I], dh f32 [M, I] -> (dq u8 [M, 2I], ds f32 [M, 2I/128]).
    d (f32 [M, 2I], optional) receives [dg | du] unquantised."""
    _need(gate_up, "gate_up", torch.float32)
    M, twoI = gate_up.shape
    I = _even(twoI, "gate_up columns (2I)")
    _need(dh, "dh", torch.float32, (M, I))
    dq = _out(dq, "dq", (M, twoI), torch.uint8, gate_up.device)
    ds = _out(ds, "ds", (M, twoI // 128), torch.float32, gate_up.device)
    if d is not None:
        _need(d, "d", torch.float32, (M, twoI))
    _check("swiglu_backward", lib.swiglu_backward(_p(gate_up), _p(dh), M, I, _p(dq), _p(ds), _p(d), _stream()))
    return dq, ds


def moe_route_backward(logits, topk_idx, d_gate, mode="sigmoid_bias", normalize=True, d_logits=None):
    """-> d_logits f32 [T, E], the router-logit gradient through the selected experts."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    _need(topk_idx, "topk_idx", torch.int32)
    K = topk_idx.shape[1]
    _need(d_gate, "d_gate", torch.float32, (T, K))
    m = ROUTE_SIGMOID_BIAS if mode == "sigmoid_bias" else ROUTE_SOFTMAX_GROUPED
    d_logits = _out(d_logits, "d_logits", (T, E), torch.float32, logits.device)
    _check("moe_route_backward", lib.moe_route_backward(
        _p(logits), _p(topk_idx), _p(d_gate), T, E, K, m, int(bool(normalize)), _p(d_logits), _stream()))
    return d_logits


def moe_wgrad_padded_rows(M, G):
    """Smallest admissible row stride of the 128x1-quantised operands."""
    n = _i64(0)
    _check("moe_wgrad_padded_rows", lib.moe_wgrad_padded_rows(int(M), int(G), ctypes.byref(n)))
    return n.value


def quant_act_128x1_grouped_e4m3(x, group_offsets, M=None, row_index=None, row_scale=None, swiglu_input=False,
                                 ld=None, qt=None, st=None, padded_offsets=None):
    """128x1 (token-dimension) quantisation of a grouped operand, transposed:
    x [x_rows, C] (f32/bf16) or, with swiglu_input, f32 gate|up [x_rows, 2C]
    -> (qt u8 [C, ld], st f32 [ld/128, C] (tile-major), padded_offsets i32 [G+1])."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _need(x, "x", x.dtype)
    x_rows, cols = x.shape
    C = _even(cols, "gate|up input columns (2C)") if swiglu_input else cols
    _need(group_offsets, "group_offsets", torch.int32)
    G = group_offsets.shape[0] - 1
    if M is None:
        M = row_index.shape[0] if row_index is not None else x_rows
    if row_index is not None:
        _need(row_index, "row_index", torch.int32, (M,))
    if row_scale is not None:
        _need(row_scale, "row_scale", torch.float32, (M,))
    ld = moe_wgrad_padded_rows(M, G) if ld is None else int(ld)
    qt = _out(qt, "qt", (C, ld), torch.uint8, x.device)
    st = _out(st, "st", (ld // 128, C), torch.float32, x.device)
    padded_offsets = _out(padded_offsets, "padded_offsets", (G + 1,), torch.int32, x.device)
    _check("quant_act_128x1_grouped_e4m3", lib.quant_act_128x1_grouped_e4m3(
        _p(x), _dtype_code(x), int(bool(swiglu_input)), x_rows, C, _p(row_index), _p(row_scale),
        _p(group_offsets), G, M, ld, _p(padded_offsets), _p(qt), _p(st), _stream()))
    return qt, st, padded_offsets


def grouped_wgrad_fp8(aq, as_, bq, bs, padded_offsets, out_dtype=torch.float32, c=None, accumulate=False):
    """dW [G, Na, Nb] = per-expert dOut^T . In over the 128x1-quantised operands
    aq [Na, ld] (output gradient) and bq [Nb, ld] (input), scales tile-major
    as [ld/128, Na], bs [ld/128, Nb]."""
    _need(aq, "aq", torch.uint8)
    Na, ld = aq.shape
    _need(as_, "as", torch.float32, (ld // 128, Na))
    _need(bq, "bq", torch.uint8)
    Nb = bq.shape[0]
    if bq.shape[1] != ld:
        raise ValueError("aq and bq must share the padded row stride")
    _need(bs, "bs", torch.float32, (ld // 128, Nb))
    _need(padded_offsets, "padded_offsets", torch.int32)
    G = padded_offsets.shape[0] - 1
    if c is not None and c.dtype in (torch.float32, torch.bfloat16):
        out_dtype = c.dtype
    c = _out(c, "c", (G, Na, Nb), out_dtype, aq.device)
    _check("grouped_wgrad_fp8", lib.grouped_wgrad_fp8(
        _p(aq), _p(as_), _p(bq), _p(bs), _p(padded_offsets), G, Na, Nb, ld, _p(c), _dtype_code(c),
        int(bool(accumulate)), _stream()))
    return c


def moe_router_logits(x, w_router, logits=None):
    """x bf16 [T, H], w_router f32 [E, H] -> logits f32 [T, E] = x . W_r^T."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    _need(w_router, "w_router", torch.float32)
    E = w_router.shape[0]
    if w_router.shape[1] != H:
        raise ValueError("w_router must be [E, H]")
    logits = _out(logits, "logits", (T, E), torch.float32, x.device)
    _check("moe_router_logits", lib.moe_router_logits(_p(x), _p(w_router), T, H, E, _p(logits), _stream()))
    return logits


def moe_bias_update(expert_offsets, gamma, bias):
    """In place: bias[e] -= gamma * sign(load_e - mean load), loads from the
    permutation's expert offsets."""
    _need(expert_offsets, "expert_offsets", torch.int32)
    E = expert_offsets.shape[0] - 1
    _need(bias, "bias", torch.float32, (E,))
    _check("moe_bias_update", lib.moe_bias_update(_p(expert_offsets), E, float(gamma), _p(bias), _stream()))
    return bias


def moe_probe_mfma_fp8(iters, blocks, waves_per_block, code=0x38, out=None):
    """Measurement helper (not a layer step): `blocks` workgroups of
    `waves_per_block` waves run 8 chains of `iters` FP8 matrix instructions
    on register operands (every code `code`); returns (out, flops) with out
    the per-lane accumulator sums [blocks * 64 * waves_per_block] and flops
    the launch's flop count."""
    n = blocks * 64 * waves_per_block
    out = _out(out, "out", (n,), torch.float32, torch.device("cuda", torch.cuda.current_device()))
    fl = ctypes.c_double(0.0)
    _check("moe_probe_mfma_fp8", lib.moe_probe_mfma_fp8(int(code), int(iters), int(blocks), int(waves_per_block),
                                                         _p(out), ctypes.byref(fl), _stream()))
    return out, fl.value
