"""ctypes wrapper of oracle_c.c, the plain C forms of the oracle's weight
quantisation, E4M3 encoder, GEMM rows and binary32 sigmoid (oracle; test
infrastructure only).

They compute exactly what ``quant.quant_weight_128x128``,
``codec.e4m3_encode``, ``gemm.grouped_gemm`` and ``specmath.spec_sigmoid``
compute (the CPU tests hold them to those bit for bit); they exist because
the full-size checks touch hundreds of expert matrices of 4096 x 7168, and
the sigmoid check covers all 2^32 binary32 inputs, where the numpy forms
take seconds per matrix and minutes for the sweep.  The library is
compiled with gcc on first use (or by ``build()``), next to this file.
"""

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle_c.c")
LIB = os.path.join(_HERE, "liboracle_c.so")
_lib = None


def build():
    """Compile oracle_c.c: -O2, no contraction of a*b+c, no fast-math,
    OpenMP over independent outputs."""
    cc = os.environ.get("CC", "gcc")
    tmp = LIB + ".tmp"
    cmd = [cc, "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-Wall", "-o", tmp, SRC, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"oracle C build failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        p = ctypes.c_void_p
        lib.orc_e4m3_encode_many.argtypes = [p, ctypes.c_int64, p]
        lib.orc_quant_weight_128x128.argtypes = [p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, p, p]
        lib.orc_gemm_rows.argtypes = [p, p, ctypes.c_int64, p, p, ctypes.c_int32, ctypes.c_int32, p, p]
        f32 = ctypes.c_float
        lib.orc_spec_sigmoid_bits.argtypes = [ctypes.c_uint32, ctypes.c_int64, f32, f32, f32, p, p]
        lib.orc_spec_sigmoid.argtypes = [p, ctypes.c_int64, f32, f32, f32, p, p]
        for f in (lib.orc_e4m3_encode_many, lib.orc_quant_weight_128x128, lib.orc_gemm_rows,
                  lib.orc_spec_sigmoid_bits, lib.orc_spec_sigmoid):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def e4m3_encode(v):
    """As codec.e4m3_encode (finite values, |v| <= 448)."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > 448.0):
        raise ValueError("e4m3_encode expects finite values with |v| <= 448")
    out = np.empty(v.shape, np.uint8)
    _load().orc_e4m3_encode_many(_ptr(v), v.size, _ptr(out))
    return out


def quant_weight_128x128(w):
    """As quant.quant_weight_128x128: w [G, rows, cols] (or [rows, cols]) ->
    (codes u8 [G, rows, cols], scales f32 [G, rows/128, cols/128])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim == 2:
        w = w[None]
    G, rows, cols = w.shape
    if rows % 128 or cols % 128:
        raise ValueError("rows and cols must be multiples of 128")
    if not np.all(np.isfinite(w)):
        raise ValueError("finite weights expected")
    q = np.empty(w.shape, np.uint8)
    s = np.empty((G, rows // 128, cols // 128), np.float32)
    _load().orc_quant_weight_128x128(_ptr(w), G, rows, cols, _ptr(q), _ptr(s))
    return q, s


def gemm_rows(aq, as_, bq, bs, with_mag=True):
    """As gemm.grouped_gemm with one group: rows aq [m, K] (scales [m, K/128])
    against bq [N, K] (block scales [N/128, K/128]) -> (C float64 [m, N],
    Mag or None)."""
    aq = np.ascontiguousarray(aq, dtype=np.uint8)
    as_ = np.ascontiguousarray(as_, dtype=np.float32)
    bq = np.ascontiguousarray(bq, dtype=np.uint8)
    bs = np.ascontiguousarray(bs, dtype=np.float32)
    m, K = aq.shape
    N = bq.shape[0]
    if bq.shape[1] != K or K % 128 or N % 128:
        raise ValueError("shape mismatch or dims not multiples of 128")
    if as_.shape != (m, K // 128) or bs.shape != (N // 128, K // 128):
        raise ValueError("scale shapes")
    C = np.empty((m, N))
    Mag = np.empty((m, N)) if with_mag else None
    _load().orc_gemm_rows(_ptr(aq), _ptr(as_), m, _ptr(bq), _ptr(bs), N, K, _ptr(C),
                          None if Mag is None else _ptr(Mag))
    return C, Mag


def _spec_consts():
    from .specmath import LN2_HI, LN2_LO, LOG2E, TAYLOR
    taylor = np.array(TAYLOR, np.float32)
    return float(LOG2E), float(LN2_HI), float(LN2_LO), taylor


def spec_sigmoid(x):
    """As specmath.spec_sigmoid (NaN inputs give NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.float32)
    log2e, hi, lo, taylor = _spec_consts()
    _load().orc_spec_sigmoid(_ptr(x), x.size, log2e, hi, lo, _ptr(taylor), _ptr(out))
    return out


def spec_sigmoid_bits(start, n):
    """spec_sigmoid of the n binary32 values with bit patterns start, start+1,
    ... (modulo 2^32)."""
    out = np.empty(int(n), np.float32)
    log2e, hi, lo, taylor = _spec_consts()
    _load().orc_spec_sigmoid_bits(int(start) & 0xFFFFFFFF, int(n), log2e, hi, lo, _ptr(taylor), _ptr(out))
    return out
