"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/moefp8.h declares, reports workspace sizes, and
rejects bad arguments with the documented status before touching the device.
Every call here fails validation or is an empty problem, so no kernel is
ever launched."""

import ctypes
import os
import re

import pytest

from routed_experts_fp8_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = open(os.path.join(ROOT, "include", "moefp8.h")).read()
DECLARED = re.findall(r"^MOE_API\s+[\w\s\*]*?\b(\w+)\s*\(", HEADER, flags=re.M)

OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5
P = ctypes.c_void_p(0x10000)          # aligned non-NULL fake device pointer (never dereferenced)
PM = ctypes.c_void_p(0x10004)         # 4-byte aligned, not 16-byte aligned
N0 = None
S = None                              # null stream


# the eight operations of the layer's problem statement (routing, permutation,
# the two quantisers, the block-scaled grouped GEMM, SwiGLU, the combine and
# the block transpose)
CORE = ["moe_route", "moe_permute", "quant_act_1x128_e4m3", "quant_weight_128x128_e4m3",
        "grouped_gemm_fp8_blockscaled", "swiglu", "moe_combine", "fp8_block_transpose"]


def test_every_declared_symbol_is_exported():
    assert set(CORE) <= set(DECLARED), DECLARED
    for name in DECLARED:
        assert hasattr(L.lib, name), name
    assert set(DECLARED) == set(L._SIGNATURES)


def test_status_strings():
    for s in range(7):
        assert L.status_string(s).startswith("MOE_")
    assert "unknown" in L.status_string(99)


def test_workspace_size():
    n = ctypes.c_size_t(0)
    assert L.lib.moe_permute_workspace_size(4096, 8, 256, ctypes.byref(n)) == OK
    assert n.value == 2 * 16 * 256 * 4 + 256
    assert L.lib.moe_permute_workspace_size(0, 1, 1, ctypes.byref(n)) == OK
    assert L.lib.moe_permute_workspace_size(10, 9, 8, ctypes.byref(n)) == SHAPE
    assert L.lib.moe_permute_workspace_size(10, 8, 2048, ctypes.byref(n)) == UNSUP
    assert L.lib.moe_permute_workspace_size(10, 8, 64, None) == NULL


def _detail():
    return L.lib.moe_last_error_detail().decode()


def test_quant_errors():
    f = L.lib.quant_act_1x128_e4m3
    assert f(P, 0, 4, 100, P, P, S) == SHAPE and "cols" in _detail()
    assert f(P, 0, -1, 128, P, P, S) == SHAPE
    assert f(P, 7, 4, 128, P, P, S) == UNSUP
    assert f(N0, 0, 4, 128, P, P, S) == NULL
    assert f(PM, 1, 4, 128, P, P, S) == ALIGN
    assert f(N0, 0, 0, 128, N0, N0, S) == OK          # empty: nothing to do
    g = L.lib.quant_weight_128x128_e4m3
    assert g(P, 0, 2, 100, 128, P, P, S) == SHAPE
    assert g(P, 0, 2, 128, 130, P, P, S) == SHAPE
    assert g(P, 0, 2, 128, 128, N0, P, S) == NULL
    assert g(P, 0, 2, 128, 128, PM, P, S) == ALIGN
    assert g(P, 7, 2, 128, 128, P, P, S) == UNSUP
    assert g(N0, 0, 0, 128, 128, N0, N0, S) == OK
    t = L.lib.quant_weight_128x128_e4m3_t
    assert t(P, 0, 2, 100, 128, P, P, P, P, S) == SHAPE
    assert t(P, 0, 2, 128, 128, N0, P, P, P, S) == NULL
    assert t(P, 0, 2, 128, 128, P, P, P, N0, S) == NULL                  # qt without scale_t
    assert t(P, 0, 2, 128, 128, P, P, N0, P, S) == NULL                  # scale_t without qt
    assert t(P, 0, 2, 128, 128, PM, P, P, P, S) == ALIGN
    assert t(P, 0, 2, 128, 128, P, P, PM, P, S) == ALIGN                 # qt 16-byte
    assert t(N0, 0, 0, 128, 128, N0, N0, N0, N0, S) == OK


def test_route_errors():
    f = L.lib.moe_route
    sig, grp = L.ROUTE_SIGMOID_BIAS, L.ROUTE_SOFTMAX_GROUPED
    assert f(P, N0, 4, 2048, 8, 1, 8, sig, 1, P, P, S) == UNSUP
    assert f(P, N0, 4, 16, 17, 1, 17, sig, 1, P, P, S) == SHAPE
    assert f(P, N0, 4, 16, 0, 1, 0, sig, 1, P, P, S) == SHAPE
    assert f(P, N0, 4, 18, 4, 4, 1, grp, 0, P, P, S) == SHAPE      # E % G
    assert f(P, N0, 4, 16, 8, 4, 1, grp, 0, P, P, S) == SHAPE      # K != G*K'
    assert f(P, N0, 4, 16, 20, 4, 5, grp, 0, P, P, S) == SHAPE      # K' > E/G
    assert f(P, N0, 4, 16, 4, 4, 1, grp, 1, P, P, S) == UNSUP      # no renormalisation
    assert f(N0, N0, 4, 16, 4, 1, 4, sig, 1, P, P, S) == NULL
    assert f(P, N0, 0, 16, 4, 1, 4, sig, 1, N0, N0, S) == OK        # T = 0
    assert f(P, N0, 4, 16, 4, 1, 4, 9, 1, P, P, S) == UNSUP


def test_permute_errors():
    f = L.lib.moe_permute
    assert f(P, 8, 9, 8, N0, N0, 0, P, P, P, N0, N0, P, 1 << 20, S) == SHAPE       # K > E
    assert f(P, 8, 2, 4096, N0, N0, 0, P, P, P, N0, N0, P, 1 << 20, S) == UNSUP    # E > 1024
    assert f(P, 8, 2, 8, P, N0, 128, P, P, P, P, P, P, 1 << 20, S) == NULL         # partial gather set
    assert f(P, 8, 2, 8, P, P, 100, P, P, P, P, P, P, 1 << 20, S) == SHAPE         # H % 128
    assert f(P, 8, 2, 8, PM, P, 128, P, P, P, P, P, P, 1 << 20, S) == ALIGN
    assert f(P, 8, 2, 8, N0, N0, 0, P, P, P, N0, N0, P, 16, S) == WS
    assert f(P, 8, 2, 8, N0, N0, 0, N0, P, P, N0, N0, P, 1 << 20, S) == NULL


def test_gemm_errors():
    f = L.lib.grouped_gemm_fp8_blockscaled
    assert f(P, P, P, P, P, 4, 64, 100, 128, P, 0, S) == SHAPE
    assert f(P, P, P, P, P, 4, 64, 128, 130, P, 0, S) == SHAPE
    assert f(P, P, P, P, P, 2048, 64, 128, 128, P, 0, S) == UNSUP            # G > 1024
    assert f(P, P, P, P, P, 4, 64, 128, 65536 + 128, P, 0, S) == UNSUP       # K > 65536
    assert f(P, P, P, P, P, 0, 64, 128, 128, P, 0, S) == SHAPE
    assert f(P, P, P, P, N0, 4, 64, 128, 128, P, 0, S) == NULL
    assert f(P, P, P, P, P, 4, 64, 128, 128, N0, 0, S) == NULL
    assert f(PM, P, P, P, P, 4, 64, 128, 128, P, 0, S) == ALIGN
    assert f(P, P, P, P, P, 4, 64, 128, 128, P, 5, S) == UNSUP
    assert f(N0, N0, N0, N0, P, 4, 0, 128, 128, N0, 0, S) == OK           # M = 0
    # row gather: no index array, misaligned index array, no source rows,
    # source above 4 GiB
    f = L.lib.grouped_gemm_fp8_blockscaled_gather
    assert f(P, P, N0, 16, P, P, P, 4, 64, 128, 128, P, 0, S) == NULL
    assert f(P, P, ctypes.c_void_p(0x10002), 16, P, P, P, 4, 64, 128, 128, P, 0, S) == ALIGN
    assert f(P, P, P, 0, P, P, P, 4, 64, 128, 128, P, 0, S) == SHAPE
    assert f(P, P, P, 1 << 26, P, P, P, 4, 64, 128, 128, P, 0, S) == UNSUP
    assert f(P, P, P, 16, P, P, P, 4, 64, 100, 128, P, 0, S) == SHAPE
    assert f(N0, N0, N0, 0, N0, N0, P, 4, 0, 128, 128, N0, 0, S) == OK    # M = 0
    g = L.lib.grouped_gemm_fp8_swiglu
    assert g(P, P, N0, 0, P, P, P, 4, 64, 100, 128, P, P, S) == SHAPE
    assert g(P, P, N0, 0, P, P, P, 4, 64, 128, 128, P, N0, S) == NULL
    assert g(P, P, P, 0, P, P, P, 4, 64, 128, 128, P, P, S) == SHAPE


def test_swiglu_combine_transpose_errors():
    assert L.lib.swiglu(P, 4, 100, P, P, S) == SHAPE
    assert L.lib.swiglu(N0, 4, 128, P, P, S) == NULL
    assert L.lib.swiglu(N0, 0, 128, N0, N0, S) == OK
    c = L.lib.moe_combine
    assert c(P, P, P, N0, 4, 2, 12, P, S) == SHAPE
    assert c(P, P, P, PM, 4, 2, 16, P, S) == ALIGN
    assert c(N0, P, P, N0, 4, 2, 16, P, S) == NULL
    assert c(N0, N0, N0, N0, 0, 2, 16, N0, S) == OK
    t = L.lib.fp8_block_transpose
    assert t(P, P, 2, 100, 128, P, P, S) == SHAPE
    assert t(P, P, 2, 128, 128, N0, P, S) == NULL
    assert t(P, P, 2, 128, 128, PM, P, S) == ALIGN
    assert t(N0, N0, 0, 128, 128, N0, N0, S) == OK


def test_binding_requires_device_tensors():
    import torch
    with pytest.raises((ValueError, TypeError)):
        L.quant_act_1x128_e4m3(torch.zeros(4, 128))


def test_binding_rejects_odd_gate_up_width():
    """A gate|up width of 2I + 1 would pass the library's I % 128 check with
    the wrong row stride; the binding refuses it."""
    assert L._even(512, "gate_up columns") == 256
    with pytest.raises(ValueError):
        L._even(257, "gate_up columns")


def test_backward_errors():
    c = L.lib.moe_combine_backward
    assert c(P, P, P, P, 4, 2, 100, P, P, P, N0, S) == SHAPE             # H % 128
    assert c(P, P, P, P, 4, 17, 128, P, P, P, N0, S) == UNSUP            # K > 16
    assert c(P, N0, P, P, 4, 2, 128, P, P, P, N0, S) == NULL
    assert c(PM, P, P, P, 4, 2, 128, P, P, P, N0, S) == ALIGN
    assert c(P, P, P, P, 4, 2, 128, P, P, P, ctypes.c_void_p(0x10002), S) == ALIGN   # gate_row
    assert c(N0, N0, N0, N0, 0, 2, 128, N0, N0, N0, N0, S) == OK          # T = 0
    g = L.lib.swiglu_backward
    assert g(P, P, 4, 100, P, P, N0, S) == SHAPE
    assert g(P, N0, 4, 128, P, P, N0, S) == NULL
    assert g(PM, P, 4, 128, P, P, N0, S) == ALIGN
    assert g(P, P, 4, 128, P, P, PM, S) == ALIGN                          # d needs 16 bytes
    assert g(N0, N0, 0, 128, N0, N0, N0, S) == OK
    r = L.lib.moe_route_backward
    assert r(P, P, P, 4, 8, 9, 0, 1, P, S) == SHAPE                       # K > E
    assert r(P, P, P, 4, 128, 65, 0, 1, P, S) == UNSUP                    # K > 64
    assert r(P, P, P, 4, 8, 2, 7, 1, P, S) == UNSUP                       # mode
    assert r(P, P, N0, 4, 8, 2, 0, 1, P, S) == NULL
    assert r(N0, N0, N0, 0, 8, 2, 1, 0, N0, S) == OK


def test_wgrad_errors():
    n = ctypes.c_int64(0)
    assert L.lib.moe_wgrad_padded_rows(300, 4, ctypes.byref(n)) == OK and n.value == 128 * (3 + 4)
    assert L.lib.moe_wgrad_padded_rows(0, 1, ctypes.byref(n)) == OK and n.value == 128
    assert L.lib.moe_wgrad_padded_rows(-1, 1, ctypes.byref(n)) == SHAPE
    assert L.lib.moe_wgrad_padded_rows(5, 0, ctypes.byref(n)) == SHAPE
    assert L.lib.moe_wgrad_padded_rows(5, 1, None) == NULL
    q = L.lib.quant_act_128x1_grouped_e4m3
    #     x  dt sw rows  C   idx scl off  G   M   ld    poff qt st
    assert q(P, 0, 0, 300, 100, N0, N0, P, 4, 300, 896, P, P, P, S) == SHAPE       # C % 128
    assert q(P, 0, 0, 300, 128, N0, N0, P, 4, 300, 768, P, P, P, S) == SHAPE       # ld < 128 (3 + 4)
    assert "ld" in _detail()
    assert q(P, 0, 0, 300, 128, N0, N0, P, 4, 300, 900, P, P, P, S) == SHAPE       # ld % 128
    assert q(P, 0, 0, 200, 128, N0, N0, P, 4, 300, 896, P, P, P, S) == SHAPE       # x_rows < M, no index
    assert q(P, 1, 1, 300, 128, N0, N0, P, 4, 300, 896, P, P, P, S) == UNSUP       # bf16 gate|up
    assert q(P, 5, 0, 300, 128, N0, N0, P, 4, 300, 896, P, P, P, S) == UNSUP       # dtype
    assert q(P, 0, 0, 300, 128, N0, N0, P, 1025, 300, 128 * 1028, P, P, P, S) == UNSUP   # G
    assert q(P, 0, 0, 300, 128, N0, N0, P, 0, 300, 896, P, P, P, S) == UNSUP       # G = 0
    assert q(P, 0, 0, 300, 128, N0, N0, N0, 4, 300, 896, P, P, P, S) == NULL      # offsets
    assert q(N0, 0, 0, 300, 128, N0, N0, P, 4, 300, 896, P, P, P, S) == NULL      # x
    assert q(PM, 0, 0, 300, 128, N0, N0, P, 4, 300, 896, P, P, P, S) == ALIGN
    assert q(P, 0, 0, 300, 128, N0, N0, P, 4, 300, 896, P, PM, P, S) == ALIGN     # qt
    assert q(P, 0, 0, 1 << 20, 1 << 30, N0, N0, P, 4, 1 << 20, (1 << 20) + 512, P, P, P, S) == UNSUP   # blocks
    w = L.lib.grouped_wgrad_fp8
    #     aq as bq bs poff G  Na   Nb   ld   c dt acc
    assert w(P, P, P, P, P, 4, 100, 128, 256, P, 0, 0, S) == SHAPE
    assert w(P, P, P, P, P, 4, 128, 128, 200, P, 0, 0, S) == SHAPE                 # ld % 128
    assert w(P, P, P, P, P, 0, 128, 128, 256, P, 0, 0, S) == UNSUP
    assert w(P, P, P, P, P, 4, 128, 128, 256, P, 3, 0, S) == UNSUP                 # c dtype
    assert w(P, P, P, P, N0, 4, 128, 128, 256, P, 0, 0, S) == NULL
    assert w(P, P, PM, P, P, 4, 128, 128, 256, P, 0, 0, S) == ALIGN
    assert w(P, P, P, P, P, 4, 128, 128, 256, ctypes.c_void_p(0x10008), 0, 0, S) == ALIGN   # f32 c
    assert w(P, P, P, P, P, 1024, 524288, 524288, 256, P, 0, 0, S) == UNSUP        # tile count
    assert w(P, P, P, P, P, 4, 128, 128, 2 ** 29 + 128, P, 0, 0, S) == UNSUP       # ld above 2^29


def test_router_errors():
    r = L.lib.moe_router_logits
    assert r(P, P, 4, 100, 8, P, S) == SHAPE                              # H % 64
    assert r(P, P, 4, 128, 0, P, S) == SHAPE                              # E >= 1
    assert r(P, P, 4, 128, 2 ** 31 - 1, P, S) == UNSUP
    assert r(N0, P, 4, 128, 8, P, S) == NULL
    assert r(PM, P, 4, 128, 8, P, S) == ALIGN
    assert r(N0, N0, 0, 128, 8, N0, S) == OK                              # T = 0
    b = L.lib.moe_bias_update
    assert b(P, 0, 0.1, P, S) == SHAPE
    assert b(N0, 8, 0.1, P, S) == NULL
    assert b(P, 8, 0.1, ctypes.c_void_p(0x10002), S) == ALIGN


def test_probe_argument_errors():
    pr = L.lib.moe_probe_mfma_fp8
    fl = ctypes.c_double(0.0)
    assert pr(0x38, 10, 0, 8, P, ctypes.byref(fl), S) == SHAPE          # no workgroup
    assert pr(0x38, -1, 1, 8, P, ctypes.byref(fl), S) == SHAPE
    assert pr(0x38, 2**40, 1, 8, P, ctypes.byref(fl), S) == SHAPE       # iterations above 2^32
    assert pr(0x38, 10, 1, 17, P, ctypes.byref(fl), S) == SHAPE         # more than 16 waves
    assert pr(0x38, 10, 1, 8, N0, ctypes.byref(fl), S) == NULL
    assert pr(0x38, 10, 1, 8, P, None, S) == NULL
    assert pr(0x38, 10, 1, 8, ctypes.c_void_p(0x10002), ctypes.byref(fl), S) == ALIGN


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library the binding raises instead of falling back."""
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "libmoefp8.so"))
    with pytest.raises(ImportError):
        L._load()


def test_product_path_does_not_use_the_oracle():
    """No module of the package imports or names the oracle (test
    infrastructure only): the computation has no CPU path."""
    import ast
    import pathlib
    pkg = pathlib.Path(L.__file__).parent
    for f in pkg.glob("*.py"):
        tree = ast.parse(f.read_text())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                assert not any(a.name.split(".")[0] == "oracle" for a in node.names), f
            if isinstance(node, ast.ImportFrom):
                assert (node.module or "").split(".")[0] != "oracle", f


def test_c_caller_of_the_eight_operations(tmp_path):
    """A C program that declares the eight operations' prototypes itself (not
    from include/moefp8.h) links against libmoefp8.so and gets the documented
    status from one failing (or empty) call of each: a prototype that drifted
    would shift its arguments and miss the expected codes."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = os.path.join(ROOT, "tests", "abi_c", "caller_8ops.c")
    libdir = os.path.dirname(L.LIB_PATH)
    exe = str(tmp_path / "caller_8ops")
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Werror", "-o", exe, src, "-L", libdir, "-lmoefp8",
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "PASSED" in r.stdout


def test_sigmoid_errors():
    f = L.lib.moe_sigmoid_f32
    assert f(P, -1, P, S) == SHAPE
    assert f(N0, 16, P, S) == NULL
    assert f(PM, 16, P, S) == ALIGN
    assert f(P, 1 << 41, P, S) == UNSUP
    assert f(N0, 0, N0, S) == OK


def test_permute_noalloc_errors():
    """The scratch-array variant checks everything on the host before it
    looks up its scratch: bad sizes, NULLs, alignment and a problem larger
    than the static scratch never touch the device."""
    f = L.lib.moe_permute_noalloc
    assert f(P, 8, 9, 8, N0, N0, 0, P, P, P, N0, N0, S) == SHAPE                # K > E
    assert f(P, 8, 2, 4096, N0, N0, 0, P, P, P, N0, N0, S) == UNSUP             # E > 1024
    assert f(P, 8, 2, 8, P, N0, 128, P, P, P, P, P, S) == NULL                  # partial gather set
    assert f(P, 8, 2, 8, PM, P, 128, P, P, P, P, P, S) == ALIGN
    assert f(P, 8, 2, 8, N0, N0, 0, N0, P, P, N0, N0, S) == NULL                # no offsets
    assert f(P, 600000, 2, 256, N0, N0, 0, P, P, P, N0, N0, S) == WS            # beyond the 4 MiB scratch
    assert "scratch" in _detail()


def test_route_permute_errors():
    """The single-launch routing + permutation checks moe_route's and
    moe_permute's arguments and its workspace on the host (every call here
    fails validation; T = 0 would still launch, to write the zero offsets)."""
    n = ctypes.c_size_t(0)
    assert L.lib.moe_route_permute_workspace_size(4096, 8, 256, ctypes.byref(n)) == OK
    assert n.value == 256 + 2 * 64 * 256 * 4          # header + counts and base rows of 64-token blocks
    assert L.lib.moe_route_permute_workspace_size(0, 8, 256, ctypes.byref(n)) == OK and n.value == 256
    assert L.lib.moe_route_permute_workspace_size(10, 9, 8, ctypes.byref(n)) == SHAPE
    f = L.lib.moe_route_permute
    sig, grp = L.ROUTE_SIGMOID_BIAS, L.ROUTE_SOFTMAX_GROUPED
    big = 1 << 20
    assert f(P, N0, 4, 2048, 8, 1, 8, sig, 1, P, P, P, P, P, P, big, S) == UNSUP      # E > 1024
    assert f(P, N0, 4, 16, 17, 1, 17, sig, 1, P, P, P, P, P, P, big, S) == SHAPE      # K > E
    assert f(P, N0, 4, 18, 4, 4, 1, grp, 0, P, P, P, P, P, P, big, S) == SHAPE        # E % G
    assert f(P, N0, 4, 16, 4, 4, 1, grp, 1, P, P, P, P, P, P, big, S) == UNSUP        # no renormalisation
    assert f(P, N0, 4, 16, 4, 1, 4, 9, 1, P, P, P, P, P, P, big, S) == UNSUP          # mode
    assert f(N0, N0, 4, 16, 4, 1, 4, sig, 1, P, P, P, P, P, P, big, S) == NULL        # logits
    assert f(P, N0, 4, 16, 4, 1, 4, sig, 1, P, P, N0, P, P, P, big, S) == NULL        # offsets
    assert f(P, N0, 4, 16, 4, 1, 4, sig, 1, P, P, P, P, P, N0, big, S) == NULL        # workspace
    assert f(P, N0, 4, 16, 4, 1, 4, sig, 1, P, P, P, P, P, PM, big, S) == ALIGN       # workspace 16 B
    assert f(P, N0, 4, 16, 4, 1, 4, sig, 1, P, P, P, P, P, P, 255, S) == WS
    assert f(P, N0, 1 << 28, 16, 16, 1, 16, sig, 1, P, P, P, P, P, P, big, S) == UNSUP  # T*K


def test_gemm_combine_errors():
    n = ctypes.c_size_t(0)
    assert L.lib.grouped_gemm_fp8_combine_workspace_size(4096, 7168, ctypes.byref(n)) == OK
    assert n.value == 4096 * 28 * 4
    assert L.lib.grouped_gemm_fp8_combine_workspace_size(4, 384, ctypes.byref(n)) == OK and n.value == 4 * 2 * 4
    f = L.lib.grouped_gemm_fp8_combine
    ws = 1 << 20
    assert f(P, P, P, P, P, 4, 64, 256, 128, P, P, P, P, N0, 16, 3, P, P, ws, S) == SHAPE    # M != T*topk
    assert f(P, P, P, P, P, 4, 64, 100, 128, P, P, P, P, N0, 16, 4, P, P, ws, S) == SHAPE    # N % 128
    assert f(P, P, P, P, P, 4, 64, 256, 128, P, N0, P, P, N0, 16, 4, P, P, ws, S) == NULL    # src_token
    assert f(P, P, P, P, P, 4, 64, 256, 128, P, P, P, P, N0, 16, 4, P, N0, ws, S) == NULL    # counters
    assert f(P, P, P, P, P, 4, 64, 256, 128, P, P, P, P, PM, 16, 4, P, P, ws, S) == ALIGN    # shared
    assert f(P, P, P, P, P, 4, 64, 256, 128, P, P, P, P, N0, 16, 4, P, P, 63, S) == WS       # 16*1*4 bytes
    assert f(P, P, P, P, P, 4, 64, 256, 128, P, P, P, P, N0, 16, 0, P, P, ws, S) == SHAPE    # topk
    assert f(N0, N0, N0, N0, P, 4, 0, 256, 128, N0, N0, N0, N0, N0, 0, 4, N0, N0, 0, S) == OK  # empty
