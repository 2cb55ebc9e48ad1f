"""The library's host code (argument checks, size arithmetic, status and
detail reporting, workspace and scratch bookkeeping) under
AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of libmoefp8 is compiled with the sanitizers on its host side
only (the device code is the ordinary gfx950 build) and linked into the C
driver tests/abi_c/host_checks.c, which calls every entry point with
arguments the checks must refuse, including extreme sizes, or with empty
problems; nothing is launched, so no GPU is needed.  Any sanitizer report
(an out-of-bounds access, a signed overflow, a misaligned load, a use of an
uninitialised status) fails the run."""

import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routed_experts_fp8_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SANITIZE = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _library_sources():
    import importlib.util
    spec = importlib.util.spec_from_file_location("moefp8_build", os.path.join(ROOT, "routed_experts_fp8_amd",
                                                                               "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b.SOURCES, b.FLAGS, b.DEVICE_FLAGS


@pytest.mark.timeout(1200)
def test_host_checks_under_asan_and_ubsan(tmp_path):
    if not all(os.path.exists(t) for t in (HIPCC, CLANG, CLANGXX)):
        pytest.skip("ROCm compilers not found")
    sources, flags, dev_flags = _library_sources()
    host_san = [f for s in SANITIZE for f in ("-Xarch_host", s)]   # host side only

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC] + flags + ["-x", "hip"] + dev_flags + host_san + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [HIPCC] + flags + host_san + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{src}:\n{r.stderr[-3000:]}"
        return obj

    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, sources))
    drv = str(tmp_path / "host_checks.o")
    r = subprocess.run([CLANG, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include")] + SANITIZE +
                       ["-c", os.path.join(ROOT, "tests", "abi_c", "host_checks.c"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "host_checks")
    r = subprocess.run([CLANGXX] + SANITIZE + ["-o", exe, drv] + objs +
                       ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    print(r.stdout)
    assert r.returncode == 0, out[-4000:]
    assert "PASSED" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


def test_detail_format_strings_are_valid():
    """Every printf-style detail message the library formats uses only valid
    conversions (a bare '%' in a message is undefined behaviour in vsnprintf;
    one was found by the sanitizer run above)."""
    import glob
    import re
    bad = []
    for f in sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp"))):
        s = open(f).read()
        for m in re.finditer(r"(MOE_REQUIRE|fail)\((.*?)\);", s, re.S):
            for lit in re.findall(r'"((?:[^"\\]|\\.)*)"', m.group(2)):
                for pm in re.finditer(r"%", lit):
                    if not re.match(r"%(%|[-+ #0]*\d*(\.\d+)?(hh|h|ll|l|z|j|t)?[diouxXeEfgGcspn])", lit[pm.start():]):
                        bad.append((os.path.basename(f), lit))
    assert not bad, bad
